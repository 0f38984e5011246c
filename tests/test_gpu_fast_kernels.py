"""GPU parity of RMS layernorm, RoPE and cross entropy (through the C ABI)
against the fp64 oracle (oracle/fast_kernels.py).

Bar: max|gpu - oracle| / max|oracle| <= 2e-2 per output tensor; the loss
scalar and the label count are checked exactly or to 1e-5 relative. Inputs
are seeded synthetic draws in bf16; the oracle sees the same bf16 values.
Cases: ragged row widths and vocabularies (V not a multiple of 8), both norm
weightings, long-context positions, strided and in-place RoPE on slices of a
fused q/k/v buffer, Gemma's 256K vocabulary, ignored labels, all labels
ignored, an upstream dloss, in-place gradient, and full Llama-7B sizes
(8192 tokens: RMS layernorm over 4096, RoPE on 32 heads of 128, cross entropy
over a 32000 vocabulary).
"""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import fast_kernels as F
from qlora_fine_tuning_amd import inputs as I

from _util import TOL, f64, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check(name, got, ref, tol=TOL):
    e = rel_err(got, ref)
    say(f"  {name}: rel error {e:.3e}")
    assert e <= tol, (name, e)


# ----------------------------------------------------------- RMS layernorm --
@pytest.mark.parametrize("m,d,gemma,eps", [(37, 264, False, 1e-6), (37, 264, True, 1e-6),
                                           (1, 8, False, 1e-5), (300, 4096, False, 1e-5),
                                           (64, 3072, True, 1e-6), (8192, 4096, False, 1e-6),
                                           (16, 6152, False, 1e-6), (8, 12296, True, 1e-5)])
def test_rmsnorm(m, d, gemma, eps):
    X = I.normal_bf16("X", (m, d), 1.0, seed=m + d)
    w = I.normal_bf16("W", (d,), 0.1 if gemma else 0.3, seed=d) + (0 if gemma else 1)
    w = w.to(torch.bfloat16)
    dY = I.normal_bf16("dY", (m, d), 1.0, seed=m + d + 1)
    say(f"rmsnorm m={m} d={d} gemma={gemma}")
    Y, rstd = Q.rmsnorm_fwd(X.to(DEV), w.to(DEV), eps, gemma)
    dX = Q.rmsnorm_bwd(dY.to(DEV), X.to(DEV), rstd, w.to(DEV), gemma)
    torch.cuda.synchronize()
    Yr, r = F.rms_layernorm_fwd(f64(X), f64(w), eps, gemma)
    dXr = F.rms_layernorm_bwd(f64(dY), f64(X), r, f64(w), gemma)
    _check("Y", Y, Yr)
    _check("rstd", rstd, r, 1e-5)
    _check("dX", dX, dXr)


def test_rmsnorm_empty():
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    Y, rstd = Q.rmsnorm_fwd(X, w, 1e-6)
    dX = Q.rmsnorm_bwd(X, X, rstd, w)
    torch.cuda.synchronize()
    assert Y.shape == (0, 64) and dX.shape == (0, 64)


# ------------------------------------------------------------------- RoPE --
@pytest.mark.parametrize("m,heads,hd,base,pmax", [(19, 3, 16, 10000.0, 2048), (19, 5, 32, 500000.0, 1 << 20),
                                                 (33, 9, 128, 10000.0, 8192), (7, 2, 256, 10000.0, 8192),
                                                 (1, 1, 16, 10000.0, 1)])
def test_rope(m, heads, hd, base, pmax):
    X = I.normal_bf16("X", (m, heads, hd), 1.0, seed=m * heads + hd)
    pos = torch.from_numpy(np.random.default_rng(hd).integers(0, pmax, size=m).astype(np.int64))
    say(f"rope m={m} heads={heads} hd={hd} base={base} pmax={pmax}")
    Y = Q.rope_fwd(X.to(DEV), pos.to(DEV), base)
    dX = Q.rope_bwd(X.to(DEV), pos.to(DEV), base)
    torch.cuda.synchronize()
    _check("Y", Y, F.rope_fwd(f64(X), pos.numpy(), base))
    _check("dX", dX, F.rope_bwd(f64(X), pos.numpy(), base))


def test_rope_on_qkv_slices_in_place():
    # Q and K as column slices of one [m][(32 + 8 + 8) * 128] q/k/v buffer, rotated in place
    m, hd = 300, 128
    buf = I.normal_bf16("X", (m, 48 * hd), 1.0, seed=31).to(DEV)
    ref = buf.clone()
    pos = torch.arange(m, dtype=torch.int64, device=DEV) % 97
    q = buf[:, : 32 * hd].view(m, 32, hd)
    k = buf[:, 32 * hd: 40 * hd].view(m, 8, hd)
    say("rope in place on q/k/v slices")
    Q.rope_fwd(q, pos, 10000.0, inplace=True)
    Q.rope_fwd(k, pos, 10000.0, inplace=True)
    torch.cuda.synchronize()
    p = pos.cpu().numpy()
    R = f64(ref)
    _check("q", buf[:, : 32 * hd], F.rope_fwd(R[:, : 32 * hd].reshape(m, 32, hd), p, 10000.0).reshape(m, -1))
    _check("k", buf[:, 32 * hd: 40 * hd], F.rope_fwd(R[:, 32 * hd: 40 * hd].reshape(m, 8, hd), p, 10000.0).reshape(m, -1))
    assert torch.equal(buf[:, 40 * hd:], ref[:, 40 * hd:])          # v untouched
    # the backward undoes the forward up to bf16 rounding
    Q.rope_bwd(q, pos, 10000.0, inplace=True)
    torch.cuda.synchronize()
    _check("q round trip", buf[:, : 32 * hd], R[:, : 32 * hd])


def test_rope_full_size_llama():
    m, heads, hd = 8192, 32, 128
    X = I.normal_bf16("X", (m, heads * hd), 1.0).view(m, heads, hd)
    pos = torch.arange(m, dtype=torch.int64) % 2048            # 4 sequences of 2048
    say("rope full size")
    Y = Q.rope_fwd(X.to(DEV), pos.to(DEV))
    torch.cuda.synchronize()
    rows = np.arange(0, m, 61)
    _check("Y rows", Y[torch.as_tensor(rows, device=DEV)],
           F.rope_fwd(f64(X)[rows], pos.numpy()[rows], 10000.0))


# ------------------------------------------------------------ cross entropy --
def _labels(m, V, seed, ignore=(2,)):
    g = np.random.default_rng(seed)
    lab = g.integers(0, V, size=m).astype(np.int64)
    lab[0] = 0
    if m > 1:
        lab[1] = V - 1
    for i in ignore:
        if i < m:
            lab[i] = F.IGNORE
    return lab


def _oracle_ce(X64, lab, dloss=1.0, chunk=512):
    m = X64.shape[0]
    lse = np.concatenate([F.logsumexp_rows(X64[i:i + chunk]) for i in range(0, m, chunk)])
    valid = lab != F.IGNORE
    ce = np.zeros(m)
    rows = np.nonzero(valid)[0]
    ce[rows] = lse[rows] - X64[rows, lab[rows]]
    n = int(valid.sum())
    return (ce.sum() / n if n else 0.0), ce, lse, n


@pytest.mark.parametrize("m,V,pad", [(13, 50, 6), (13, 1001, 0), (9, 32000, 8), (4, 70001, 7),
                                     (3, 256000, 0), (1, 8, 0)])
def test_cross_entropy(m, V, pad):
    ld = (V + pad + 7) // 8 * 8
    full = I.normal_bf16("X", (m, ld), 3.0, seed=V + m)
    X = full[:, :V]
    lab = _labels(m, V, seed=V)
    dloss = torch.tensor([0.625], dtype=torch.float32)
    say(f"cross entropy m={m} V={V} ld={ld}")
    Xd = full.to(DEV)[:, :V]
    fwd = Q.cross_entropy_fwd(Xd, torch.from_numpy(lab).to(DEV))
    dX = Q.cross_entropy_bwd(Xd, torch.from_numpy(lab).to(DEV), fwd, dloss=dloss.to(DEV))
    torch.cuda.synchronize()
    X64 = f64(X)
    loss, ce, lse, n = F.cross_entropy_fwd(X64, lab)
    dXr = F.cross_entropy_bwd(X64, lab, lse, n, dloss=0.625)
    assert int(fwd["n_valid"].item()) == n
    assert abs(fwd["loss"].item() - loss) <= 1e-5 * abs(loss)
    _check("lse", fwd["lse"], lse, 1e-5)
    _check("ce", fwd["ce"], ce, 1e-4)
    _check("dX", dX, dXr)


def test_cross_entropy_all_ignored_and_in_place():
    m, V = 5, 4000
    X = I.normal_bf16("X", (m, V), 2.0, seed=77)
    lab = np.full(m, F.IGNORE, dtype=np.int64)
    Xd = X.to(DEV)
    fwd = Q.cross_entropy_fwd(Xd, torch.from_numpy(lab).to(DEV))
    dX = Q.cross_entropy_bwd(Xd, torch.from_numpy(lab).to(DEV), fwd, inplace=True)
    torch.cuda.synchronize()
    assert fwd["loss"].item() == 0.0 and int(fwd["n_valid"].item()) == 0
    assert dX.data_ptr() == Xd.data_ptr() and torch.count_nonzero(dX).item() == 0
    # in place with labels: same bits as the out-of-place gradient
    lab = _labels(m, V, seed=5)
    Xa, Xb = X.to(DEV), X.to(DEV)
    fa = Q.cross_entropy_fwd(Xa, torch.from_numpy(lab).to(DEV))
    ga = Q.cross_entropy_bwd(Xa, torch.from_numpy(lab).to(DEV), fa)
    fb = Q.cross_entropy_fwd(Xb, torch.from_numpy(lab).to(DEV))
    gb = Q.cross_entropy_bwd(Xb, torch.from_numpy(lab).to(DEV), fb, inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(ga, gb)


def test_cross_entropy_full_size_llama():
    m, V = 8192, 32000
    X = I.normal_bf16("X", (m, V), 2.0, seed=11)
    lab = _labels(m, V, seed=12, ignore=tuple(range(2, m, 37)))
    say("cross entropy full size")
    Xd = X.to(DEV)
    fwd = Q.cross_entropy_fwd(Xd, torch.from_numpy(lab).to(DEV))
    dX = Q.cross_entropy_bwd(Xd, torch.from_numpy(lab).to(DEV), fwd)
    torch.cuda.synchronize()
    loss, ce, lse, n = _oracle_ce(f64(X), lab)
    assert int(fwd["n_valid"].item()) == n
    assert abs(fwd["loss"].item() - loss) <= 1e-5 * abs(loss)
    _check("lse", fwd["lse"], lse, 1e-5)
    rows = np.arange(0, m, 97)
    X64 = f64(X[rows])
    dXr = F.cross_entropy_bwd(X64, lab[rows], lse[rows], n)
    _check("dX rows", dX[torch.as_tensor(rows, device=DEV)], dXr)


@pytest.mark.parametrize("m,V,pad", [(13, 1001, 8), (64, 32000, 0), (3, 256000, 0)])
def test_cross_entropy_fused_equals_separate_calls(m, V, pad):
    ld = (V + pad + 7) // 8 * 8
    full = I.normal_bf16("X", (m, ld), 3.0, seed=V + 2 * m)
    lab = torch.from_numpy(_labels(m, V, seed=V + 1)).to(DEV)
    Xd = full.to(DEV)[:, :V]
    say(f"cross entropy fused m={m} V={V}")
    sep = Q.cross_entropy_fwd(Xd, lab)
    g_sep = Q.cross_entropy_bwd(Xd, lab, sep, dloss=torch.tensor([0.375], device=DEV))
    fus = Q.cross_entropy_fused(Xd, lab, dloss=0.375)
    X2 = full.to(DEV)[:, :V]   # a second padded copy, overwritten in place
    fin = Q.cross_entropy_fused(X2, lab, dloss=0.375, inplace=True)
    torch.cuda.synchronize()
    for k in ("loss", "n_valid", "lse", "ce"):
        assert torch.equal(sep[k], fus[k]) and torch.equal(sep[k], fin[k]), k
    assert torch.equal(g_sep, fus["dlogits"]) and torch.equal(g_sep, fin["dlogits"])
    assert fin["dlogits"].data_ptr() == X2.data_ptr()
    loss, ce, lse, n = F.cross_entropy_fwd(f64(full[:, :V]), lab.cpu().numpy())
    _check("dX vs oracle", fus["dlogits"], F.cross_entropy_bwd(f64(full[:, :V]), lab.cpu().numpy(), lse, n, 0.375))
