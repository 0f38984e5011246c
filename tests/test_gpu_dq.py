"""GPU parity of the double-quantized absmax (second-level quantization of the
NF4 constants) against the fp64 oracle, through the C ABI.

- qlora_absmax_dq_quantize: codes, scales and offsets bit-exact against
  oracle.nf4.absmax_dq_quantize (full weight arrays of the workloads, a ragged
  last group, zero, constant and on-grid groups);
- qlora_absmax_dq_dequant: the reconstructed constants bit-exact;
- every layer entry point given a double-quantized weight: the dequantized
  weight bit-exact against the oracle's dequant with the reconstructed
  constants, and every output equal bit for bit to the same call given those
  constants as a plain fp32 absmax (staged and fused dequant, linear, MLP,
  q/k/v), plus the oracle tolerance on the linear layer.
"""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import nf4 as onf4
from oracle import qlora as OQ
from qlora_fine_tuning_amd import inputs as I

from _util import TOL, dequant_oracle, f64, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _dq_both(absmax_np):
    say(f"absmax dq quantize nb={absmax_np.size}")
    dq = Q.absmax_dq_quantize(torch.from_numpy(absmax_np.reshape(-1).copy()).to(DEV))
    back = Q.absmax_dq_dequant(dq)
    torch.cuda.synchronize()
    q, sc, of = onf4.absmax_dq_quantize(absmax_np)
    return dq, back, (q, sc, of)


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n,k", [(11008, 4096), (4096, 11008), (24576, 3072), (1024, 4096), (25, 640)])
def test_dq_quantize_dequant_bit_exact(n, k):
    _, absmax = I.synthetic_nf4("Wg", n, k)
    a = absmax.numpy()
    dq, back, (q, sc, of) = _dq_both(a)
    assert np.array_equal(dq.q.cpu().numpy(), q)
    assert np.array_equal(_bits(dq.scale), sc.view(np.uint32))
    assert np.array_equal(_bits(dq.offset), of.view(np.uint32))
    assert np.array_equal(_bits(back), onf4.absmax_dq_dequant(q, sc, of).view(np.uint32))


def test_dq_special_groups():
    g = np.random.default_rng(3)
    parts = [np.zeros(256, np.float32),                                   # zero group
             np.full(256, np.float32(0.03125)),                           # constant group
             (np.float32(0.375) + np.float32(2.0 ** -12) *
              np.concatenate([np.arange(-127, 128), [0]]).astype(np.float32)).astype(np.float32),
             (np.abs(g.standard_normal(256)) * 1e-30).astype(np.float32),   # tiny values
             (np.abs(g.standard_normal(256)) * 1e30).astype(np.float32),    # huge values
             np.abs(g.standard_normal(77)).astype(np.float32)]               # ragged last group
    a = np.concatenate(parts)
    dq, back, (q, sc, of) = _dq_both(a)
    assert np.array_equal(dq.q.cpu().numpy(), q)
    assert np.array_equal(_bits(dq.scale), sc.view(np.uint32))
    assert np.array_equal(_bits(dq.offset), of.view(np.uint32))
    assert np.array_equal(_bits(back), onf4.absmax_dq_dequant(q, sc, of).view(np.uint32))
    assert np.all(back[:256].cpu().numpy() == 0)


def _dq_weight(codes, absmax):
    """(plain weight with the reconstructed constants, double-quantized weight)."""
    dq = Q.absmax_dq_quantize(absmax.to(DEV))
    recon = Q.absmax_dq_dequant(dq).reshape(absmax.shape)
    c = codes.to(DEV)
    return Q.NF4Weight(c, recon), Q.NF4Weight(c, None, dq)


@pytest.mark.parametrize("n,k", [(11008, 4096), (3072, 24576), (192, 320)])
def test_dq_weight_dequant_bit_exact(n, k):
    codes, absmax = I.synthetic_nf4("Wd", n, k)
    plain, dqw = _dq_weight(codes, absmax)
    say(f"nf4 dequant of a double-quantized weight {n}x{k}")
    got = Q.nf4_dequant(dqw)
    torch.cuda.synchronize()
    q, sc, of = onf4.absmax_dq_quantize(absmax.numpy())
    recon = onf4.absmax_dq_dequant(q, sc, of).reshape(absmax.shape)
    want = onf4.dequant_bf16_bits(codes.numpy(), recon)
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("mode", ["staged", "fused"])
def test_dq_linear_equals_plain_and_oracle(mode):
    cfg = I.LinearCfg("dq_linear", 300, 320, 448, 16, 1.0, 1.0)
    d = I.linear_inputs(cfg, dense_w=False, seed=21)
    plain, dqw = _dq_weight(d["codes"], d["absmax"])
    X, A, B, dY = (d[k].to(DEV) for k in ("X", "A", "B", "dY"))
    say(f"linear with double-quantized absmax mode={mode}")
    out = []
    for w in (plain, dqw):
        Y, U = Q.linear_fwd(X, w, A, B, cfg.s, mode=mode)
        dX, dA, dB = Q.linear_bwd(dY, X, U, w, A, B, cfg.s, mode=mode)
        out.append((Y, U, dX, dA, dB))
    torch.cuda.synchronize()
    for a, b in zip(*out):
        assert torch.equal(a, b)
    Wr = onf4.dequant_f64(d["codes"].numpy(), plain.absmax.cpu().numpy())
    Yr, Ur = OQ.linear_fwd(f64(d["X"]), Wr, f64(d["A"]), f64(d["B"]), cfg.s)
    dXr, dAr, dBr, _ = OQ.linear_bwd(f64(d["dY"]), f64(d["X"]), Ur, Wr, f64(d["A"]), f64(d["B"]), cfg.s)
    for g_, r_ in zip(out[1], (Yr, Ur, dXr, dAr, dBr)):
        assert rel_err(g_, r_) <= TOL
    # the noalloc forward accepts the double-quantized weight as well
    Yn, Un = Q.linear_fwd_noalloc(X, dqw, A, B, cfg.s, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(Yn, out[0][0]) and torch.equal(Un, out[0][1])


@pytest.mark.parametrize("mode", ["staged", "fused"])
def test_dq_mlp_equals_plain(mode):
    cfg = I.MlpCfg("dq_mlp", 257, 192, 320, 8, 1.0, "geglu_tanh", 0.01)
    d = I.mlp_inputs(cfg, dense_w=False, seed=22)
    ws = {}
    for wn in ("Wg", "Wu", "Wd"):
        ws[wn] = _dq_weight(d[wn + "_codes"], d[wn + "_absmax"])
    lora = [d[k].to(DEV) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")]
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    say(f"mlp with double-quantized absmax mode={mode}")
    res = []
    for i in (0, 1):
        w = Q.MlpWeights(ws["Wg"][i], ws["Wu"][i], ws["Wd"][i], *lora, s=cfg.s, act=cfg.act)
        Y, sv = Q.mlp_fwd(X, w, mode=mode)
        gr = Q.mlp_bwd(dY, X, sv, w, mode=mode)
        res.append(dict(Y=Y, **sv, **gr))
    torch.cuda.synchronize()
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k


def test_dq_qkv_equals_plain():
    cfg = I.QkvCfg("dq_qkv", 130, 256, 256, 128, 128, 8, 1.0)
    d = I.qkv_inputs(cfg, dense_w=False, seed=23)
    ws = {p: _dq_weight(d["W" + p + "_codes"], d["W" + p + "_absmax"]) for p in "qkv"}
    lora = [d[k + p].to(DEV) for p in "qkv" for k in ("A", "B")]
    X = d["X"].to(DEV)
    dys = [d["dY" + p].to(DEV) for p in "qkv"]
    say("qkv with double-quantized absmax")
    res = []
    for i in (0, 1):
        w = Q.QkvWeights(ws["q"][i], ws["k"][i], ws["v"][i], *lora, s=cfg.s)
        Yq, Yk, Yv, U = Q.qkv_fwd(X, w)
        gr = Q.qkv_bwd(*dys, X, U, w)
        res.append([Yq, Yk, Yv, U] + (list(gr.values()) if isinstance(gr, dict) else list(gr)))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        if a is None:
            continue
        assert torch.equal(a, b)
