"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: NF4 dequant bit-exact; every other output max|gpu - oracle| / max|oracle|
<= 2e-2 per tensor (the tolerance stated for this path: bf16 storage, fp32
accumulation). Inputs are the seeded synthetic workloads of
qlora_fine_tuning_amd.inputs; the oracle never sees a GPU value.

Sizes: small cases compare every element (several tiles, ragged token
counts); full-size workloads compare sampled token rows of every per-token
output (Y, g, u, U, dX depend only on their own row) and the full LoRA
gradients. The MLP's LoRA gradients sum over every token, so at full token
count the oracle computes them in row blocks (oracle.qlora.mlp_lora_grads,
the blocks added in fp64) on a pool of host threads. Identity inputs with
B = 0 turn the GEMMs into copies of the dequantized weight, which checks the
dequant inside every GEMM path bit for bit at the workloads' weight shapes.
"""
import concurrent.futures as cf
import dataclasses
import os

import numpy as np
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import qlora as OQ
from qlora_fine_tuning_amd import inputs as I

from _util import TOL, dequant_oracle, f64, need_gpu, quantize_dense, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _rows(m, n=32, seed=7):
    g = np.random.default_rng(seed)
    base = [0, 1, m - 1, m // 2]
    extra = g.choice(m, size=min(n, m), replace=False).tolist()
    return np.array(sorted(set([r for r in base + extra if 0 <= r < m])))


# ------------------------------------------------------------------ dequant --
@pytest.mark.parametrize("n,k", [(512, 256), (4096, 4096), (11008, 4096), (4096, 11008),
                                 (1024, 4096), (24576, 3072), (3072, 24576), (64, 64)])
def test_dequant_bit_exact(n, k):
    if (n, k) == (512, 256):
        codes, absmax = quantize_dense(I.normal_bf16("W", (n, k), 0.02))
    else:
        codes, absmax = I.synthetic_nf4("Wg", n, k)
    say(f"dequant {n}x{k}")
    w = Q.NF4Weight(codes.to(DEV), absmax.to(DEV))
    out = Q.nf4_dequant(w)
    torch.cuda.synchronize()
    from oracle import nf4 as onf4
    want = onf4.dequant_bf16_bits(codes.numpy(), absmax.numpy())
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_library_table_matches_oracle():
    from oracle import nf4 as onf4
    assert np.array_equal(Q.nf4_levels().numpy().view(np.uint32), onf4.nf4_levels().view(np.uint32))


# ------------------------------------------------------------- linear layer --
def _linear_case(m, k, n, r, s, dy_std=1.0, seed=3407, dense=True):
    cfg = I.LinearCfg("case", m, k, n, r, s, dy_std)
    d = I.linear_inputs(cfg, dense_w=dense, seed=seed)
    if dense:
        d["codes"], d["absmax"] = quantize_dense(d.pop("W"))
    return cfg, d


def _run_linear(cfg, d, mode):
    w = Q.NF4Weight(d["codes"].to(DEV), d["absmax"].to(DEV))
    X, A, B, dY = (d[k].to(DEV) for k in ("X", "A", "B", "dY"))
    say(f"linear m={cfg.m} k={cfg.k} n={cfg.n} r={cfg.r} mode={mode}")
    Y, U = Q.linear_fwd(X, w, A, B, cfg.s, mode=mode)
    dX, dA, dB = Q.linear_bwd(dY, X, U, w, A, B, cfg.s, mode=mode)
    torch.cuda.synchronize()
    return dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)


def _oracle_linear(cfg, d, rows=None):
    W = dequant_oracle(d["codes"], d["absmax"])
    X, A, B, dY = (f64(d[k]) for k in ("X", "A", "B", "dY"))
    U = X @ A.T
    T = dY @ B
    out = dict(U=U, dA=cfg.s * (T.T @ X), dB=cfg.s * (dY.T @ U))
    if rows is None:
        out["Y"], _ = OQ.linear_fwd(X, W, A, B, cfg.s)
        out["dX"], _, _, _ = OQ.linear_bwd(dY, X, U, W, A, B, cfg.s)
    else:
        out["Y"], _ = OQ.linear_fwd(X[rows], W, A, B, cfg.s)
        out["dX"], _, _, _ = OQ.linear_bwd(dY[rows], X[rows], U[rows], W, A, B, cfg.s)
    return out


def _check(got, want, rows=None, keys=None):
    errs = {}
    for k in keys or want:
        g = got[k]
        if rows is not None and k in ("Y", "dX", "g", "u", "Ug", "Uu", "Ud", "U"):
            g = g[torch.as_tensor(rows, device=g.device)]
            ref = want[k] if want[k].shape[0] == len(rows) else want[k][rows]
        else:
            ref = want[k]
        errs[k] = rel_err(g, ref)
    say(f"  rel errors: {errs}")
    for k, e in errs.items():
        assert e <= TOL, (k, e)
    return errs


@pytest.mark.parametrize("mode", ["staged", "fused"])
def test_linear_tiny(mode):
    cfg, d = _linear_case(256, 256, 512, 8, 2.0)
    got = _run_linear(cfg, d, mode)
    _check(got, _oracle_linear(cfg, d))


@pytest.mark.parametrize("m,k,n,r", [(1, 64, 64, 1), (17, 128, 192, 3), (300, 192, 320, 16),
                                     (513, 256, 128, 32), (64, 128, 64, 64), (129, 320, 576, 8)])
def test_linear_ragged_shapes(m, k, n, r):
    cfg, d = _linear_case(m, k, n, r, 16.0 / r, seed=11)
    for mode in ("staged", "fused"):
        _check(_run_linear(cfg, d, mode), _oracle_linear(cfg, d))


@pytest.mark.parametrize("m,k,n", [(300, 256, 320), (200, 2048, 1024), (96, 1024, 4096)])
def test_linear_fused_equals_staged_bitwise(m, k, n):
    """Fused and staged run the same kernel on the same bf16 values in the
    same order, so every output is equal bit for bit; the last two shapes
    have fewer output tiles than CUs, so both modes split K (forward and dX)."""
    cfg, d = _linear_case(m, k, n, 16, 1.0, seed=5)
    a = _run_linear(cfg, d, "staged")
    b = _run_linear(cfg, d, "fused")
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_linear_b_zero_reduces_to_base():
    cfg, d = _linear_case(256, 256, 512, 8, 2.0)
    d["B"] = torch.zeros_like(d["B"])
    got = _run_linear(cfg, d, "auto")
    want = _oracle_linear(cfg, d)
    _check(got, want)
    assert torch.count_nonzero(got["dA"]).item() == 0


@pytest.mark.parametrize("cfg", [I.QPROJ, I.MISTRAL_KV], ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["auto", "fused"])
def test_linear_full_size(cfg, mode):
    d = I.linear_inputs(cfg, dense_w=False, role="k" if cfg is I.MISTRAL_KV else "")
    got = _run_linear(cfg, d, mode)
    rows = _rows(cfg.m)
    want = _oracle_linear(cfg, d, rows=rows)
    _check(got, want, rows=rows)


# every base-weight shape of the workloads: q_proj, Mistral k/v, and the
# gate/up and down weights of the Llama, Mistral and Gemma MLPs
WEIGHT_SHAPES = [(4096, 4096), (1024, 4096), (11008, 4096), (4096, 11008), (14336, 4096),
                 (4096, 14336), (24576, 3072), (3072, 24576)]


@pytest.mark.parametrize("n,k", WEIGHT_SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("mode", ["staged", "fused"])
def test_linear_identity_input_gives_weight_bits(n, k, mode):
    """X = I (k tokens) and B = 0: Y = X W^T is W^T, every output element a
    single product 1 * w plus exact zeros, so Y must hold the dequantized
    weight bit for bit (forward: row dequant, or the in-LDS dequant of the
    fused GEMM). dY = I (n tokens) and B = 0: dX = dY W is W itself
    (backward: transposed dequant, or the fused transposed form)."""
    from oracle import nf4 as onf4
    codes, absmax = I.synthetic_nf4("W", n, k)
    want = onf4.dequant_bf16_bits(codes.numpy(), absmax.numpy())
    w = Q.NF4Weight(codes.to(DEV), absmax.to(DEV))
    r = 16
    A = I.kaiming_uniform_bf16("A", (r, k), k).to(DEV)
    B = torch.zeros((n, r), dtype=torch.bfloat16, device=DEV)
    say(f"identity fwd {n}x{k} mode={mode}")
    X = torch.eye(k, dtype=torch.bfloat16, device=DEV)
    Y, _ = Q.linear_fwd(X, w, A, B, 1.0, mode=mode)
    torch.cuda.synchronize()
    got = Y.t().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    del X, Y
    say(f"identity bwd {n}x{k} mode={mode}")
    dY = torch.eye(n, dtype=torch.bfloat16, device=DEV)
    Xz = torch.zeros((n, k), dtype=torch.bfloat16, device=DEV)
    Uz = torch.zeros((n, r), dtype=torch.float32, device=DEV)
    dX, dA, _ = Q.linear_bwd(dY, Xz, Uz, w, A, B, 1.0, mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(dX.cpu().view(torch.int16).numpy().view(np.uint16), want)
    assert torch.count_nonzero(dA).item() == 0
    del dY, Xz, dX
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- MLP block --
def _mlp_case(cfg, m=None, dense=False, seed=3407):
    d = I.mlp_inputs(cfg, dense_w=dense, seed=seed, m=m)
    if dense:
        for wn in ("Wg", "Wu", "Wd"):
            d[wn + "_codes"], d[wn + "_absmax"] = quantize_dense(d.pop(wn))
    return d


def _weights(cfg, d):
    nf = lambda wn: Q.NF4Weight(d[wn + "_codes"].to(DEV), d[wn + "_absmax"].to(DEV))  # noqa: E731
    return Q.MlpWeights(nf("Wg"), nf("Wu"), nf("Wd"),
                        *(d[k].to(DEV) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")),
                        s=cfg.s, act=cfg.act)


def _run_mlp(cfg, d, mode="auto"):
    w = _weights(cfg, d)
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    say(f"mlp {cfg.name} m={X.shape[0]} d={cfg.d} h={cfg.h} act={cfg.act} mode={mode}")
    Y, sv = Q.mlp_fwd(X, w, mode=mode)
    gr = Q.mlp_bwd(dY, X, sv, w, mode=mode)
    torch.cuda.synchronize()
    out = dict(Y=Y, **sv, **gr)
    return out


def _oracle_mlp(cfg, d, rows=None):
    W = {wn: dequant_oracle(d[wn + "_codes"], d[wn + "_absmax"]) for wn in ("Wg", "Wu", "Wd")}
    L = {k: f64(d[k]) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    X, dY = f64(d["X"]), f64(d["dY"])
    args = (W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"], L["Ad"], L["Bd"], cfg.s,
            cfg.act)
    if rows is not None:
        return OQ.mlp_rows(rows, X, dY, *args)
    Y, sv = OQ.mlp_fwd(X, *args)
    gr = OQ.mlp_bwd(dY, X, sv, *args)
    return dict(Y=Y, **sv, **gr)


TINY_MLP = [I.MlpCfg("tiny_swiglu", 200, 128, 192, 8, 2.0, "swiglu", 1.0),
            I.MlpCfg("tiny_geglu", 200, 128, 192, 8, 2.0, "geglu_tanh", 1.0),
            I.MlpCfg("odd_swiglu", 77, 64, 320, 3, 1.0, "swiglu", 1.0),
            I.MlpCfg("r32_geglu", 300, 192, 256, 32, 0.5, "geglu_tanh", 1.0),
            # r > 32: gate and up take separate row products and reductions
            I.MlpCfg("r64_swiglu", 150, 128, 192, 64, 0.25, "swiglu", 1.0),
            I.MlpCfg("r64_geglu", 97, 192, 256, 64, 0.5, "geglu_tanh", 1.0),
            I.MlpCfg("r33_swiglu", 130, 64, 128, 33, 1.0, "swiglu", 1.0),
            I.MlpCfg("r40_geglu", 64, 128, 320, 40, 0.4, "geglu_tanh", 1.0),
            # d = 320: 5 k-steps in the gate/up and dH GEMMs, so the last step's
            # free ring slots start at slot 0 (the other starts come from d = 64,
            # 128, 3072 and 4096)
            I.MlpCfg("d320_swiglu", 150, 320, 256, 8, 1.0, "swiglu", 1.0)]


@pytest.mark.parametrize("cfg", TINY_MLP, ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["staged", "fused"])
def test_mlp_small(cfg, mode):
    d = _mlp_case(cfg, dense=True)
    _check(_run_mlp(cfg, d, mode), _oracle_mlp(cfg, d))


@pytest.mark.parametrize("cfg", [TINY_MLP[0], I.MlpCfg("h256_geglu", 130, 128, 256, 16, 1.0,
                                                      "geglu_tanh", 1.0),
                                 # down and dX GEMMs split K (4 x 1 output tiles)
                                 I.MlpCfg("splitk_swiglu", 256, 1024, 2048, 16, 1.0, "swiglu", 1.0),
                                 I.MlpCfg("r40_splitk", 200, 1024, 2048, 40, 0.5, "geglu_tanh", 1.0)],
                         ids=lambda c: c.name)
def test_mlp_fused_matches_staged(cfg):
    """Dequantizing inside the GEMM gives the bits of the staged weight, and
    both modes run the same kernel with the same K order, row products and
    split-K, so every output of the two modes is equal bit for bit. The
    backward runs from one saved set in both modes."""
    d = _mlp_case(cfg, dense=True)
    w = _weights(cfg, d)
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    say(f"mlp staged/fused {cfg.name} m={X.shape[0]} d={cfg.d} h={cfg.h}")
    Ya, sva = Q.mlp_fwd(X, w, mode="staged")
    Yb, svb = Q.mlp_fwd(X, w, mode="fused")
    gra = Q.mlp_bwd(dY, X, sva, w, mode="staged")
    grb = Q.mlp_bwd(dY, X, sva, w, mode="fused")
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb), "Y"
    for k in sva:
        assert torch.equal(sva[k], svb[k]), k
    for k in gra:
        assert torch.equal(gra[k], grb[k]), k


@pytest.mark.parametrize("cfg", [I.LLAMA_MLP, I.MISTRAL_MLP, I.GEMMA_MLP,
                                 dataclasses.replace(I.LLAMA_MLP, name="llama7b_mlp_r64", r=64)],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("mode", ["auto", "fused"])
def test_mlp_full_weights_token_slice(cfg, mode):
    """Full-size weights, 512 tokens: every output including the LoRA gradients
    (fused: the in-LDS dequant of the gate/up pair and the transposed stacked
    gate/up weight at the workloads' widths)."""
    d = _mlp_case(cfg, m=512)
    _check(_run_mlp(cfg, d, mode), _oracle_mlp(cfg, d))


@pytest.mark.parametrize("cfg", [I.LLAMA_MLP, I.MISTRAL_MLP, I.GEMMA_MLP], ids=lambda c: c.name)
def test_mlp_identity_input_gives_gate_up_weight_bits(cfg):
    """X = I (d tokens) and Bg = Bu = 0: the saved g and u are Wg^T and Wu^T
    bit for bit (the interleaved gate/up dequant and the activation epilogue
    in staged mode, the paired in-LDS dequant in fused mode)."""
    from oracle import nf4 as onf4
    d = _mlp_case(cfg, m=8)
    for k in ("Bg", "Bu"):
        d[k] = torch.zeros_like(d[k])
    w = _weights(cfg, d)
    X = torch.eye(cfg.d, dtype=torch.bfloat16, device=DEV)
    for mode in ("staged", "fused"):
        say(f"mlp identity {cfg.name} mode={mode}")
        _, sv = Q.mlp_fwd(X, w, mode=mode)
        torch.cuda.synchronize()
        for wn, key in (("Wg", "g"), ("Wu", "u")):
            want = onf4.dequant_bf16_bits(d[wn + "_codes"].numpy(), d[wn + "_absmax"].numpy())
            got = sv[key].t().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got, want), (mode, key)
        del sv
    torch.cuda.empty_cache()


def _oracle_mlp_lora_grads(cfg, d, block=512):
    """The six LoRA gradients of the whole batch: oracle.qlora.mlp_lora_grads
    on row blocks, run on a pool of host threads (one BLAS thread each), the
    block results added in fp64 in block order."""
    from threadpoolctl import threadpool_limits
    W = {wn: dequant_oracle(d[wn + "_codes"], d[wn + "_absmax"]) for wn in ("Wg", "Wu", "Wd")}
    L = {k: f64(d[k]) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    args = (W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"], L["Ad"], L["Bd"], cfg.s,
            cfg.act)
    m = d["X"].shape[0]

    def one(a):
        return OQ.mlp_lora_grads(f64(d["X"][a:a + block]), f64(d["dY"][a:a + block]), *args)

    workers = max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(one, range(0, m, block)))
    out = parts[0]
    for p_ in parts[1:]:
        out = {k: out[k] + p_[k] for k in out}
    return out


@pytest.mark.parametrize("cfg", [I.LLAMA_MLP, I.MISTRAL_MLP, I.GEMMA_MLP], ids=lambda c: c.name)
def test_mlp_full_size(cfg):
    """The workloads at full token count: sampled rows of every per-token
    output, and the six LoRA gradients in full against the oracle's blockwise
    sum over all tokens (at 40960 tokens the row products and reductions run
    as separate passes instead of in the GEMM epilogues)."""
    d = _mlp_case(cfg)
    got = _run_mlp(cfg, d)
    rows = _rows(cfg.m, n=16)
    want = _oracle_mlp(cfg, d, rows=rows)
    _check(got, want, rows=rows, keys=["Y", "g", "u", "Ug", "Uu", "Ud", "dX"])
    grads = {k: got[k].cpu() for k in ("dAg", "dBg", "dAu", "dBu", "dAd", "dBd")}
    del got
    torch.cuda.empty_cache()
    say(f"  oracle LoRA gradients over {cfg.m} tokens")
    _check(grads, _oracle_mlp_lora_grads(cfg, d))


def test_mlp_deterministic():
    cfg = I.LLAMA_MLP
    d = _mlp_case(cfg, m=512)
    a = _run_mlp(cfg, d)
    b = _run_mlp(cfg, d)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_mlp_b_zero_gives_zero_a_grads():
    cfg = TINY_MLP[0]
    d = _mlp_case(cfg, dense=True)
    for k in ("Bg", "Bu", "Bd"):
        d[k] = torch.zeros_like(d[k])
    got = _run_mlp(cfg, d)
    _check(got, _oracle_mlp(cfg, d), keys=["Y", "dX", "dBg", "dBu", "dBd"])
    for k in ("dAg", "dAu", "dAd"):
        assert torch.count_nonzero(got[k]).item() == 0, k


def test_empty_batch_writes_zero_lora_grads():
    # m == 0: no token contributes, so every LoRA gradient is zero; the
    # per-token tensors are empty (null device pointers)
    cfg, d = _linear_case(4, 128, 192, 8, 2.0)
    w = Q.NF4Weight(d["codes"].to(DEV), d["absmax"].to(DEV))
    A, B = d["A"].to(DEV), d["B"].to(DEV)
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=DEV)  # noqa: E731
    dA = torch.full((8, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    dB = torch.full((192, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    U0 = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    _, dA2, dB2 = Q.linear_bwd(e(0, 192), e(0, 128), U0, w, A, B, 2.0)
    mc = I.MlpCfg("empty", 4, 64, 128, 4, 1.0, "swiglu", 1.0)
    md = _mlp_case(mc, dense=True)
    mw = _weights(mc, md)
    sv = dict(g=e(0, 128), u=e(0, 128), **{k: torch.empty((0, 4), dtype=torch.float32, device=DEV)
                                           for k in ("Ug", "Uu", "Ud")})
    gr = Q.mlp_bwd(e(0, 64), e(0, 64), sv, mw)
    torch.cuda.synchronize()
    for t in (dA2, dB2, *(gr[k] for k in ("dAg", "dBg", "dAu", "dBu", "dAd", "dBd"))):
        assert torch.count_nonzero(t).item() == 0
