"""GPU parity of the split-K base GEMM (outputs with fewer than 256 tiles).

A store-epilogue GEMM on a bf16 weight whose output has few 256 x 256 tiles
runs as several K ranges writing fp32 partials, summed afterwards in a fixed
order. The shapes below are chosen so that every GEMM of the case splits
(2 to 8 ranges, including a short last range and the LoRA K-extension riding
on the first range), checked against the fp64 oracle:
- linear layer, NF4 staged and 16-bit paths (forward and dX GEMMs), with the
  unsplit fused-dequant path on the same inputs as a second witness;
- gated MLP, down and dX GEMMs, both activations;
- q/k/v, the three-way routed forward store and the K-segmented dX GEMM whose
  split boundaries fall inside and on the projection boundaries.
"""
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import qlora as OQ
from qlora_fine_tuning_amd import inputs as I

import test_gpu_parity as TP
import test_gpu_qkv as TQ
from _util import TOL, f64, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("m,k,n,r,fwd_sp,bwd_sp", [(300, 2368, 320, 16, 4, 1),
                                                   (129, 1024, 4160, 8, 2, 8),
                                                   (1, 1536, 64, 4, 3, 1)])
def test_linear_split(m, k, n, r, fwd_sp, bwd_sp):
    assert Q.gemm_split_count(m, n, k) == fwd_sp and Q.gemm_split_count(m, k, n) == bwd_sp
    cfg, d = TP._linear_case(m, k, n, r, 16.0 / r, seed=31)
    want = TP._oracle_linear(cfg, d)
    for mode in ("staged", "fused"):
        TP._check(TP._run_linear(cfg, d, mode), want)


def test_linear16_split():
    m, k, n, r = 129, 1024, 4160, 8
    cfg = I.LinearCfg("w16", m, k, n, r, 2.0, 1.0)
    d = I.linear_inputs(cfg, dense_w=True, seed=32)
    X, W, A, B, dY = (d[k_].to(DEV) for k_ in ("X", "W", "A", "B", "dY"))
    say(f"linear16 split m={m} k={k} n={n} r={r}")
    Y, U = Q.linear16_fwd(X, W, A, B, cfg.s)
    dX, dA, dB = Q.linear16_bwd(dY, X, U, W, A, B, cfg.s)
    torch.cuda.synchronize()
    X, W, A, B, dY = (f64(d[k_]) for k_ in ("X", "W", "A", "B", "dY"))
    Yo, Uo = OQ.linear_fwd(X, W, A, B, cfg.s)
    dXo, dAo, dBo, _ = OQ.linear_bwd(dY, X, Uo, W, A, B, cfg.s)
    errs = {"Y": rel_err(Y, Yo), "dX": rel_err(dX, dXo), "dA": rel_err(dA, dAo), "dB": rel_err(dB, dBo)}
    say(f"  rel errors: {errs}")
    assert max(errs.values()) <= TOL, errs


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_split(act):
    cfg = I.MlpCfg("split_" + act, 200, 1024, 2816, 8, 2.0, act, 1.0)
    assert Q.gemm_split_count(cfg.m, cfg.d, cfg.h) == 5          # down
    assert Q.gemm_split_count(cfg.m, cfg.d, 2 * cfg.h) == 8      # dX
    d = TP._mlp_case(cfg, dense=True, seed=33)
    TP._check(TP._run_mlp(cfg, d, "staged"), TP._oracle_mlp(cfg, d))


@pytest.mark.parametrize("w16", [False, True])
def test_qkv_split(w16):
    cfg = I.QkvCfg("split", 100, 1024, 1024, 256, 256, 8, 2.0, 1.0)
    assert Q.gemm_split_count(cfg.m, 1536, cfg.d) == 2           # forward, three-way store
    assert Q.gemm_split_count(cfg.m, cfg.d, 1536) == 3           # dX over [dY_q | dY_k | dY_v]
    d = TQ._case(cfg, w16=w16, seed=34)
    TQ._check(TQ._run(cfg, d, w16=w16), TQ._oracle(cfg, d, w16=w16))


def test_split_results_are_deterministic():
    cfg, d = TP._linear_case(129, 1024, 4160, 8, 2.0, seed=35)
    a = TP._run_linear(cfg, d, "staged")
    b = TP._run_linear(cfg, d, "staged")
    for key in a:
        assert torch.equal(a[key], b[key]), key
