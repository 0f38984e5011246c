"""GPU parity of the 16-bit base-weight variant (qlora_linear16_*, qlora_mlp16_*).

The layer is the one of the NF4 path with W a plain bf16 matrix. Two pins:
- the fp64 oracle on the same bf16 W (max|gpu - oracle| / max|oracle| <= 2e-2
  per output), on ragged shapes, both activations and a full-width slice;
- with W equal to the oracle's dequantization of an NF4 weight, every output
  equals the NF4 staged path's output bit for bit (the two paths run the same
  GEMM on the same bf16 operand).
"""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import nf4 as onf4
from oracle import qlora as OQ
from qlora_fine_tuning_amd import inputs as I

from _util import TOL, f64, need_gpu, quantize_dense, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check(got, want):
    errs = {k: rel_err(got[k], want[k]) for k in want}
    say(f"  rel errors: {errs}")
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def _bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)


# ------------------------------------------------------------------ linear --
def _run_linear16(cfg, d):
    X, W, A, B, dY = (d[k].to(DEV) for k in ("X", "W", "A", "B", "dY"))
    say(f"linear16 m={cfg.m} k={cfg.k} n={cfg.n} r={cfg.r}")
    Y, U = Q.linear16_fwd(X, W, A, B, cfg.s)
    dX, dA, dB = Q.linear16_bwd(dY, X, U, W, A, B, cfg.s)
    torch.cuda.synchronize()
    return dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)


@pytest.mark.parametrize("m,k,n,r", [(1, 64, 64, 1), (17, 128, 192, 3), (300, 192, 320, 16),
                                     (129, 320, 576, 8), (64, 128, 64, 64)])
def test_linear16_matches_oracle(m, k, n, r):
    cfg = I.LinearCfg("w16", m, k, n, r, 16.0 / r, 1.0)
    d = I.linear_inputs(cfg, dense_w=True, seed=13)
    got = _run_linear16(cfg, d)
    X, W, A, B, dY = (f64(d[k_]) for k_ in ("X", "W", "A", "B", "dY"))
    Y, U = OQ.linear_fwd(X, W, A, B, cfg.s)
    dX, dA, dB, _ = OQ.linear_bwd(dY, X, U, W, A, B, cfg.s)
    _check(got, dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB))


@pytest.mark.parametrize("r", [16, 64])
def test_linear16_rank_stabilized_scale(r):
    # RSLoRA: s = alpha / sqrt(r) instead of alpha / r (alpha 16)
    cfg = I.LinearCfg("rslora", 200, 256, 192, r, 16.0 / np.sqrt(r), 1.0)
    d = I.linear_inputs(cfg, dense_w=True, seed=17)
    got = _run_linear16(cfg, d)
    X, W, A, B, dY = (f64(d[k_]) for k_ in ("X", "W", "A", "B", "dY"))
    Y, U = OQ.linear_fwd(X, W, A, B, cfg.s)
    dX, dA, dB, _ = OQ.linear_bwd(dY, X, U, W, A, B, cfg.s)
    _check(got, dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB))


def test_linear16_equals_nf4_staged_bitwise():
    cfg = I.LinearCfg("w16", 300, 256, 320, 16, 1.0, 1.0)
    d = I.linear_inputs(cfg, dense_w=True, seed=5)
    codes, absmax = quantize_dense(d.pop("W"))
    d["W"] = _bf16_from_bits(onf4.dequant_bf16_bits(codes.numpy(), absmax.numpy()))
    a = _run_linear16(cfg, d)
    w = Q.NF4Weight(codes.to(DEV), absmax.to(DEV))
    X, A, B, dY = (d[k].to(DEV) for k in ("X", "A", "B", "dY"))
    Y, U = Q.linear_fwd(X, w, A, B, cfg.s, mode="staged")
    dX, dA, dB = Q.linear_bwd(dY, X, U, w, A, B, cfg.s, mode="staged")
    torch.cuda.synchronize()
    b = dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB)
    for k in a:
        assert torch.equal(a[k], b[k]), k


# --------------------------------------------------------------------- MLP --
def _w16(cfg, d):
    return Q.Mlp16Weights(d["Wg"].to(DEV), d["Wu"].to(DEV), d["Wd"].to(DEV),
                          *(d[k].to(DEV) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")),
                          s=cfg.s, act=cfg.act)


def _run_mlp16(cfg, d):
    w = _w16(cfg, d)
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    say(f"mlp16 {cfg.name} m={X.shape[0]} d={cfg.d} h={cfg.h} act={cfg.act}")
    Y, sv = Q.mlp16_fwd(X, w)
    gr = Q.mlp16_bwd(dY, X, sv, w)
    torch.cuda.synchronize()
    return dict(Y=Y, **sv, **gr)


def _oracle_mlp16(cfg, d):
    args = tuple(f64(d[k]) for k in ("Wg", "Wu", "Wd", "Ag", "Bg", "Au", "Bu", "Ad", "Bd"))
    X, dY = f64(d["X"]), f64(d["dY"])
    Y, sv = OQ.mlp_fwd(X, *args, cfg.s, cfg.act)
    gr = OQ.mlp_bwd(dY, X, sv, *args, cfg.s, cfg.act)
    return dict(Y=Y, **sv, **gr)


MLP16 = [I.MlpCfg("w16_swiglu", 200, 128, 192, 8, 2.0, "swiglu", 1.0),
         I.MlpCfg("w16_geglu", 77, 64, 320, 3, 1.0, "geglu_tanh", 1.0),
         I.MlpCfg("w16_r32", 300, 192, 256, 32, 0.5, "swiglu", 1.0)]


@pytest.mark.parametrize("cfg", MLP16, ids=lambda c: c.name)
def test_mlp16_matches_oracle(cfg):
    d = I.mlp_inputs(cfg, dense_w=True, seed=17)
    _check(_run_mlp16(cfg, d), _oracle_mlp16(cfg, d))


def test_mlp16_full_width_slice():
    # Llama-7B MLP widths with a 512-token slice: every output in full
    cfg = I.LLAMA_MLP
    d = I.mlp_inputs(cfg, dense_w=True, m=512)
    _check(_run_mlp16(cfg, d), _oracle_mlp16(cfg, d))


def test_mlp16_equals_nf4_staged_bitwise():
    cfg = I.MlpCfg("w16_eq", 300, 192, 320, 16, 1.0, "swiglu", 1.0)
    d = I.mlp_inputs(cfg, dense_w=True, seed=9)
    nf = {}
    for wn in ("Wg", "Wu", "Wd"):
        codes, absmax = quantize_dense(d[wn])
        nf[wn] = Q.NF4Weight(codes.to(DEV), absmax.to(DEV))
        d[wn] = _bf16_from_bits(onf4.dequant_bf16_bits(codes.numpy(), absmax.numpy()))
    a = _run_mlp16(cfg, d)
    w = Q.MlpWeights(nf["Wg"], nf["Wu"], nf["Wd"],
                     *(d[k].to(DEV) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")), s=cfg.s, act=cfg.act)
    X, dY = d["X"].to(DEV), d["dY"].to(DEV)
    Y, sv = Q.mlp_fwd(X, w, mode="staged")
    gr = Q.mlp_bwd(dY, X, sv, w, mode="staged")
    torch.cuda.synchronize()
    b = dict(Y=Y, **sv, **gr)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_mlp16_empty_batch_zero_grads():
    cfg = I.MlpCfg("w16_empty", 0, 64, 128, 4, 1.0, "swiglu", 1.0)
    d = I.mlp_inputs(cfg, dense_w=True, m=4)
    w = _w16(cfg, d)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    sv = dict(g=torch.empty((0, 128), dtype=torch.bfloat16, device=DEV),
              u=torch.empty((0, 128), dtype=torch.bfloat16, device=DEV),
              Ug=torch.empty((0, 4), dtype=torch.float32, device=DEV),
              Uu=torch.empty((0, 4), dtype=torch.float32, device=DEV),
              Ud=torch.empty((0, 4), dtype=torch.float32, device=DEV))
    gr = Q.mlp16_bwd(X, X, sv, w)
    torch.cuda.synchronize()
    for k in ("dAg", "dBg", "dAu", "dBu", "dAd", "dBd"):
        assert torch.count_nonzero(gr[k]).item() == 0, k
