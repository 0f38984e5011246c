"""The no-allocation linear forward (qlora_linear_fwd_noalloc) against the
workspace entry point qlora_linear_fwd, both called through the C ABI.

Two calls in a row on the library's per-device scratch, the second with a
smaller input (what the first left in the scratch must not matter), each
compared with qlora_linear_fwd on the same inputs (same kernels, so the bits
must agree) and with the fp64 oracle (2e-2 of the largest magnitude). A call
larger than the scratch is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import qlora_fine_tuning_amd as Q
from oracle import qlora as OQ
from qlora_fine_tuning_amd import _lib
from qlora_fine_tuning_amd import inputs as I

from _util import TOL, dequant_oracle, f64, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_both(cfg, d, mode):
    L = _lib.lib()
    w = Q.NF4Weight(d["codes"].to(DEV), d["absmax"].to(DEV))
    X, A, B = (d[k].to(DEV) for k in ("X", "A", "B"))
    m, n, r = cfg.m, cfg.n, cfg.r
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    Ya = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    Ua = torch.empty((m, r), dtype=torch.float32, device=DEV)
    nb = L.qlora_linear_workspace_bytes(m, cfg.k, n, r, _lib.MODE[mode])
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    say(f"linear fwd (workspace) m={m} k={cfg.k} n={n} r={r} mode={mode}")
    rc = L.qlora_linear_fwd(_p(X), m, w.c_struct(), _p(A), _p(B), r, float(cfg.s), _p(Ya), _p(Ua),
                            _lib.MODE[mode], _p(ws), nb, st)
    assert rc == 0
    Yb = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV)
    Ub = torch.full((m, r), 7.0, dtype=torch.float32, device=DEV)
    say(f"linear fwd (no allocation) m={m} k={cfg.k} n={n} r={r} mode={mode} scratch need {nb}")
    rc = L.qlora_linear_fwd_noalloc(_p(X), m, w.c_struct(), _p(A), _p(B), r, float(cfg.s), _p(Yb),
                                    _p(Ub), _lib.MODE[mode], st)
    assert rc == 0, L.qlora_last_error()
    torch.cuda.synchronize()
    return Ya, Ua, Yb, Ub


def _oracle(cfg, d):
    W = dequant_oracle(d["codes"], d["absmax"])
    return OQ.linear_fwd(f64(d["X"]), W, f64(d["A"]), f64(d["B"]), cfg.s)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_noalloc_matches_workspace_entry_point_twice():
    # first: the Llama-7B q_proj at 8192 tokens, staged (the bf16 weight copy
    # and the row-product partials live in the scratch); then smaller calls: a
    # ragged one whose GEMM splits K (fp32 partials in the scratch) and a
    # fused-mode one
    cases = [(I.LinearCfg("noalloc_qproj", 8192, 4096, 4096, 16, 1.0, 1.0), "staged"),
             (I.LinearCfg("noalloc_split", 129, 1024, 4160, 8, 2.0, 1.0), "staged"),
             (I.LinearCfg("noalloc_fused", 77, 256, 320, 3, 0.5, 1.0), "fused")]
    for cfg, mode in cases:
        d = I.linear_inputs(cfg, dense_w=False, seed=cfg.m)
        Ya, Ua, Yb, Ub = _call_both(cfg, d, mode)
        assert torch.equal(Ya, Yb) and torch.equal(Ua, Ub), cfg.name
        Yr, Ur = _oracle(cfg, d)
        assert rel_err(Yb, Yr) <= TOL and rel_err(Ub, Ur) <= TOL, cfg.name


def test_noalloc_refuses_more_than_its_scratch():
    L = _lib.lib()
    cap = L.qlora_linear_fwd_noalloc_max_bytes()
    assert cap == 64 << 20
    # staged gate projection at 8192 tokens: the bf16 weight copy alone is 90 MB
    f = ctypes.c_void_p(0x1000)
    rc = L.qlora_linear_fwd_noalloc(f, 8192, _lib.Nf4(0x1000, 0x2000, 11008, 4096), f, f, 16, 1.0, f,
                                    f, _lib.MODE["staged"], None)
    assert rc == -3
    msg = L.qlora_last_error().decode()
    assert str(cap) in msg and "bytes of scratch" in msg
