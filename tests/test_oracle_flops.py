"""Pins of the oracle's FLOP accounting against the pages' printed numbers.

The Mistral benchmark page (breakdown items 10-11) gives the slow and fast
costs of the LoRA gradient chain, (h d)(m + r) and (m r)(h + d), and prints the
large-m ratios 186.58 (Llama 7b) and 398.22 (Llama 70b); both are stored in
tests/golden/bracketing_ratios.txt with that citation. The per-layer FLOP
counters are pinned by counting, product by product, the matrix products the
oracle's own forward and backward take.
"""
import os

import numpy as np
import pytest

from oracle import qlora as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bracketing_ratios.txt")


def test_chain_costs_are_the_pages_closed_forms():
    for m, d, h, r in ((8192, 4096, 11008, 16), (16384, 8192, 28672, 64), (7, 3, 5, 2)):
        _, slow, fast = Q.lora_grad_bracketing_ratio(m, d, h, r)
        assert slow == h * d * (m + r)
        assert fast == m * r * (h + d)


def test_large_m_ratio_reproduces_printed_values():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 2
    for _, h, d, r, printed in rows:
        ratio, _, _ = Q.lora_grad_bracketing_ratio(10 ** 12, int(d), int(h), int(r))
        assert f"{ratio:.2f}" == printed


def test_mlp_flops_count_six_base_products():
    m, d, h, r = 8192, 4096, 11008, 16
    f = Q.mlp_algorithmic_flops(m, d, h, r)
    # each base product is 2*m*d*h; the LoRA share is under 1%
    assert 6 * 2 * m * d * h < f < 1.01 * 6 * 2 * m * d * h
    assert f == 4468041056256


class _Counted(np.ndarray):
    """An ndarray that tallies the multiply-accumulates of every matrix product
    it takes part in (p x q times q x t costs p*q*t), so the oracle's own
    forward and backward can be counted product by product."""
    macs = 0

    def __array_ufunc__(self, ufunc, method, *inputs, **kw):
        args = [np.asarray(x) if isinstance(x, _Counted) else x for x in inputs]
        if ufunc is np.matmul and method == "__call__":
            a, b = args[0], args[1]
            assert a.ndim == 2 and b.ndim == 2
            _Counted.macs += a.shape[0] * a.shape[1] * b.shape[1]
        out = getattr(ufunc, method)(*args, **kw)
        return out.view(_Counted) if isinstance(out, np.ndarray) else out


def _c(g, *shape):
    return g.standard_normal(shape).view(_Counted)


def _count(fn):
    _Counted.macs = 0
    fn()
    return _Counted.macs


SHAPES = ((5, 64, 128, 2), (17, 192, 64, 3), (3, 128, 320, 8), (1, 64, 64, 1))


@pytest.mark.parametrize("m,k,n,r", SHAPES)
def test_linear_flops_count_the_oracles_products(m, k, n, r):
    """Two FLOPs per multiply-accumulate of the matrix products the oracle's
    linear forward and backward actually take (rank-r bracketing)."""
    g = np.random.default_rng(m * 1000 + k)
    X, W, A, B, dY = _c(g, m, k), _c(g, n, k), _c(g, r, k), _c(g, n, r), _c(g, m, n)

    def run():
        Y, U = Q.linear_fwd(X, W, A, B, 0.5)
        Q.linear_bwd(dY, X, U, W, A, B, 0.5)

    assert 2 * _count(run) == Q.linear_algorithmic_flops(m, k, n, r)


@pytest.mark.parametrize("m,d,h,r", SHAPES)
@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_flops_count_the_oracles_products(m, d, h, r, act):
    g = np.random.default_rng(m * 1000 + d + 7)
    X, dY = _c(g, m, d), _c(g, m, d)
    Wg, Wu, Wd = _c(g, h, d), _c(g, h, d), _c(g, d, h)
    L = (_c(g, r, d), _c(g, h, r), _c(g, r, d), _c(g, h, r), _c(g, r, h), _c(g, d, r))

    def run():
        _, sv = Q.mlp_fwd(X, Wg, Wu, Wd, *L, 1.0, act)
        Q.mlp_bwd(dY, X, sv, Wg, Wu, Wd, *L, 1.0, act)

    assert 2 * _count(run) == Q.mlp_algorithmic_flops(m, d, h, r)


@pytest.mark.parametrize("m,d,r", [(5, 64, 2), (9, 128, 4)])
def test_qkv_flops_count_the_oracles_products(m, d, r):
    g = np.random.default_rng(m + d)
    ns = (128, 64, 64)
    X = _c(g, m, d)
    Ws = [_c(g, n, d) for n in ns]
    As = [_c(g, r, d) for _ in ns]
    Bs = [_c(g, n, r) for n in ns]
    dYs = [_c(g, m, n) for n in ns]

    def run():
        _, Us = Q.qkv_fwd(X, Ws, As, Bs, 1.0)
        Q.qkv_bwd(dYs, X, Us, Ws, As, Bs, 1.0)

    assert 2 * _count(run) == Q.qkv_algorithmic_flops(m, d, ns, r)


def test_counter_sees_every_product():
    # the counting array itself: a chain of known cost, and the count for the
    # page's fast bracketing agrees with chain_macs
    g = np.random.default_rng(0)
    Xt, dW, Bt = _c(g, 6, 11), _c(g, 11, 9), _c(g, 9, 2)
    assert _count(lambda: Xt @ (dW @ Bt)) == Q.chain_macs([(6, 11), (11, 9), (9, 2)], (0, (1, 2)))[0]
    assert _count(lambda: (Xt @ dW) @ Bt) == 6 * 11 * 9 + 6 * 9 * 2


def test_linear_flops_at_the_two_linear_workloads():
    # tiny linear layer (256 tokens, 256 -> 512, r 8) and Llama-7B q_proj
    # (8192 tokens, 4096 -> 4096, r 16), worked by hand:
    # 4*256*256*512 + 6*256*8*(256+512) = 134217728 + 9437184
    assert Q.linear_algorithmic_flops(256, 256, 512, 8) == 143654912
    # 4*8192*4096*4096 + 6*8192*16*(4096+4096) = 549755813888 + 6442450944
    assert Q.linear_algorithmic_flops(8192, 4096, 4096, 16) == 556198264832


def test_bench_formulas_equal_the_oracle():
    import bench
    for m, k, n, r in SHAPES + ((8192, 4096, 11008, 16), (40960, 3072, 24576, 16)):
        assert bench.linear_flops(m, k, n, r) == Q.linear_algorithmic_flops(m, k, n, r)
        assert bench.mlp_flops(m, k, n, r) == Q.mlp_algorithmic_flops(m, k, n, r)
        ns = (n, n // 4, n // 4)
        assert bench.qkv_flops(m, k, ns, r) == Q.qkv_algorithmic_flops(m, k, ns, r)
