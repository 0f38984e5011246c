"""Pins of the oracle's q, k, v projections on one shared input (oracle/qlora.py).

- torch autograd (fp64) of sum_p <dY_p, Y_p> for dX and all six LoRA factors;
- the merged-weight form: Y_p = X (W_p + s B_p A_p)^T and
  dX = sum_p dY_p (W_p + s B_p A_p), formed only here;
- central finite differences in X (exact up to rounding: the map is linear);
- zero k and v weights and factors reduce dX to the q layer's alone;
- the FLOP count adds three linear layers.
"""
import numpy as np
import pytest
import torch

from oracle import qlora as Q


def _case(m=5, d=128, ns=(128, 64, 64), r=3, s=0.7, seed=0):
    g = np.random.default_rng(seed)
    X = g.standard_normal((m, d))
    Ws = [g.standard_normal((n, d)) * 0.1 for n in ns]
    As = [g.standard_normal((r, d)) * 0.2 for _ in ns]
    Bs = [g.standard_normal((n, r)) * 0.2 for n in ns]
    dYs = [g.standard_normal((m, n)) for n in ns]
    return X, Ws, As, Bs, dYs, s


@pytest.mark.parametrize("seed", [0, 1])
def test_qkv_matches_torch_autograd(seed):
    X, Ws, As, Bs, dYs, s = _case(seed=seed)
    Ys, Us = Q.qkv_fwd(X, Ws, As, Bs, s)
    dX, dA, dB = Q.qkv_bwd(dYs, X, Us, Ws, As, Bs, s)
    tX = torch.tensor(X, requires_grad=True)
    tA = [torch.tensor(a, requires_grad=True) for a in As]
    tB = [torch.tensor(b, requires_grad=True) for b in Bs]
    loss = 0
    for p in range(3):
        Y = tX @ torch.tensor(Ws[p]).T + s * (tX @ tA[p].T) @ tB[p].T
        assert np.allclose(Y.detach().numpy(), Ys[p], rtol=1e-13, atol=1e-13)
        loss = loss + (Y * torch.tensor(dYs[p])).sum()
    loss.backward()
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    for p in range(3):
        assert np.allclose(dA[p], tA[p].grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(dB[p], tB[p].grad.numpy(), rtol=1e-12, atol=1e-12)


def test_qkv_merged_weight_form():
    X, Ws, As, Bs, dYs, s = _case(ns=(192, 64, 128), r=4, seed=2)
    Ys, Us = Q.qkv_fwd(X, Ws, As, Bs, s)
    dX, _, _ = Q.qkv_bwd(dYs, X, Us, Ws, As, Bs, s)
    merged = [W + s * (B @ A) for W, A, B in zip(Ws, As, Bs)]
    for p in range(3):
        assert np.allclose(Ys[p], X @ merged[p].T, rtol=1e-12, atol=1e-12)
    ref = sum(dY @ Wm for dY, Wm in zip(dYs, merged))
    assert np.allclose(dX, ref, rtol=1e-12, atol=1e-12)


def test_qkv_dx_central_difference():
    X, Ws, As, Bs, dYs, s = _case(m=2, d=64, ns=(64, 64, 64), r=2, seed=3)
    Ys, Us = Q.qkv_fwd(X, Ws, As, Bs, s)
    dX, _, _ = Q.qkv_bwd(dYs, X, Us, Ws, As, Bs, s)

    def loss(Xv):
        Yv, _ = Q.qkv_fwd(Xv, Ws, As, Bs, s)
        return sum(float((Y * dY).sum()) for Y, dY in zip(Yv, dYs))

    h = 1e-3
    fd = np.zeros_like(X)
    for i in range(X.shape[0]):
        for j in range(X.shape[1]):
            E = np.zeros_like(X)
            E[i, j] = h
            fd[i, j] = (loss(X + E) - loss(X - E)) / (2 * h)
    assert np.max(np.abs(fd - dX)) <= 1e-9 * np.max(np.abs(dX))


def test_qkv_reduces_to_one_linear_layer():
    X, Ws, As, Bs, dYs, s = _case(seed=4)
    for p in (1, 2):
        Ws[p] = np.zeros_like(Ws[p])
        Bs[p] = np.zeros_like(Bs[p])
    Ys, Us = Q.qkv_fwd(X, Ws, As, Bs, s)
    dX, dA, dB = Q.qkv_bwd(dYs, X, Us, Ws, As, Bs, s)
    dXq, _, _, _ = Q.linear_bwd(dYs[0], X, Us[0], Ws[0], As[0], Bs[0], s)
    assert np.array_equal(dX, dXq + 0.0)
    for p in (1, 2):
        assert not Ys[p].any() and not dA[p].any()


def test_qkv_flops_adds_three_layers():
    m, d, r = 8192, 4096, 16
    # one layer: 4 m k n base + 6 m r (k + n) LoRA
    want = sum(4 * m * d * n + 6 * m * r * (d + n) for n in (4096, 1024, 1024))
    assert Q.qkv_algorithmic_flops(m, d, (4096, 1024, 1024), r) == want
