"""Pins of the oracle's QLoRA linear layer (oracle/qlora.py).

- B = 0 or s = 0 reduces the layer to the plain product X W^T, bit for bit;
- the rank-first bracketing equals the merged-weight form X (W + s B A)^T
  (formed here only, never by the method);
- the manual backward equals central finite differences of <dY, Y> (exact up
  to rounding, since Y is linear in each of X, A, B) and torch autograd;
- B = 0 gives dA = 0 exactly and dX = dY W.
"""
import numpy as np
import torch

from oracle import qlora as Q


def _case(m=5, k=8, n=6, r=3, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((m, k)), g.standard_normal((n, k)) * 0.3,
            g.standard_normal((r, k)) * 0.5, g.standard_normal((n, r)) * 0.5,
            g.standard_normal((m, n)))


def test_b_zero_and_s_zero_reduce_to_plain_product():
    X, W, A, B, _ = _case()
    Y, _ = Q.linear_fwd(X, W, A, np.zeros_like(B), 2.0)
    assert np.array_equal(Y, X @ W.T)
    Y0, _ = Q.linear_fwd(X, W, A, B, 0.0)
    assert np.array_equal(Y0, X @ W.T)


def test_bracketing_equals_merged_weight():
    X, W, A, B, _ = _case(m=7, k=16, n=12, r=4, seed=1)
    s = 1.75
    Y, U = Q.linear_fwd(X, W, A, B, s)
    merged = X @ (W + s * B @ A).T
    assert np.max(np.abs(Y - merged)) <= 1e-12 * np.max(np.abs(merged))
    assert np.allclose(U, X @ A.T, rtol=0, atol=0)


def _loss(dY, X, W, A, B, s):
    return float(np.sum(dY * Q.linear_fwd(X, W, A, B, s)[0]))


def test_backward_matches_central_differences():
    X, W, A, B, dY = _case(seed=2)
    s = 2.0
    _, U = Q.linear_fwd(X, W, A, B, s)
    dX, dA, dB, T = Q.linear_bwd(dY, X, U, W, A, B, s)
    for name, P, G in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + 0.5
            lp = _loss(dY, X, W, A, B, s)
            P[idx] = old - 0.5
            lm = _loss(dY, X, W, A, B, s)
            P[idx] = old
            fd[idx] = (lp - lm) / 1.0
        err = np.max(np.abs(fd - G)) / np.max(np.abs(G))
        assert err < 1e-12, (name, err)


def test_backward_matches_torch_autograd():
    X, W, A, B, dY = _case(m=9, k=10, n=7, r=2, seed=3)
    s = 0.5
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    tY = tX @ torch.tensor(W).T + s * (tX @ tA.T) @ tB.T
    (tY * torch.tensor(dY)).sum().backward()
    _, U = Q.linear_fwd(X, W, A, B, s)
    dX, dA, dB, _ = Q.linear_bwd(dY, X, U, W, A, B, s)
    for mine, ref in ((dX, tX.grad), (dA, tA.grad), (dB, tB.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_b_zero_backward():
    X, W, A, B, dY = _case(seed=4)
    Bz = np.zeros_like(B)
    _, U = Q.linear_fwd(X, W, A, Bz, 2.0)
    dX, dA, dB, _ = Q.linear_bwd(dY, X, U, W, A, Bz, 2.0)
    assert np.array_equal(dA, np.zeros_like(dA))
    assert np.array_equal(dX, dY @ W)
    assert np.abs(dB).max() > 0
