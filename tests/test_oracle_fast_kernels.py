"""Pins of the oracle's RMS layernorm, RoPE and cross entropy (oracle/fast_kernels.py).

- RMS layernorm: torch's rms_norm (fp64) for the forward, Llama and Gemma
  weights; torch autograd for dX; scale invariance at eps = 0; unit mean square
  at w = 1; central differences.
- RoPE: the explicit block-rotation matrix R (formed only here) for the
  forward and R^T for the backward; position 0 is the identity; pair norms
  are kept; the backward inverts the forward; <rope(q, p1), rope(k, p2)>
  depends on p1 - p2 only; torch autograd of the half-rotation formula.
- Cross entropy: torch's cross_entropy (mean, ignore_index -100, fp64) and its
  autograd gradient, including a vocabulary above 65536; invariance to a
  per-row shift; gradient rows sum to zero; scipy's logsumexp at large values;
  all rows ignored gives 0.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import fast_kernels as F


# ----------------------------------------------------------- RMS layernorm --
def _norm_case(m=6, d=256, seed=0):
    g = np.random.default_rng(seed)
    return g.standard_normal((m, d)) * 1.7, g.standard_normal(d) * 0.3 + 1.0, g.standard_normal((m, d))


@pytest.mark.parametrize("gemma", [False, True])
def test_rmsnorm_matches_torch_forward_and_autograd(gemma):
    X, w, dY = _norm_case()
    eps = 1e-6
    Y, r = F.rms_layernorm_fwd(X, w, eps, gemma)
    dX = F.rms_layernorm_bwd(dY, X, r, w, gemma)
    tX = torch.tensor(X, requires_grad=True)
    tw = torch.tensor(1.0 + w if gemma else w)
    tY = torch.nn.functional.rms_norm(tX, (X.shape[1],), tw, eps)
    (tY * torch.tensor(dY)).sum().backward()
    assert np.allclose(Y, tY.detach().numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariance_and_unit_mean_square():
    X, w, _ = _norm_case(seed=1)
    Y1, _ = F.rms_layernorm_fwd(X, w, 0.0)
    Y2, _ = F.rms_layernorm_fwd(X * 37.5, w, 0.0)
    assert np.allclose(Y1, Y2, rtol=1e-13, atol=1e-13)
    Y, _ = F.rms_layernorm_fwd(X, np.ones(X.shape[1]), 0.0)
    assert np.allclose(np.mean(Y * Y, axis=1), 1.0, rtol=1e-13)
    # Gemma's 1 + w at w = 0 is Llama's w = 1
    Yg, _ = F.rms_layernorm_fwd(X, np.zeros(X.shape[1]), 1e-6, gemma=True)
    Yl, _ = F.rms_layernorm_fwd(X, np.ones(X.shape[1]), 1e-6)
    assert np.array_equal(Yg, Yl)


def test_rmsnorm_central_difference():
    X, w, dY = _norm_case(m=3, d=64, seed=2)
    eps = 1e-5
    Y, r = F.rms_layernorm_fwd(X, w, eps)
    dX = F.rms_layernorm_bwd(dY, X, r, w)
    h = 1e-6
    fd = np.zeros_like(X)
    for i in range(X.shape[0]):
        for j in range(X.shape[1]):
            E = np.zeros_like(X)
            E[i, j] = h
            fd[i, j] = (np.sum(F.rms_layernorm_fwd(X + E, w, eps)[0] * dY)
                        - np.sum(F.rms_layernorm_fwd(X - E, w, eps)[0] * dY)) / (2 * h)
    assert np.max(np.abs(fd - dX)) <= 1e-7 * np.max(np.abs(dX))


# ------------------------------------------------------------------- RoPE --
def _rope_case(m=5, heads=3, hd=16, seed=3):
    g = np.random.default_rng(seed)
    return g.standard_normal((m, heads, hd)), g.integers(0, 9000, size=m)


def _rotation_matrix(theta_row, hd):
    """Block rotation on the (j, j + hd/2) pairs, formed explicitly."""
    R = np.zeros((hd, hd))
    h = hd // 2
    for j, t in enumerate(theta_row):
        c, s = np.cos(t), np.sin(t)
        R[j, j], R[j, j + h] = c, -s
        R[j + h, j], R[j + h, j + h] = s, c
    return R


def test_rope_is_a_rotation_matrix_and_backward_its_transpose():
    X, pos = _rope_case()
    base = 10000.0
    Y = F.rope_fwd(X, pos, base)
    dX = F.rope_bwd(X, pos, base)
    th = F.rope_angles(pos, X.shape[-1], base)
    for i in range(X.shape[0]):
        R = _rotation_matrix(th[i], X.shape[-1])
        assert np.allclose(Y[i], X[i] @ R.T, rtol=1e-13, atol=1e-13)
        assert np.allclose(dX[i], X[i] @ R, rtol=1e-13, atol=1e-13)


def test_rope_identity_norms_and_inverse():
    X, pos = _rope_case(seed=4)
    base = 10000.0
    assert np.allclose(F.rope_fwd(X, np.zeros_like(pos), base), X, rtol=0, atol=0)
    Y = F.rope_fwd(X, pos, base)
    h = X.shape[-1] // 2
    pair = lambda T: T[..., :h] ** 2 + T[..., h:] ** 2  # noqa: E731
    assert np.allclose(pair(Y), pair(X), rtol=1e-12)
    assert np.allclose(F.rope_bwd(Y, pos, base), X, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    g = np.random.default_rng(5)
    q, k = g.standard_normal((1, 1, 32)), g.standard_normal((1, 1, 32))
    dots = []
    for p1, p2 in ((7, 3), (104, 100), (5004, 5000)):
        a = F.rope_fwd(q, np.array([p1]), 10000.0)
        b = F.rope_fwd(k, np.array([p2]), 10000.0)
        dots.append(float(np.sum(a * b)))
    assert np.allclose(dots, dots[0], rtol=1e-9)


def test_rope_matches_torch_half_rotation_autograd():
    X, pos = _rope_case(m=4, heads=2, hd=32, seed=6)
    base = 500000.0
    dY = np.random.default_rng(7).standard_normal(X.shape)
    tX = torch.tensor(X, requires_grad=True)
    inv = 1.0 / (base ** (torch.arange(0, 32, 2, dtype=torch.float64) / 32))
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * inv[None, :]
    emb = torch.cat([ang, ang], dim=-1)[:, None, :]
    rot = torch.cat([-tX[..., 16:], tX[..., :16]], dim=-1)
    tY = tX * emb.cos() + rot * emb.sin()
    (tY * torch.tensor(dY)).sum().backward()
    assert np.allclose(F.rope_fwd(X, pos, base), tY.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(F.rope_bwd(dY, pos, base), tX.grad.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ cross entropy --
def _ce_case(m=7, V=50, seed=8, ignore_rows=(2,)):
    g = np.random.default_rng(seed)
    X = g.standard_normal((m, V)) * 3.0
    labels = g.integers(0, V, size=m)
    labels[0], labels[1] = 0, V - 1
    for i in ignore_rows:
        labels[i] = F.IGNORE
    return X, labels


@pytest.mark.parametrize("V", [50, 70001])
def test_cross_entropy_matches_torch(V):
    X, labels = _ce_case(V=V, m=5 if V > 1000 else 7)
    loss, ce, lse, n = F.cross_entropy_fwd(X, labels)
    dX = F.cross_entropy_bwd(X, labels, lse, n, dloss=0.75)
    tX = torch.tensor(X, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(tX, torch.tensor(labels), ignore_index=-100)
    (tl * 0.75).backward()
    assert abs(loss - tl.item()) <= 1e-12 * abs(tl.item())
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert n == int((labels != F.IGNORE).sum())


def test_cross_entropy_shift_invariance_and_gradient_rows():
    X, labels = _ce_case(seed=9)
    loss, ce, lse, n = F.cross_entropy_fwd(X, labels)
    shift = np.arange(X.shape[0], dtype=np.float64)[:, None] * 13.0
    loss2, ce2, lse2, _ = F.cross_entropy_fwd(X + shift, labels)
    assert np.allclose(ce, ce2, rtol=1e-12, atol=1e-12)
    dX = F.cross_entropy_bwd(X, labels, lse, n)
    assert np.allclose(dX.sum(axis=1), 0.0, atol=1e-15)
    assert not dX[2].any()                               # the ignored row
    assert np.allclose(lse, logsumexp(X, axis=1), rtol=1e-14)


def test_cross_entropy_large_logits_and_all_ignored():
    X = np.array([[1e4, 1e4 - 1.0, -1e4], [-3.0, 2e4, 0.0]])
    loss, ce, lse, n = F.cross_entropy_fwd(X, np.array([1, 2]))
    assert np.allclose(lse, logsumexp(X, axis=1), rtol=1e-15)
    assert np.isfinite(ce).all() and abs(ce[0] - (1.0 + np.log1p(np.exp(-1.0)))) < 1e-12
    loss0, ce0, lse0, n0 = F.cross_entropy_fwd(X, np.array([F.IGNORE, F.IGNORE]))
    assert loss0 == 0.0 and n0 == 0 and not ce0.any()
    assert not F.cross_entropy_bwd(X, np.array([F.IGNORE, F.IGNORE]), lse0, n0).any()
