"""fp64 reference of the QLoRA linear layer and gated MLP, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

All arrays are fp64 holding exactly the bf16 input values (and the bf16
dequantized base weights). Row-major, tokens along axis 0. LoRA factors use
the orientation A [r][in], B [out][r]; the Mistral benchmark page writes the
same products with the transposed factors (its A is our A^T, its B our B^T).

Linear layer (Mistral benchmark page, items 10-11 "manual autograd"; Reddit
talk summary, "fused LoRA" and "chained matrix multiplication"):
    forward   U  = X A^T                  (rank-r product first)
              Y  = X W^T + s U B^T
    backward  T  = dY B
              dX = dY W + s T A
              dA = s T^T X
              dB = s dY^T U
There is no gradient for the frozen base W and no bias; LoRA dropout is 0
(benchmark configuration block), so the LoRA branch sees X itself.

Gated MLP (Mistral benchmark page, breakdown row "Manual Autograd MLP";
Gemma page, section "GeGLU vs SwiGLU activation"):
    g = QL_gate(X), u = QL_up(X), H = act(g) * u, Y = QL_down(H)
    dH from the down layer's backward; dg = dH * u * act'(g); du = dH * act(g);
    dX = dX_gate + dX_up.
act is SwiGLU's silu or the tanh form of GELU (GeGLU). The exact-erf GELU is
not used (reading: Gemma's GeGLU is the tanh approximation).
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_C = 0.044715


# ------------------------------------------------------------ activations --
def sigmoid(x: np.ndarray) -> np.ndarray:
    """Numerically stable logistic function in fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(g):
    return g * sigmoid(g)


def silu_grad(g):
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def gelu_tanh(g):
    z = SQRT_2_OVER_PI * (g + GELU_C * g ** 3)
    return 0.5 * g * (1.0 + np.tanh(z))


def gelu_tanh_grad(g):
    z = SQRT_2_OVER_PI * (g + GELU_C * g ** 3)
    t = np.tanh(z)
    dz = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_C * g ** 2)
    return 0.5 * (1.0 + t) + 0.5 * g * (1.0 - t * t) * dz


ACTS = {
    "swiglu": (silu, silu_grad),
    "geglu_tanh": (gelu_tanh, gelu_tanh_grad),
}


# ----------------------------------------------------------- linear layer --
def linear_fwd(X, W, A, B, s):
    """Returns (Y, U) with U = X A^T saved for the backward."""
    U = X @ A.T
    Y = X @ W.T + s * (U @ B.T)
    return Y, U


def linear_bwd(dY, X, U, W, A, B, s):
    """Returns (dX, dA, dB, T) for the frozen-base LoRA linear layer."""
    T = dY @ B
    dX = dY @ W + s * (T @ A)
    dA = s * (T.T @ X)
    dB = s * (dY.T @ U)
    return dX, dA, dB, T


# ------------------------------------------------------------- gated MLP --
def mlp_fwd(X, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act="swiglu"):
    """Returns (Y, saved) where saved holds g, u, Ug, Uu, Ud (H is not saved)."""
    f, _ = ACTS[act]
    g, Ug = linear_fwd(X, Wg, Ag, Bg, s)
    u, Uu = linear_fwd(X, Wu, Au, Bu, s)
    H = f(g) * u
    Y, Ud = linear_fwd(H, Wd, Ad, Bd, s)
    return Y, dict(g=g, u=u, Ug=Ug, Uu=Uu, Ud=Ud)


def mlp_bwd(dY, X, saved, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act="swiglu"):
    """Manual backward of the gated MLP; H is recomputed from g and u.

    Returns a dict with dX, dAg, dBg, dAu, dBu, dAd, dBd.
    """
    f, fprime = ACTS[act]
    g, u = saved["g"], saved["u"]
    a = f(g)
    H = a * u                                   # recomputed, not stored
    dH, dAd, dBd, _ = linear_bwd(dY, H, saved["Ud"], Wd, Ad, Bd, s)
    dg = dH * u * fprime(g)
    du = dH * a
    dXg, dAg, dBg, _ = linear_bwd(dg, X, saved["Ug"], Wg, Ag, Bg, s)
    dXu, dAu, dBu, _ = linear_bwd(du, X, saved["Uu"], Wu, Au, Bu, s)
    return dict(dX=dXg + dXu, dAg=dAg, dBg=dBg, dAu=dAu, dBu=dBu, dAd=dAd, dBd=dBd)


def mlp_lora_grads(X, dY, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act="swiglu"):
    """The six LoRA weight gradients of the gated MLP alone.

    The same definitions as mlp_fwd followed by mlp_bwd, with the two
    products that feed only Y (H Wd^T) and dX (dg Wg, du Wu) left out. Every
    gradient is a sum over tokens, so a long batch may be passed in row
    blocks and the block results added. Returns dAg, dBg, dAu, dBu, dAd, dBd.
    """
    f, fprime = ACTS[act]
    Ug, Uu = X @ Ag.T, X @ Au.T
    g = X @ Wg.T + s * (Ug @ Bg.T)
    u = X @ Wu.T + s * (Uu @ Bu.T)
    a = f(g)
    H = a * u
    Ud = H @ Ad.T
    Td = dY @ Bd
    dH = dY @ Wd + s * (Td @ Ad)
    dg = dH * u * fprime(g)
    du = dH * a
    Tg, Tu = dg @ Bg, du @ Bu
    return dict(dAg=s * (Tg.T @ X), dBg=s * (dg.T @ Ug), dAu=s * (Tu.T @ X), dBu=s * (du.T @ Uu),
                dAd=s * (Td.T @ H), dBd=s * (dY.T @ Ud))


def mlp_rows(rows, X, dY, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act="swiglu"):
    """Per-token outputs for a subset of rows: Y, g, u, Ug, Uu, Ud and dX.

    Every one of these depends only on its own token (the LoRA weight
    gradients are the only outputs that sum over tokens), so a sample of rows
    can be checked at full size without the full-size computation.
    """
    Xs, dYs = X[rows], dY[rows]
    Y, sv = mlp_fwd(Xs, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act)
    gr = mlp_bwd(dYs, Xs, sv, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, s, act)
    return dict(Y=Y, dX=gr["dX"], **sv)


# ---------------------------------------- q, k, v on one shared input --
def qkv_fwd(X, Ws, As, Bs, s):
    """The q, k, v projections of one input (Mistral benchmark page, breakdown
    row "Manual Autograd QKV"; Show HN thread, the author's list of savings).

    Ws, As, Bs: the three base weights W_p [N_p][d] and LoRA factors A_p
    [r][d], B_p [N_p][r]. Each output is the linear layer's Y_p; returns
    (list of Y_p, list of U_p = X A_p^T).
    """
    outs = [linear_fwd(X, W, A, B, s) for W, A, B in zip(Ws, As, Bs)]
    return [o[0] for o in outs], [o[1] for o in outs]


def qkv_bwd(dYs, X, Us, Ws, As, Bs, s):
    """Manual backward of the three projections: X feeds all three, so its
    gradient is the sum dX = sum_p (dY_p W_p + s T_p A_p) with T_p = dY_p B_p;
    each projection has its own dA_p = s T_p^T X and dB_p = s dY_p^T U_p.

    Returns (dX, list of dA_p, list of dB_p).
    """
    dX = np.zeros_like(X)
    dA, dB = [], []
    for dY, U, W, A, B in zip(dYs, Us, Ws, As, Bs):
        dXp, dAp, dBp, _ = linear_bwd(dY, X, U, W, A, B, s)
        dX = dX + dXp
        dA.append(dAp)
        dB.append(dBp)
    return dX, dA, dB


def qkv_algorithmic_flops(m, d, ns, r):
    """FLOPs for the q, k, v forward + backward: each projection counts as one
    linear layer (the shared input adds no work)."""
    return sum(linear_algorithmic_flops(m, d, n, r) for n in ns)


# ------------------------------------------------- chained-matmul FLOPs --
def chain_macs(shapes, order):
    """Multiply-accumulates of a matrix chain evaluated in a given bracketing.

    shapes: list of (rows, cols) of the factors; order: nested tuple of factor
    indices, e.g. ((0, 1), 2) or (0, (1, 2)). Returns (macs, result_shape).
    A (p x q) times (q x t) product costs p*q*t multiply-accumulates.
    """
    if isinstance(order, int):
        return 0, shapes[order]
    left, right = order
    ml, (p, q) = chain_macs(shapes, left)
    mr, (q2, t) = chain_macs(shapes, right)
    if q != q2:
        raise ValueError("inner dimensions differ")
    return ml + mr + p * q * t, (p, t)


def lora_grad_bracketing_ratio(m, d, h, r):
    """Slow / fast cost of X^T dW B^T (Mistral benchmark page, items 10-11).

    X^T is (d, m), the upstream gradient dW is (m, h), B^T is (h, r) in the
    page's naming. Slow: (X^T dW) B^T; fast: X^T (dW B^T).
    """
    shapes = [(d, m), (m, h), (h, r)]
    slow, _ = chain_macs(shapes, ((0, 1), 2))
    fast, _ = chain_macs(shapes, (0, (1, 2)))
    return slow / fast, slow, fast


def mlp_algorithmic_flops(m, d, h, r):
    """FLOPs (2 per MAC) the method must do for one MLP forward + backward.

    Three base products forward and three backward (no base weight gradient),
    plus 2*m*r*(in+out) per LoRA projection forward and twice that backward.
    Recomputation, dequant and elementwise work are not counted.
    """
    base = 6 * 2 * m * d * h
    lora_proj = 2 * m * r * (d + h)
    return base + 3 * lora_proj * 3


def linear_algorithmic_flops(m, k, n, r):
    """FLOPs for one QLoRA linear forward + backward (same counting rules)."""
    return 2 * 2 * m * k * n + 3 * 2 * m * r * (k + n)
