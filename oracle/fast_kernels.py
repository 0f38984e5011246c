"""fp64 reference of the pages' other hand-derived training kernels: RMS
layernorm, RoPE embeddings and the cross-entropy loss, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

RMS layernorm (Mistral benchmark page, breakdown item 8 "Fast RMS Layernorm",
derivative by the chain rule; Gemma page, "+1 to RMS LayerNorm": Llama and
Mistral scale by w, Gemma by 1 + w). Per row i of X [m][d]:
    r_i  = 1 / sqrt(mean_j x_ij^2 + eps)
    y_ij = x_ij * r_i * w'_j,     w' = w (Llama, Mistral) or 1 + w (Gemma)
Backward with the norm weight frozen (LoRA trains the adapters only), g = dy * w':
    dx_ij = r_i * (g_ij - x_ij * r_i^2 * mean_k(g_ik * x_ik))

RoPE (same page, breakdown item 7 "Fast RoPE Embeddings": RoPE is a product
with a rotation matrix R, so its derivative is R^T; Reddit talk summary: the
derivative is the same with the sign reversed). A head vector of length hd is
split into halves (a, b); with theta_j = pos * base^(-2j/hd), j < hd/2:
    y = (a cos theta - b sin theta,  b cos theta + a sin theta)
    dx = R^T dy = (da cos theta + db sin theta,  db cos theta - da sin theta)
The angle is formed from the integer position in fp64: the Gemma page reports
RoPE losing precision at long context when positions pass through bfloat16.

Cross entropy (same page, breakdown item 9 "Fast Cross Entropy Loss"; Reddit
talk summary, "chunked cross entropy"; Gemma page, "256K vocabulary"). Per row
i of logits X [m][V] with label y_i (IGNORE = -100 marks a row without a
target):
    CE_i  = logsumexp(x_i) - x_i[y_i]    (0 for an ignored row)
    loss  = (1/n) sum_i CE_i,  n = number of rows with a target
    dx_i  = (softmax(x_i) - onehot(y_i)) * dloss / n   (0 for an ignored row)
The derivative of logsumexp is softmax, as the page notes. Chunking the
vocabulary (any size, Gemma's 256K included) changes how the row is walked,
not the value. Reading where the pages are silent: n = 0 gives loss 0 and a
zero gradient.
"""
from __future__ import annotations

import numpy as np

IGNORE = -100


# ----------------------------------------------------------- RMS layernorm --
def _wprime(w, gemma):
    w = np.asarray(w, dtype=np.float64)
    return 1.0 + w if gemma else w


def rms_layernorm_fwd(X, w, eps, gemma=False):
    """Returns (Y [m][d], r [m]) with r the inverse root-mean-square per row."""
    X = np.asarray(X, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(X * X, axis=1) + eps)
    return X * r[:, None] * _wprime(w, gemma)[None, :], r


def rms_layernorm_bwd(dY, X, r, w, gemma=False):
    """dX of the RMS layernorm for a frozen weight."""
    X = np.asarray(X, dtype=np.float64)
    g = np.asarray(dY, dtype=np.float64) * _wprime(w, gemma)[None, :]
    dot = np.mean(g * X, axis=1)
    return r[:, None] * (g - X * (r * r * dot)[:, None])


# ------------------------------------------------------------------- RoPE --
def rope_angles(pos, hd, base):
    """theta [m][hd/2] in fp64 from integer positions."""
    j = np.arange(hd // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * j / hd)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def _rotate(X, theta, sign):
    X = np.asarray(X, dtype=np.float64)
    hd = X.shape[-1]
    a, b = X[..., : hd // 2], X[..., hd // 2:]
    c = np.cos(theta)[:, None, :]
    s = sign * np.sin(theta)[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_fwd(X, pos, base):
    """X [m][heads][hd] -> rotated by the angles of each row's position."""
    return _rotate(X, rope_angles(pos, X.shape[-1], base), 1.0)


def rope_bwd(dY, pos, base):
    """dX = R^T dY: the rotation by the opposite angle."""
    return _rotate(dY, rope_angles(pos, dY.shape[-1], base), -1.0)


# ------------------------------------------------------------ cross entropy --
def logsumexp_rows(X):
    X = np.asarray(X, dtype=np.float64)
    mx = X.max(axis=1)
    return mx + np.log(np.sum(np.exp(X - mx[:, None]), axis=1))


def cross_entropy_fwd(X, labels):
    """Returns (loss, ce_rows [m], lse [m], n) for logits X [m][V]."""
    X = np.asarray(X, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    lse = logsumexp_rows(X)
    valid = labels != IGNORE
    ce = np.zeros(X.shape[0])
    rows = np.nonzero(valid)[0]
    ce[rows] = lse[rows] - X[rows, labels[rows]]
    n = int(valid.sum())
    loss = float(ce.sum() / n) if n else 0.0
    return loss, ce, lse, n


def cross_entropy_bwd(X, labels, lse, n, dloss=1.0):
    """dX [m][V] of the mean loss, scaled by the upstream dloss."""
    X = np.asarray(X, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    dX = np.zeros_like(X)
    if n == 0:
        return dX
    valid = labels != IGNORE
    rows = np.nonzero(valid)[0]
    P = np.exp(X[rows] - lse[rows, None])
    P[np.arange(len(rows)), labels[rows]] -= 1.0
    dX[rows] = P * (dloss / n)
    return dX
