"""Seeded synthetic inputs for the QLoRA linear layer and gated MLP.

This module draws random numbers and rounds them to the storage types; it
holds none of the method's arithmetic (no level table, no quantizer, no
products), so the GPU path and the CPU oracle can both be fed from it.

Workload shapes follow the pages' benchmark configuration (Mistral benchmark
page, configuration block: batch 4 x 2048 tokens, rank 16, alpha 16, dropout
0, random_state 3407) and model widths (Llama-7B hidden 4096 / MLP 11008,
Mistral-7B MLP 14336 with 1024-wide k/v, Gemma-7B hidden 3072 / MLP 24576
at 5 x 8192 tokens; Gemma page, "Gemma highlights").

Distributions: X ~ N(0, 1); base W ~ N(0, 0.02); LoRA A Kaiming-uniform
U(-1/sqrt(in), 1/sqrt(in)); B ~ N(0, 0.01); upstream gradient dY ~ N(0, 1)
for the tiny case and N(0, 0.01) elsewhere. The second argument of N is the
standard deviation. Draws are fp32 and rounded to bf16 by torch (round to
nearest even).

Synthetic NF4 weights (``synthetic_nf4``) stand in for quantized N(0, sigma)
weights when a workload is too large to quantize on the host: each 64-block's
absmax is the bf16 max of |N(0, sigma)| over 64 draws, and the packed code
bytes are uniform on 0..255, i.e. two independent codes uniform on 0..15 per
byte. NF4 levels are equal-probability quantiles of the normal, so codes of
quantized normal weights are close to uniform; a block of 64 uniform codes
holds an end code (0 or 15, the +-1 levels) with probability 1 - (14/16)^64,
as the block's largest weight does after quantization.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

SEED = 3407

# Stable stream index per tensor role: each tensor gets its own generator so
# that drawing one tensor never shifts another's values.
_STREAMS = {name: i for i, name in enumerate([
    "X", "dY", "W", "A", "B",
    "Wg", "Wu", "Wd", "Ag", "Bg", "Au", "Bu", "Ad", "Bd",
    "Wk", "Wv", "Ak", "Bk", "Av", "Bv", "dYk", "dYv",
])}


def rng_for(name: str, seed: int = SEED) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _STREAMS[name]])))


def to_bf16(x32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(name, shape, std, seed=SEED) -> torch.Tensor:
    g = rng_for(name, seed)
    return to_bf16(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def kaiming_uniform_bf16(name, shape, fan_in, seed=SEED) -> torch.Tensor:
    g = rng_for(name, seed)
    bound = 1.0 / math.sqrt(fan_in)
    return to_bf16(g.uniform(-bound, bound, size=shape).astype(np.float32))


def synthetic_nf4(name, n, k, std=0.02, seed=SEED):
    """NF4-format weights [n][k] without quantizing: (codes u8 [n][k/2], absmax f32 [n][k/64])."""
    assert k % 64 == 0
    g = rng_for(name, seed)
    nb = k // 64
    amax = np.empty((n, nb), dtype=np.float32)
    rows = max(1, (1 << 22) // k)
    for r0 in range(0, n, rows):
        draws = g.standard_normal((min(rows, n - r0), nb, 64), dtype=np.float32) * np.float32(std)
        amax[r0:r0 + rows] = np.abs(draws).max(axis=2)
    absmax = to_bf16(amax).to(torch.float32)
    packed = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    return torch.from_numpy(packed), absmax


@dataclasses.dataclass(frozen=True)
class LinearCfg:
    name: str
    m: int
    k: int
    n: int
    r: int
    s: float
    dy_std: float


@dataclasses.dataclass(frozen=True)
class MlpCfg:
    name: str
    m: int
    d: int
    h: int
    r: int
    s: float
    act: str
    dy_std: float = 0.01


@dataclasses.dataclass(frozen=True)
class QkvCfg:
    name: str
    m: int
    d: int
    n_q: int
    n_k: int
    n_v: int
    r: int
    s: float
    dy_std: float = 0.01


TINY_LINEAR = LinearCfg("tiny_linear", 256, 256, 512, 8, 2.0, 1.0)
QPROJ = LinearCfg("llama7b_q_proj", 8192, 4096, 4096, 16, 1.0, 0.01)
LLAMA_MLP = MlpCfg("llama7b_mlp", 8192, 4096, 11008, 16, 1.0, "swiglu")
MISTRAL_KV = LinearCfg("mistral7b_kv_proj", 8192, 4096, 1024, 16, 1.0, 0.01)
MISTRAL_MLP = MlpCfg("mistral7b_mlp", 8192, 4096, 14336, 16, 1.0, "swiglu")
GEMMA_MLP = MlpCfg("gemma7b_mlp", 40960, 3072, 24576, 16, 1.0, "geglu_tanh")
MISTRAL_QKV = QkvCfg("mistral7b_qkv", 8192, 4096, 4096, 1024, 1024, 16, 1.0)
LLAMA_QKV = QkvCfg("llama7b_qkv", 8192, 4096, 4096, 4096, 4096, 16, 1.0)


def linear_inputs(cfg: LinearCfg, dense_w: bool, seed=SEED, role=""):
    """Inputs of one QLoRA linear layer (CPU tensors).

    role "" names the plain projection; "k"/"v" draw the k/v projections of
    the Mistral slice from their own streams (X is shared). dense_w=True
    returns the bf16 base weight under "W" (for quantization by a caller);
    otherwise synthetic NF4 under "codes"/"absmax".
    """
    out = dict(
        X=normal_bf16("X", (cfg.m, cfg.k), 1.0, seed),
        A=kaiming_uniform_bf16("A" + role, (cfg.r, cfg.k), cfg.k, seed),
        B=normal_bf16("B" + role, (cfg.n, cfg.r), 0.01, seed),
        dY=normal_bf16("dY" + role, (cfg.m, cfg.n), cfg.dy_std, seed),
    )
    if dense_w:
        out["W"] = normal_bf16("W" + role, (cfg.n, cfg.k), 0.02, seed)
    else:
        out["codes"], out["absmax"] = synthetic_nf4("W" + role, cfg.n, cfg.k, 0.02, seed)
    return out


def mlp_inputs(cfg: MlpCfg, dense_w: bool, seed=SEED, m=None):
    """Inputs of one gated MLP block (CPU tensors); m overrides the token count."""
    m = cfg.m if m is None else m
    d, h, r = cfg.d, cfg.h, cfg.r
    out = dict(
        X=normal_bf16("X", (m, d), 1.0, seed),
        dY=normal_bf16("dY", (m, d), cfg.dy_std, seed),
        Ag=kaiming_uniform_bf16("Ag", (r, d), d, seed),
        Au=kaiming_uniform_bf16("Au", (r, d), d, seed),
        Ad=kaiming_uniform_bf16("Ad", (r, h), h, seed),
        Bg=normal_bf16("Bg", (h, r), 0.01, seed),
        Bu=normal_bf16("Bu", (h, r), 0.01, seed),
        Bd=normal_bf16("Bd", (d, r), 0.01, seed),
    )
    shapes = dict(Wg=(h, d), Wu=(h, d), Wd=(d, h))
    for wn, (nn, kk) in shapes.items():
        if dense_w:
            out[wn] = normal_bf16(wn, (nn, kk), 0.02, seed)
        else:
            out[wn + "_codes"], out[wn + "_absmax"] = synthetic_nf4(wn, nn, kk, 0.02, seed)
    return out


def qkv_inputs(cfg: QkvCfg, dense_w: bool, seed=SEED, m=None):
    """Inputs of the q, k, v projections of one input (CPU tensors).

    Projection q draws from the plain linear layer's streams (W, A, B, dY), k
    and v from their own (Wk, Ak, Bk, dYk; Wv, ...); X is shared. dense_w=True
    gives bf16 base weights "Wq", "Wk", "Wv"; otherwise synthetic NF4 under
    "<name>_codes" / "<name>_absmax".
    """
    m = cfg.m if m is None else m
    d, r = cfg.d, cfg.r
    out = dict(X=normal_bf16("X", (m, d), 1.0, seed))
    for p, role, n in (("q", "", cfg.n_q), ("k", "k", cfg.n_k), ("v", "v", cfg.n_v)):
        out["A" + p] = kaiming_uniform_bf16("A" + role, (r, d), d, seed)
        out["B" + p] = normal_bf16("B" + role, (n, r), 0.01, seed)
        out["dY" + p] = normal_bf16("dY" + role, (m, n), cfg.dy_std, seed)
        if dense_w:
            out["W" + p] = normal_bf16("W" + role, (n, d), 0.02, seed)
        else:
            out["W" + p + "_codes"], out["W" + p + "_absmax"] = synthetic_nf4("W" + role, n, d, 0.02, seed)
    return out
