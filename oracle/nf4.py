"""NF4 (4-bit NormalFloat) reference: level table, quantizer, packing, dequant.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the pages fix: the frozen base weights of every projection (q, k, v, o,
gate, up, down) are stored as "QLoRA nf4" (Mistral benchmark page,
benchmark configuration block); bitsandbytes' 4-bit format is what is
dequantized, and dequantizing straight to bfloat16 instead of float16 saved a
copy ("Introducing Unsloth" page, Pro feature list; Mistral benchmark page,
breakdown item 2 "Bitsandbytes bfloat16"). The pages print no level values,
no block size and no bit layout; the readings below fill those gaps and are
each listed in the design notes.

Readings taken where the pages are silent
-----------------------------------------
* Level table: the asymmetric normal-quantile construction of the QLoRA
  paper (linked from the Show HN thread): 8 positive levels at the standard
  normal quantiles of 8 evenly spaced probabilities in (1/2, delta], 7 negative
  levels mirrored from 7 evenly spaced probabilities in (1/2, delta], an exact
  zero, all divided by Phi^-1(delta) so the ends are exactly -1 and +1.
  Phi^-1(1) is infinite, so the outermost level cannot sit at probability 1;
  it sits at the centre of the outermost equal-probability bin instead. The
  positive half is cut as if into 16 bins (centre 1 - 1/32) and the negative
  half as if into 15 (centre 1 - 1/30), and both halves share one outermost
  probability, so delta is the mean of the two centres:
  delta = ((1 - 1/30) + (1 - 1/32)) / 2 = 0.96770833... This is the offset of
  the QLoRA paper's construction, so codes from a standard NF4 quantizer
  decode to the same levels. Values are formed in fp64 and rounded once to
  fp32.
* Blocks: 64 consecutive weights along a row share one fp32 absmax.
* Code choice: the level nearest to w/absmax (fp64), ties to the lower code.
* All-zero block: absmax 0, every code 7 (the exact-zero level).
* Packing: element 2j of a row goes to the HIGH nibble of byte j, element
  2j+1 to the LOW nibble.
* Dequant: W = bf16_rne(fp32_rne(L[c] * absmax)). The product is exact in
  fp64 (24 x 24 significant bits), then rounded to fp32, then to bf16; the
  order of the two roundings is part of the contract.
* Double quantization (optional): the absmax array itself stored as 8-bit
  codes with one fp32 scale and one fp32 offset per 256 values; see
  absmax_dq_quantize. A double-quantized weight dequantizes with the
  reconstructed absmax in place of the stored one.
"""
from __future__ import annotations

import numpy as np
from scipy.stats import norm

NF4_DELTA = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
BLOCK = 64


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending (index 7 is exactly 0)."""
    d = NF4_DELTA
    pos = [norm.ppf(0.5 + (d - 0.5) * j / 8.0) for j in range(1, 9)]
    neg = [-norm.ppf(0.5 + (d - 0.5) * j / 7.0) for j in range(1, 8)]
    top = norm.ppf(d)
    levels = np.array(sorted(neg + [0.0] + pos), dtype=np.float64) / top
    # The ends are exactly +-1 by construction; force the exact value in case
    # ppf(d)/ppf(d) were not evaluated as the same number.
    levels[0], levels[7], levels[15] = -1.0, 0.0, 1.0
    return levels


def nf4_levels() -> np.ndarray:
    """The level table as stored and used: fp32, 16 entries."""
    return nf4_levels_f64().astype(np.float32)


# ---------------------------------------------------------------- bf16 ----
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = np.where(nan, ((u >> 16) & 0x8000) | 0x7FC0, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ packing -----
def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[N][K] codes (0..15) -> [N][K/2] bytes; element 2j -> high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    hi = codes[..., 0::2]
    lo = codes[..., 1::2]
    return ((hi << 4) | lo).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[N][K/2] bytes -> [N][K] codes; inverse of pack_codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed >> 4
    out[..., 1::2] = packed & 0x0F
    return out


# ----------------------------------------------------------- quantize -----
def quantize(w_bf16_bits: np.ndarray, chunk_rows: int = 256):
    """Quantize bf16 weights [N][K] (K % 64 == 0) to NF4.

    Returns (packed codes uint8 [N][K/2], absmax float32 [N][K/64]).
    Follows the readings in the module docstring: per 64-block absmax,
    x = w/absmax in fp64, nearest level with ties to the lower code.
    """
    w_bits = np.asarray(w_bf16_bits, dtype=np.uint16)
    n, k = w_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 64")
    levels = nf4_levels().astype(np.float64)
    codes = np.empty((n, k), dtype=np.uint8)
    absmax = np.empty((n, k // BLOCK), dtype=np.float32)
    for r0 in range(0, n, chunk_rows):
        w = bf16_bits_to_f64(w_bits[r0:r0 + chunk_rows])
        blocks = w.reshape(w.shape[0], k // BLOCK, BLOCK)
        amax = np.abs(blocks).max(axis=2)
        absmax[r0:r0 + chunk_rows] = amax  # exact: amax is a bf16 value
        safe = np.where(amax == 0.0, 1.0, amax)
        x = blocks / safe[..., None]
        x = np.where(amax[..., None] == 0.0, 0.0, x)
        dist = np.abs(x[..., None] - levels)            # [..., 64, 16]
        c = np.argmin(dist, axis=-1)                     # first minimum = lower code
        codes[r0:r0 + chunk_rows] = c.reshape(w.shape[0], k).astype(np.uint8)
    return pack_codes(codes), absmax


# ------------------------------------------------------------ dequant -----
def dequant_bf16_bits(packed: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """NF4 -> bf16 bit patterns [N][K]: bf16_rne(fp32_rne(L[c] * absmax))."""
    codes = unpack_codes(packed)
    n, k = codes.shape
    levels = nf4_levels().astype(np.float64)
    scale = np.repeat(np.asarray(absmax, dtype=np.float32).astype(np.float64), BLOCK, axis=1)
    assert scale.shape == (n, k)
    exact = levels[codes] * scale                        # exact in fp64
    as_f32 = exact.astype(np.float32)                    # first rounding (RNE)
    return f32_to_bf16_bits(as_f32)                      # second rounding (RNE)


def dequant_f64(packed: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """Dequantized weights as fp64 values (exactly the bf16 weights)."""
    return bf16_bits_to_f64(dequant_bf16_bits(packed, absmax))


# ------------------------------------------------ double quantization -----
# The pages link the QLoRA paper for the 4-bit format but print no
# second-level format. Reading (listed in the design notes): the first-level
# constants (the fp32 absmax array, flattened row-major) are quantized again
# in groups of DQ_GROUP = 256 consecutive values (the last group may be
# shorter) with the paper's own absmax scheme, applied to the constants after
# subtracting their mean (they are all >= 0, so the mean centres them):
#   offset  mu = fp32( (a_0 + a_1 + ... + a_{n-1}) / n )   fp64 sum, index order
#   scale   c  = fp32( max_i |a_i - mu| / 127 )             fp64
#   code    q_i = clamp(rne((a_i - mu) / c), -127, 127)    int8; all 0 if c == 0
#   value   a'_i = fp32( fp32(q_i * c) + mu )               two fp32 roundings
# Storage: 1 byte per 64-weight block plus 8 bytes per 256 blocks.
DQ_GROUP = 256


def absmax_dq_quantize(absmax):
    """fp32 absmax (any shape, read flattened) -> (q int8 [n], scale f32 [g], offset f32 [g])."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    n = a.size
    ng = (n + DQ_GROUP - 1) // DQ_GROUP
    q = np.zeros(n, dtype=np.int8)
    scale = np.zeros(ng, dtype=np.float32)
    offset = np.zeros(ng, dtype=np.float32)
    for j in range(ng):
        grp = a[j * DQ_GROUP:(j + 1) * DQ_GROUP].astype(np.float64)
        total = 0.0
        for v in grp:                      # plain sequential fp64 sum
            total += float(v)
        mu = np.float32(total / grp.size)
        dev = np.abs(grp - np.float64(mu))
        c = np.float32(dev.max() / 127.0)
        offset[j], scale[j] = mu, c
        if c > 0:
            x = (grp - np.float64(mu)) / np.float64(c)
            q[j * DQ_GROUP:j * DQ_GROUP + grp.size] = np.clip(np.rint(x), -127, 127).astype(np.int8)
    return q, scale, offset


def absmax_dq_dequant(q, scale, offset):
    """Reconstructed fp32 absmax [n] = fp32(fp32(q * c) + mu) per group."""
    q = np.asarray(q, dtype=np.int8).reshape(-1)
    g = np.arange(q.size) // DQ_GROUP
    c = np.asarray(scale, dtype=np.float32)[g].astype(np.float64)
    mu = np.asarray(offset, dtype=np.float32)[g].astype(np.float64)
    prod = (q.astype(np.float64) * c).astype(np.float32)             # exact product, one rounding
    return (prod.astype(np.float64) + mu).astype(np.float32)        # sum, one rounding
