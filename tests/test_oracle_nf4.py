"""Pins of the NF4 oracle (oracle/nf4.py) against facts fixed outside it.

- level table: invariants of the construction, an independent inverse-normal
  (bisection on math.erfc) and the equal-probability spacing it encodes;
- bf16 rounding: torch's own float32 -> bfloat16 conversion;
- dequant: torch's fp32 multiply followed by torch's bf16 cast (the
  two-rounding contract as computed by a different implementation);
- quantize: exact round trips, monotonicity, brute force on one block;
- packing: a hand-written fixture.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def _phi_inv(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_table_invariants():
    L = nf4.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert L[7] == 0.0 and not np.signbit(L[7])
    assert L[0] == -1.0 and L[15] == 1.0
    assert np.all(np.diff(L) > 0)
    # 7 strictly negative, 8 strictly positive levels (asymmetric table)
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8


def test_table_matches_independent_inverse_normal():
    L = nf4.nf4_levels()
    d = nf4.NF4_DELTA
    top = _phi_inv(d)
    want = [-_phi_inv(0.5 + (d - 0.5) * j / 7) / top for j in range(7, 0, -1)]
    want += [0.0] + [_phi_inv(0.5 + (d - 0.5) * j / 8) / top for j in range(1, 9)]
    got = L.astype(np.float64)
    ulp = np.spacing(np.abs(L)).astype(np.float64)
    assert np.all(np.abs(got - np.array(want)) <= ulp + 1e-300)


def test_positive_levels_are_equal_probability_spaced():
    L = nf4.nf4_levels_f64()
    top = _phi_inv(nf4.NF4_DELTA)
    probs = [_phi(L[8 + j] * top) for j in range(8)]
    steps = np.diff([0.5] + probs)
    assert np.allclose(steps, steps[0], rtol=0, atol=1e-12)
    negs = [_phi(-L[6 - j] * top) for j in range(7)]
    nsteps = np.diff([0.5] + negs)
    assert np.allclose(nsteps, nsteps[0], rtol=0, atol=1e-12)


def test_table_matches_stored_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "nf4_levels.txt")) if not ln.startswith("#")]
    bits = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
    assert np.array_equal(nf4.nf4_levels().view(np.uint32), bits)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    x = g.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 200000)
    u = x.view(np.uint32)
    # force exact ties (low 16 bits = 0x8000) on a quarter of the values, both parities
    u[::4] = (u[::4] & 0xFFFF0000) | 0x8000
    x = u.view(np.float32)
    x = x[np.isfinite(x)]   # NaN payload handling is not part of the contract
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.f32_to_bf16_bits(x), want)


def _bf16_sweep():
    # every positive finite bf16 value: the 127 subnormals and all 254 normal
    # binades (bit patterns 0x0001 .. 0x7F7F)
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32)


def _single_rounding_to_bf16(x):
    # one round-to-nearest-even of an fp64 value to the bf16 grid: 8
    # significant bits for normal results, a fixed 2^-133 quantum below 2^-126
    m, e = np.frexp(x)
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    return np.round(x / q) * q


def test_dequant_equals_torch_two_roundings_all_codes():
    absmax = _bf16_sweep()
    n = absmax.size
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, 4))       # [n][64]
    packed = nf4.pack_codes(codes)
    got = nf4.dequant_bf16_bits(packed, absmax[:, None])
    L = torch.from_numpy(nf4.nf4_levels())
    prod = L[torch.from_numpy(codes.astype(np.int64))] * torch.from_numpy(absmax)[:, None]  # fp32 RNE
    want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # With this table a single rounding of the exact product (at most 32
    # significant bits: 24 from the level, 8 from the bf16 absmax) never lands
    # differently from the two-step rounding, over every finite positive bf16
    # absmax including subnormal products: the contract holds whichever order
    # an implementation takes.
    exact = nf4.nf4_levels().astype(np.float64)[codes] * absmax.astype(np.float64)[:, None]
    single = _single_rounding_to_bf16(exact)
    twice = nf4.bf16_bits_to_f64(want)
    assert np.array_equal(single, twice)


def test_single_rounding_helper_on_known_values():
    # the helper used above, on hand-checked values: a tie to even in the
    # normal range (1 + 2^-8 lies halfway between 1 and 1 + 2^-7), one just
    # past the tie, and the subnormal grid (2^-134 is a tie between 0 and
    # 2^-133; 3 * 2^-134 rounds to 2 * 2^-133)
    got = _single_rounding_to_bf16(np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30,
                                             2.0 ** -134, 3 * 2.0 ** -134]))
    assert list(got) == [1.0, 1 + 2.0 ** -7, 0.0, 2 * 2.0 ** -133]


def test_zero_code_and_absmax_roundtrip():
    g = np.random.default_rng(2)
    w = nf4.f32_to_bf16_bits(g.standard_normal((32, 256)).astype(np.float32) * np.float32(0.02))
    packed, absmax = nf4.quantize(w)
    deq = nf4.dequant_bf16_bits(packed, absmax)
    wv = nf4.bf16_bits_to_f64(w).reshape(32, 4, 64)
    dv = nf4.bf16_bits_to_f64(deq).reshape(32, 4, 64)
    idx = np.abs(wv).argmax(axis=2)
    assert np.array_equal(np.take_along_axis(dv, idx[..., None], 2), np.take_along_axis(wv, idx[..., None], 2))
    codes = nf4.unpack_codes(packed)
    zero = nf4.bf16_bits_to_f64(deq)[codes == 7]
    assert np.all(zero == 0.0) and not np.any(np.signbit(zero))


def test_all_zero_block():
    w = np.zeros((2, 128), dtype=np.uint16)
    w[1, 64:] = nf4.f32_to_bf16_bits(np.linspace(-1, 1, 64).astype(np.float32))
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack_codes(packed)
    assert absmax[0, 0] == 0 and absmax[0, 1] == 0 and absmax[1, 0] == 0 and absmax[1, 1] == 1.0
    assert np.all(codes[0] == 7) and np.all(codes[1, :64] == 7)
    assert np.all(nf4.dequant_bf16_bits(packed, absmax)[0] == 0)


def test_quantize_dequant_roundtrip_of_codes():
    g = np.random.default_rng(3)
    codes = g.integers(0, 16, (16, 512)).astype(np.uint8)
    codes[:, ::64] = 15                     # every block holds its +1 element
    absmax = nf4.bf16_bits_to_f64(nf4.f32_to_bf16_bits(
        np.abs(g.standard_normal((16, 8))).astype(np.float32) * np.float32(0.05) + np.float32(0.01))).astype(np.float32)
    deq = nf4.dequant_bf16_bits(nf4.pack_codes(codes), absmax)
    packed2, absmax2 = nf4.quantize(deq)
    assert np.array_equal(absmax2, absmax)
    assert np.array_equal(nf4.unpack_codes(packed2), codes)


def test_quantize_monotone_and_brute_force_one_block():
    L = [float(v) for v in nf4.nf4_levels()]
    xs = np.linspace(-1.0, 1.0, 64).astype(np.float32)
    w = nf4.f32_to_bf16_bits(xs * np.float32(0.75))[None, :]
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack_codes(packed)[0]
    assert np.all(np.diff(codes.astype(int)) >= 0)
    vals = nf4.bf16_bits_to_f64(w)[0]
    amax = max(abs(v) for v in vals)
    for v, c in zip(vals, codes):
        x = v / amax
        best = min(range(16), key=lambda i: (abs(x - L[i]), i))
        assert c == best


def test_packing_fixture():
    lines = [ln for ln in open(os.path.join(GOLDEN, "nf4_pack_example.txt")) if not ln.startswith("#")]
    codes = np.array([int(t) for t in lines[0].split()], dtype=np.uint8)[None, :]
    want = np.array([int(t, 16) for t in lines[1].split()], dtype=np.uint8)[None, :]
    assert np.array_equal(nf4.pack_codes(codes), want)
    assert np.array_equal(nf4.unpack_codes(want), codes)


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        nf4.quantize(np.zeros((1, 96), dtype=np.uint16))


def test_quantize_is_exact_nearest_level_for_every_significand_pair():
    """For every pair of bf16 significands (absmax in [1, 2); weight magnitudes
    in the 12 binades at and below it, both signs; zeros), the quantizer's fp64
    nearest-level search gives the code of exact rational arithmetic: the number
    of level midpoints strictly below w / absmax (a tie goes to the lower code).
    Exact comparison in int64: with absmax = m_a / 128, w = +-m_w 2^e / 128 and a
    midpoint mu = M / 2^28, w / absmax > mu  <=>  m_w 2^(e+39) > M m_a 2^11.
    (No quotient of two bf16 values lands exactly on a midpoint of this table,
    so the tie rule never acts on bf16 weights.)"""
    L = nf4.nf4_levels().astype(np.float64)
    mids = (L[:-1] + L[1:]) / 2
    M = np.array([int(v * 2 ** 28) for v in mids], dtype=np.int64)
    assert np.array_equal(M.astype(np.float64) / 2 ** 28, mids)       # midpoints exactly representable
    mw = np.arange(128, 256, dtype=np.int64)
    rows, want = [], []
    for ma in range(128, 256):
        a = ma / 128.0
        vals, ints = [], []
        for e in range(0, -12, -1):
            for m in mw:
                if e == 0 and m > ma:
                    continue
                for sgn in (1, -1):
                    vals.append(sgn * m * 2.0 ** e / 128.0)
                    ints.append(sgn * int(m) << (e + 39))
        vals += [0.0, -0.0]
        ints += [0, 0]
        ints = np.array(ints, dtype=np.int64)
        codes = (ints[:, None] > (M * ma * 2 ** 11)[None, :]).sum(axis=1)
        for s in range(0, len(vals), 63):                       # block: absmax first, then 63 weights
            chunk = vals[s:s + 63]
            pad = 63 - len(chunk)
            rows.append([a] + chunk + [0.0] * pad)
            want.append([15] + codes[s:s + 63].tolist() + [7] * pad)
    w = np.array(rows, dtype=np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(nf4.bf16_bits_to_f64(bits), w.astype(np.float64))   # all exact in bf16
    packed, absmax = nf4.quantize(bits)
    assert np.array_equal(absmax[:, 0], w[:, 0])
    assert np.array_equal(nf4.unpack_codes(packed), np.array(want, dtype=np.uint8))


# ------------------------------------------------ double quantization -----
def test_dq_exact_at_grid_points():
    """A group built on the grid (mean mu, step c, codes symmetric about 0 with
    extremes +-127) is recovered exactly: the same mean, step, codes and
    values. mu and c are powers of two apart, so every mu + k c is an fp32
    value and the mean of the group is mu exactly."""
    g = np.random.default_rng(7)
    k = g.integers(-126, 127, 127).astype(np.int64)
    codes = np.concatenate([k, -k, [127, -127]])            # 256 codes, sum 0
    g.shuffle(codes)
    mu, c = np.float32(0.375), np.float32(2.0 ** -12)
    a = (mu + codes * np.float64(c)).astype(np.float32)
    assert np.array_equal(a.astype(np.float64), 0.375 + codes * 2.0 ** -12)
    q, scale, offset = nf4.absmax_dq_quantize(a)
    assert offset[0] == mu and scale[0] == c
    assert np.array_equal(q.astype(np.int64), codes)
    assert np.array_equal(nf4.absmax_dq_dequant(q, scale, offset), a)


def test_dq_round_trip_error_bound_and_ragged_groups():
    """Random absmax of N(0, 0.02) weight blocks over 1000 blocks (three full
    groups and a ragged one of 232): every reconstructed value lies within
    half a step of its group (plus the two fp32 roundings), codes stay in
    [-127, 127], the extreme deviation of each group takes code +-127, and
    mean and step agree with numpy's mean and max to 1 fp32 ulp."""
    g = np.random.default_rng(8)
    w = np.abs(g.standard_normal((1000, 64))) * 0.02
    a = nf4.bf16_bits_to_f64(nf4.f32_to_bf16_bits(w.max(axis=1).astype(np.float32))).astype(np.float32)
    q, scale, offset = nf4.absmax_dq_quantize(a)
    assert q.shape == (1000,) and scale.shape == (4,) and offset.shape == (4,)
    back = nf4.absmax_dq_dequant(q, scale, offset)
    for j in range(4):
        grp = a[j * 256:(j + 1) * 256].astype(np.float64)
        mu_ref = np.float32(np.mean(grp))
        assert abs(float(offset[j]) - float(mu_ref)) <= float(np.spacing(mu_ref))
        c_ref = np.float32(np.max(np.abs(grp - np.float64(offset[j]))) / 127)
        assert scale[j] == c_ref
        qq = q[j * 256:(j + 1) * 256].astype(np.int64)
        assert qq.min() >= -127 and qq.max() <= 127 and np.abs(qq).max() == 127
        err = np.abs(back[j * 256:(j + 1) * 256].astype(np.float64) - grp)
        bound = 0.5 * float(scale[j]) + 2 * float(np.spacing(np.float32(grp.max())))
        assert err.max() <= bound
    # the code is the nearest integer step (brute force on the first group)
    mu, c = float(offset[0]), float(scale[0])
    for i in range(0, 256, 17):
        dist = [abs(float(a[i]) - mu - t * c) for t in range(-127, 128)]
        assert abs(float(a[i]) - mu - int(q[i]) * c) <= min(dist) + 1e-15


def test_dq_zero_and_constant_groups():
    a = np.zeros(300, dtype=np.float32)
    a[256:] = np.float32(0.0625)                              # ragged group: all equal
    q, scale, offset = nf4.absmax_dq_quantize(a)
    assert np.all(q == 0) and scale[0] == 0 and offset[0] == 0 and scale[1] == 0
    assert offset[1] == np.float32(0.0625)
    back = nf4.absmax_dq_dequant(q, scale, offset)
    assert np.array_equal(back, a) and not np.any(np.signbit(back))


def test_dq_weight_dequant_uses_reconstructed_absmax():
    """A double-quantized weight dequantizes exactly as the NF4 weight whose
    absmax is the reconstructed array (the second level only replaces the
    constants)."""
    g = np.random.default_rng(9)
    w = nf4.f32_to_bf16_bits(g.standard_normal((8, 512)).astype(np.float32) * np.float32(0.02))
    packed, absmax = nf4.quantize(w)
    q, scale, offset = nf4.absmax_dq_quantize(absmax)
    back = nf4.absmax_dq_dequant(q, scale, offset).reshape(absmax.shape)
    # relative change of the constants is small: within a step of 1/127 of the group's spread
    assert np.max(np.abs(back - absmax)) <= 0.5 * scale.max() + 1e-9
    deq = nf4.dequant_bf16_bits(packed, back)
    L = nf4.nf4_levels().astype(np.float64)
    codes = nf4.unpack_codes(packed)
    want = nf4.f32_to_bf16_bits((L[codes] * np.repeat(back.astype(np.float64), 64, axis=1)).astype(np.float32))
    assert np.array_equal(deq, want)
