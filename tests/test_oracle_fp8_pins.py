"""Pins the oracle's MXFP8 part (E4M3 / E5M2 elements with one E8M0 scale per 32 values) to
facts outside itself.

"Stable FP4 Training via Transposition-Invariant Block Quantization" ("The fix, and its
supporting cast") quantizes the query and key projections in MXFP8 instead of FP4; the pages fix
no element encoding, so the oracle takes the OCP MX FP8 types. The independent references here
are PyTorch's own float8_e4m3fn / float8_e5m2 types (decoding of every code, and its float ->
float8 conversion, which rounds to nearest with ties to even), brute-force searches over exact
rationals, and statistical or enumerated properties of stochastic rounding.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

FMTS = {0: (torch.float8_e4m3fn, 448.0, 464.0, 8), 1: (torch.float8_e5m2, 57344.0, 61440.0, 15)}


def torch_decode(fmt):
    return torch.arange(256, dtype=torch.uint8).view(FMTS[fmt][0]).double().numpy()


def all_finite_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_decode_matches_torch_for_every_code(orc, fmt):
    ref = torch_decode(fmt)
    got = np.array([orc.fp8_decode(c, fmt) for c in range(256)])
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # the largest magnitude and the count of finite codes per sign
    largest = FMTS[fmt][1]
    assert orc.fp8_magnitude(0x7E if fmt == 0 else 0x7B, fmt) == largest
    assert fin[:128].sum() == (127 if fmt == 0 else 124)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 2.0 ** 5])
def test_fp8_rne_matches_torch_over_all_bf16(orc, fmt, scale):
    """Every finite bf16 value (times a power of two) below torch's overflow threshold encodes
    as torch's float -> float8 conversion (nearest, ties to even, signs copied)."""
    dt, largest, overflow, _ = FMTS[fmt]
    v = all_finite_bf16_as_f32()
    v = v[np.abs(v) <= 2.0 ** 100].astype(np.float64) * scale
    v = v[np.abs(v) <= overflow if fmt == 0 else np.abs(v) < overflow].astype(np.float32)
    ref = torch.from_numpy(v.copy()).to(dt).view(torch.uint8).numpy()
    got = np.array([orc.fp8_encode(float(x), fmt) for x in v], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_rne_matches_torch_on_random_fp32(orc, fmt):
    dt, largest, _, _ = FMTS[fmt]
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 10, 20000))).astype(np.float32)
    v = np.clip(v, -largest, largest).astype(np.float32)
    ref = torch.from_numpy(v.copy()).to(dt).view(torch.uint8).numpy()
    got = np.array([orc.fp8_encode(float(x), fmt) for x in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_saturates_at_largest(orc, fmt):
    largest = FMTS[fmt][1]
    top = 0x7E if fmt == 0 else 0x7B
    for v in [largest, largest * 1.01, largest * 4, 3.0e38]:
        assert orc.fp8_encode(v, fmt) == top
        assert orc.fp8_encode(-v, fmt) == 0x80 | top
        assert orc.fp8_encode(v, fmt, 1, 0) == top


def brute_floor_e(amax, emax):
    if amax == 0:
        return -127
    a = Fraction(amax)
    e = max(e for e in range(-300, 300) if Fraction(2) ** (e + emax) <= a)
    return min(127, max(-127, e))


def brute_ceil_e(amax, largest):
    if amax == 0:
        return -127
    a = Fraction(amax)
    e = min(e for e in range(-300, 300) if a <= Fraction(largest) * Fraction(2) ** e)
    return min(127, max(-127, e))


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_scale_exponents_vs_brute_force(orc, fmt):
    """Floor: 2^(e + emax) <= amax < 2^(e + emax + 1); ceil: least e with amax <= largest 2^e.
    Checked on every 7th positive finite bf16 value and on the binade edges."""
    _, largest, _, emax = FMTS[fmt]
    vals = all_finite_bf16_as_f32()
    vals = vals[vals > 0][::7]
    edges = [largest * 2.0 ** k for k in range(-140, 110, 17)]
    edges += [np.nextafter(np.float32(x), np.float32(np.inf)) for x in edges]
    for a in list(vals) + [np.float32(x) for x in edges] + [np.float32(0.0)]:
        a = float(np.float32(a))
        if not math.isfinite(a):
            continue
        assert orc.fp8_scale_exponent(a, 0, fmt) == brute_floor_e(a, emax), a
        assert orc.fp8_scale_exponent(a, 1, fmt) == brute_ceil_e(a, largest), a


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_ceil_scale_never_clips(orc, fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, size=(64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    codes, scales = orc.quantize_fp8(x, fmt=fmt, scale_rule=1)
    top = 0x7E if fmt == 0 else 0x7B
    largest = FMTS[fmt][1]
    e = scales.astype(np.int64) - 127
    xb = np.abs(x.reshape(64, 8, 32)).astype(np.float64)
    # the top code only for values at least half a top step below the largest magnitude
    emax, mb = FMTS[fmt][3], (3 if fmt == 0 else 2)
    sat = (codes.reshape(64, 8, 32) & 0x7F) == top
    assert np.all(~sat | (xb * np.exp2(-e)[..., None] >= largest - 2.0 ** (emax - mb - 1)))
    assert np.all(xb.max(-1) <= largest * np.exp2(e))


@pytest.mark.parametrize("fmt,v", [(0, 1.3), (0, 0.0037), (0, 300.0), (1, 1.3), (1, 3.1e-5),
                                   (1, 40000.0)])
def test_fp8_sr_up_count_over_all_fields(orc, fmt, v):
    """Over all 2^16 random fields the number that round up is ceil(frac * 2^16), frac the exact
    position of v between its two neighbours, and they are the smallest fields."""
    v = float(np.float32(v))
    dn = orc.fp8_encode(v, fmt, 1, 0xFFFF)
    lo, hi = orc.fp8_decode(dn, fmt), orc.fp8_decode(dn + 1, fmt)
    assert lo <= v < hi
    frac = (Fraction(v) - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
    ups = np.array([orc.fp8_encode(v, fmt, 1, r) != dn for r in range(1 << 16)])
    n = int(ups.sum())
    assert n == math.ceil(frac * (1 << 16))
    assert ups[:n].all() and not ups[n:].any()


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp8_sr_unbiased_through_quantizer(orc, fmt):
    """E[SR(x)] = x: over 200 seeds, the summed deviation of the dequantized means from x is
    within 5 standard deviations of the rounding noise, whose variance follows from each
    element's two neighbours (torch's decoding of the codes) and its position between them."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    n = 200
    acc = np.zeros_like(x, dtype=np.float64)
    for seed in range(n):
        c, s = orc.quantize_fp8(x, fmt=fmt, scale_rule=1, round_mode=1, seed=seed)
        acc += orc.dequantize_fp8_f64(c, s, 32, 64, fmt)
    mean = acc / n
    grid = np.unique(np.abs(torch_decode(fmt)[np.isfinite(torch_decode(fmt))]))
    e = (s.astype(np.int64) - 127).repeat(32, axis=1)  # the scale does not depend on the seed
    v = np.abs(x.astype(np.float64)) * np.exp2(-e)
    k = np.searchsorted(grid, v, side="right") - 1
    lo, hi = grid[k], grid[np.minimum(k + 1, grid.size - 1)]
    step = (hi - lo) * np.exp2(e)
    p = np.where(hi > lo, (v - lo) / np.where(hi > lo, hi - lo, 1.0), 0.0)
    var = step ** 2 * p * (1 - p) / n
    dev = mean - x
    assert np.all(np.abs(dev[var == 0]) == 0)
    assert abs(dev.sum()) < 5 * np.sqrt(var.sum())
    z2 = dev[var > 0] ** 2 / var[var > 0]
    assert z2.mean() < 1.5


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rule", [0, 1])
def test_fp8_quantize_rows_vs_torch_blockwise(orc, fmt, rule):
    """A row block's codes are torch's nearest-even float8 conversion of x * 2^-e, with e the
    brute-force scale exponent of the block maximum (values clamped to the largest first)."""
    dt, largest, _, emax = FMTS[fmt]
    rng = np.random.default_rng(7 + fmt + 2 * rule)
    x = (rng.standard_t(3, (16, 128)) * np.exp2(rng.integers(-8, 8, (16, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    x[5, 40] = -0.0
    codes, scales = orc.quantize_fp8(x, fmt=fmt, scale_rule=rule)
    for r in range(16):
        for b in range(4):
            blk = x[r, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            e = brute_floor_e(amax, emax) if rule == 0 else brute_ceil_e(amax, largest)
            assert scales[r, b] == e + 127
            v = (blk * np.float32(2.0 ** -e)).astype(np.float32)
            v = np.clip(v, -largest, largest)
            ref = torch.from_numpy(v.copy()).to(dt).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 32 * b:32 * b + 32], ref), (r, b)


def test_fp8_columns_are_rows_of_transpose(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    for fmt in (0, 1):
        c0, s0 = orc.quantize_fp8(x, fmt=fmt, axis=0, scale_rule=1)
        c1, s1 = orc.quantize_fp8(np.ascontiguousarray(x.T), fmt=fmt, axis=1, scale_rule=1)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_fp8_hadamard_vs_dense_rotation(orc):
    """With the rotation, a block quantizes as the unrotated quantizer applied to D H x (dense
    Sylvester matrix in float64; the butterflies are exact here on small integers)."""
    rng = np.random.default_rng(4)
    x = rng.integers(-8, 9, (8, 64)).astype(np.float32)
    mask = 0xA5A5F00F
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)], float)
    D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])
    y = np.concatenate([(x[:, 32 * b:32 * b + 32] * D) @ H.T for b in range(2)], axis=1)
    for fmt in (0, 1):
        c1, s1 = orc.quantize_fp8(x, fmt=fmt, hadamard=1, sign_mask=mask, scale_rule=1)
        c2, s2 = orc.quantize_fp8(y.astype(np.float32), fmt=fmt, scale_rule=1)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_fp8_round_trip_within_half_step(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    for fmt in (0, 1):
        c, s = orc.quantize_fp8(x, fmt=fmt, scale_rule=1)
        d = orc.dequantize_fp8_f64(c, s, 32, 128, fmt)
        mb = 3 if fmt == 0 else 2
        # relative half step of the element format, above its subnormal range
        big = np.abs(x) >= np.repeat(np.abs(x).reshape(32, 4, 32).max(-1), 32, 1) * 2.0 ** -5
        rel = np.abs(d - x) / np.abs(x)
        assert np.all(rel[big] <= 2.0 ** -(mb + 1) + 1e-12)


def test_fp8_gemm_matches_rational_brute_force(orc):
    rng = np.random.default_rng(6)
    M, N, K = 3, 4, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    aq, as_ = orc.quantize_fp8(a, fmt=0)
    bq, bs = orc.quantize_fp8(b, fmt=1)
    C, Cabs = orc.gemm_fp8(aq, as_, 0, bq, bs, 1, M, N, K, alpha_exp=-3)
    ta = torch.from_numpy(aq).view(torch.float8_e4m3fn).double().numpy()
    tb = torch.from_numpy(bq).view(torch.float8_e5m2).double().numpy()
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = (Fraction(ta[m, k]) * Fraction(2) ** (int(as_[m, k // 32]) - 127) *
                     Fraction(tb[n, k]) * Fraction(2) ** (int(bs[n, k // 32]) - 127))
                s += p
                sa += abs(p)
            assert Fraction(C[m, n]) == s / 8 and Fraction(Cabs[m, n]) == sa / 8
