"""Pins the CPU oracle to facts outside itself (closed forms, brute force, invariants).

Each test states the page fact or mathematical identity it checks. Pages, by title and section:
  [P1] "Block-Scaled MXFP4 With Stochastic Hadamard Rounding ..." paragraphs 1-2
  [P3] "Stable FP4 Training via Transposition-Invariant Block Quantization",
       "Why FP4 training is the current frontier", "The fix, and its supporting cast"
  [P4] "Training LLMs with MXFP4", abstract
"""
from fractions import Fraction
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_grid():
    vals = []
    with open(os.path.join(HERE, "golden", "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return np.array(vals, dtype=np.float64)


GRID = golden_grid()


def all_finite_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def brute_rne_code(v: float) -> int:
    """Nearest magnitude by exhaustive distance, ties to the even index; sign bit copied."""
    a = Fraction(abs(float(v)))
    d = [abs(a - Fraction(g)) for g in GRID]  # exact distances
    dmin = min(d)
    best = [i for i in range(8) if d[i] == dmin]
    idx = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
    return (8 if np.signbit(v) else 0) | idx


def brute_floor_e(amax: float) -> int:
    if amax == 0:
        return -127
    e = max(e for e in range(-200, 200) if 2.0 ** (e + 2) <= amax)
    return min(127, max(-127, e))


def brute_ceil_e(amax: float) -> int:
    if amax == 0:
        return -127
    e = min(e for e in range(-200, 200) if amax <= 6.0 * 2.0 ** e)
    return min(127, max(-127, e))


def pack(codes_2d: np.ndarray) -> np.ndarray:
    c = codes_2d.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def decode_f64(code: int) -> float:
    mag = GRID[code & 7]
    return -mag if code & 8 else mag


# ----------------------------------------------------------------------------------------------
# E2M1 element format [P3 "Why FP4 ..."]
# ----------------------------------------------------------------------------------------------
def test_e2m1_decode_matches_format_grid(orc):
    for code in range(16):
        want = GRID[code & 7] * (-1.0 if code & 8 else 1.0)
        got = orc.e2m1_decode(code)
        assert got == want and np.signbit(got) == bool(code & 8)
    # 8 magnitudes per sign, 16 codes in all, strictly increasing
    assert len(GRID) == 8 and np.all(np.diff(GRID) > 0)


@pytest.mark.parametrize("e", [0, -3, 5])
def test_rne_exhaustive_over_bf16(orc, e):
    """Round-to-nearest-even: every finite bf16 value, scaled by 2^-e, vs brute force."""
    xs = all_finite_bf16_as_f32()
    # keep the scaled values in a range where the grid matters, plus all the small/large ones
    with np.errstate(over="ignore"):
        vs = xs[:: 1 if e == 0 else 7] * np.float32(2.0 ** -e)
    for v in vs[np.isfinite(vs)]:
        assert orc.e2m1_encode(float(v), 0) == brute_rne_code(float(v)), float(v)


def test_rne_ties_go_to_even_code(orc):
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, idx in ties.items():
        assert orc.e2m1_encode(v, 0) == idx
        assert orc.e2m1_encode(-v, 0) == 8 | idx
    assert orc.e2m1_encode(7.99, 0) == 7 and orc.e2m1_encode(1e30, 0) == 7  # saturation
    assert orc.e2m1_encode(-0.0, 0) == 8 and orc.e2m1_encode(-1e-30, 0) == 8  # sign copied


# ----------------------------------------------------------------------------------------------
# E8M0 scale [P1 paragraph 1; P3 "Why FP4 ..." and "The fix ..."]
# ----------------------------------------------------------------------------------------------
def test_scale_exponents_exhaustive_over_positive_bf16(orc):
    xs = all_finite_bf16_as_f32()
    xs = xs[xs >= 0]
    for a in xs:
        a = float(a)
        assert orc.scale_exponent(a, 0) == brute_floor_e(a), a
        assert orc.scale_exponent(a, 1) == brute_ceil_e(a), a


def test_ceil_scale_never_clips_and_is_minimal(orc):
    """'rounded up to the next power of two ... nothing ever clips' [P3 "The fix ..."]."""
    rng = np.random.default_rng(7)
    amaxes = np.concatenate([
        all_finite_bf16_as_f32()[::3],
        (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)])
    for a in np.abs(amaxes):
        a = float(a)
        if a == 0 or not np.isfinite(a):
            continue
        e = orc.scale_exponent(a, 1)
        assert a * 2.0 ** -e <= 6.0
        if -127 < e:  # one step smaller would clip (unless clamped)
            assert a * 2.0 ** -(e - 1) > 6.0


def test_floor_scale_puts_max_in_top_binades(orc):
    """OCP floor rule: the scaled maximum lands in [4, 8), so only > 6 saturates."""
    rng = np.random.default_rng(8)
    for a in np.abs(rng.standard_normal(5000) * 10.0 ** rng.uniform(-20, 20, 5000)):
        a = float(np.float32(a))
        e = orc.scale_exponent(a, 0)
        if -127 < e < 127:
            assert 4.0 <= a * 2.0 ** -e < 8.0


# ----------------------------------------------------------------------------------------------
# stochastic rounding: E[round(x)] = x [P3 "The fix ..."; P4]
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("v", [0.1, 0.3, 0.7, 1.2, 1.6, 2.25, 2.99, 3.3, 4.5, 5.9, -0.9, -5.0,
                               0.5, 4.0, 6.0])
def test_sr_is_unbiased_over_all_random_fields(orc, v):
    """Enumerate all 2^16 random fields: the mean equals v up to 2^-16 of the grid step."""
    v32 = float(np.float32(v))
    total = Fraction(0)
    for r in range(1 << 16):
        total += Fraction(decode_f64(orc.e2m1_encode(v32, 1, r)))
    mean = total / (1 << 16)
    a = abs(v32)
    lo = max(g for g in GRID if g <= a)
    hi = min([g for g in GRID if g > a] or [6.0])
    step = hi - lo if hi > lo else 2.0
    assert abs(mean - Fraction(v32)) <= Fraction(step) / (1 << 16)
    # grid points never move
    if a in GRID:
        assert mean == Fraction(v32)


@pytest.mark.parametrize("v", [0.1, 0.3, 0.7, 1.2, 1.6, 2.25, 2.99, 3.3, 4.5, 5.9, -0.9, -5.0,
                               0.75, 1.0000001, 5.9999995, 0.5, 4.0, 3e-9, 0.7500001])
def test_sr_up_count_over_all_fields(orc, v):
    """Over all 2^16 random fields the magnitude rounds up for exactly ceil(f 2^16) of them
    (f the exact position between the grid neighbours, from Fractions), and those are the
    smallest fields: a strict comparison of the field with f 2^16."""
    v32 = float(np.float32(v))
    a = abs(Fraction(v32))
    lo = max(g for g in GRID if g <= a)
    hi = min(g for g in GRID if g > a)
    f = (a - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
    lo_code = orc.e2m1_encode(float(lo) if v32 >= 0 else -float(lo), 0)
    ups = [r for r in range(1 << 16) if orc.e2m1_encode(v32, 1, r) != lo_code]
    n = f * (1 << 16)
    assert len(ups) == (n.numerator + n.denominator - 1) // n.denominator  # ceil
    assert ups == list(range(len(ups)))


def test_sr_unbiased_over_seeds_through_quantizer(orc):
    """Full quantize path, 2000 Philox seeds: the mean reconstruction is within 4 sigma of x."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 32)).astype(np.float32)
    n = 2000
    acc = np.zeros(32)
    acc2 = np.zeros(32)
    for s in range(n):
        c, sc = orc.quantize(x, axis=1, scale_rule=1, round_mode=1, seed=s * 7919 + 11)
        d = orc.dequantize(c, sc, 1, 32).astype(np.float64)[0]
        acc += d
        acc2 += d * d
    mean = acc / n
    var = np.maximum(acc2 / n - mean ** 2, 1e-30)
    assert np.all(np.abs(mean - x[0]) <= 4.0 * np.sqrt(var / n) + 1e-7)


# ----------------------------------------------------------------------------------------------
# Philox4x32-10 (statistics here; third-party known answers in test_oracle_philox_rocrand.py)
# ----------------------------------------------------------------------------------------------
def test_philox_bits_are_balanced(orc):
    words = np.array([orc.philox4x32_10([i, 0, 0, 0], [1234, 0]) for i in range(4096)],
                     dtype=np.uint32).ravel()
    bits = ((words[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.float64)
    freq = bits.mean(axis=0)
    n = len(words)
    assert np.all(np.abs(freq - 0.5) < 5 * 0.5 / np.sqrt(n))
    f16 = np.concatenate([words & 0xFFFF, words >> 16]).astype(np.float64)
    assert abs(f16.mean() - 32767.5) < 5 * 18918.6 / np.sqrt(len(f16))


def test_philox_avalanche(orc):
    base = orc.philox4x32_10([5, 6, 7, 8], [9, 10])
    flips = []
    for w in range(4):
        for b in range(32):
            c = [5, 6, 7, 8]
            c[w] ^= 1 << b
            o = orc.philox4x32_10(c, [9, 10])
            flips.append(sum(bin(int(x) ^ int(y)).count("1") for x, y in zip(o, base)))
    assert 60 < np.mean(flips) < 68  # ~64 of 128 output bits change


def test_sr_field_mapping(orc):
    """Element i takes 16-bit field i % 8 of the Philox output at counter i / 8."""
    seed = (0xDEADBEEF << 32) | 1234
    for i in [0, 1, 2, 7, 8, 15, 1 << 33, (1 << 33) + 5]:
        g = i >> 3
        out = orc.philox4x32_10([g & 0xFFFFFFFF, g >> 32, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        w = int(out[(i & 7) >> 1])
        assert orc.sr_field(seed, i) == ((w >> 16) if i & 1 else (w & 0xFFFF))


# ----------------------------------------------------------------------------------------------
# Walsh-Hadamard [P1 paragraph 2]: H32 with H.H = 32 I
# ----------------------------------------------------------------------------------------------
def sylvester_h32():
    i = np.arange(32)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def test_fwht_columns_form_sylvester_matrix(orc):
    H = np.stack([orc.fwht32(np.eye(32, dtype=np.float32)[j]) for j in range(32)], axis=1)
    assert np.array_equal(H.astype(np.int64), sylvester_h32())
    assert np.array_equal(H.astype(np.int64) @ H.astype(np.int64), 32 * np.eye(32, dtype=np.int64))


def test_fwht_matches_dense_product(orc):
    rng = np.random.default_rng(4)
    H = sylvester_h32().astype(np.float64)
    for _ in range(200):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-5, 5)).astype(np.float32)
        y = orc.fwht32(x).astype(np.float64)
        ref = H @ x.astype(np.float64)
        assert np.all(np.abs(y - ref) <= 5 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum())
    # small integers: exact, and applying twice gives 32 x
    for _ in range(50):
        x = rng.integers(-1000, 1000, 32).astype(np.float32)
        y = orc.fwht32(x)
        assert np.array_equal(y.astype(np.float64), H @ x.astype(np.float64))
        assert np.array_equal(orc.fwht32(y), 32 * x)


# ----------------------------------------------------------------------------------------------
# whole quantizer vs per-block brute force
# ----------------------------------------------------------------------------------------------
def brute_quantize_rows(x: np.ndarray, rule: int, H=None, mask=0):
    """Brute force 1x32 along rows; rotation (if any) done exactly in float64 on integer data."""
    rows, cols = x.shape
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])
    for r in range(rows):
        for b in range(cols // 32):
            blk = x[r, b * 32:(b + 1) * 32].astype(np.float64)
            if H is not None:
                blk = H @ (D * blk)
            amax = float(np.abs(blk).max())
            e = brute_floor_e(amax) if rule == 0 else brute_ceil_e(amax)
            scales[r, b] = e + 127
            for j in range(32):
                codes[r, b * 32 + j] = brute_rne_code(blk[j] * 2.0 ** -e)
    return pack(codes), scales


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_rows_vs_brute_force(orc, rule):
    rng = np.random.default_rng(10 + rule)
    x = (rng.standard_normal((6, 96)) * 10.0 ** rng.uniform(-3, 3, (6, 1))).astype(np.float32)
    x[2, 5] *= 300.0
    x[4, 32:64] = 0.0  # an all-zero block
    c, s = orc.quantize(x, axis=1, scale_rule=rule)
    bc, bs = brute_quantize_rows(x, rule)
    assert np.array_equal(s, bs) and np.array_equal(c, bc)


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_columns_is_rows_of_transpose(orc, rule):
    """axis=0 output equals the axis=1 brute force of the materialised transpose."""
    rng = np.random.default_rng(20 + rule)
    x = rng.standard_normal((64, 40)).astype(np.float32)
    c, s = orc.quantize(x, axis=0, scale_rule=rule)
    bc, bs = brute_quantize_rows(np.ascontiguousarray(x.T), rule)
    assert np.array_equal(s, bs) and np.array_equal(c, bc)


@pytest.mark.parametrize("mask", [0, 0x8F3A51C7])
def test_quantize_hadamard_vs_dense_rotation(orc, mask):
    """Integer data keeps the fp32 butterflies exact, so the dense float64 rotation H.D.x must
    give identical scales and codes [P1 paragraph 2; P4]."""
    rng = np.random.default_rng(30)
    x = rng.integers(-64, 64, (4, 64)).astype(np.float32)
    x[1, 3] = 4000.0  # outlier spread over its block by the rotation
    c, s = orc.quantize(x, axis=1, scale_rule=1, hadamard=1, sign_mask=mask)
    bc, bs = brute_quantize_rows(x, 1, H=sylvester_h32().astype(np.float64), mask=mask)
    assert np.array_equal(s, bs) and np.array_equal(c, bc)


def test_sr_uses_source_element_index(orc):
    """The random field of each element is the Philox field of its source row-major index, in
    both block orientations."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    seed = 99
    for axis in (1, 0):
        c, s = orc.quantize(x, axis=axis, scale_rule=1, round_mode=1, seed=seed)
        src = x if axis == 1 else np.ascontiguousarray(x.T)
        want = np.zeros(src.shape, dtype=np.uint8)
        for r in range(src.shape[0]):
            for b in range(src.shape[1] // 32):
                e = int(s[r, b]) - 127
                for j in range(32):
                    cc = b * 32 + j
                    i = r * 64 + cc if axis == 1 else cc * 64 + r  # source (row, col) index
                    want[r, cc] = orc.e2m1_encode(float(np.float32(src[r, cc]) * np.float32(2.0 ** -e)),
                                                  1, orc.sr_field(seed, i))
        assert np.array_equal(c, pack(want))


def test_hadamard_round_trip_error_bound(orc):
    """Dequantize with (1/32) D H recovers x: per block ||x - x^||_2 <= 2^e (RNE half-steps in
    the rotated domain, shrunk by the orthogonal 1/sqrt(32) factor)."""
    rng = np.random.default_rng(50)
    x = rng.standard_t(3, (16, 256)).astype(np.float32)
    mask = 0x5A5AF00F
    c, s = orc.quantize(x, axis=1, scale_rule=1, hadamard=1, sign_mask=mask)
    y = orc.dequantize(c, s, 16, 256, 1, inv_hadamard=1, sign_mask=mask)
    err = (y.astype(np.float64) - x).reshape(16, 8, 32)
    bound = 2.0 ** (s.astype(np.float64) - 127) * 1.0001
    assert np.all(np.sqrt((err ** 2).sum(-1)) <= bound)
    # the wrong mask does not round-trip
    y2 = orc.dequantize(c, s, 16, 256, 1, inv_hadamard=1, sign_mask=mask ^ 1)
    assert np.abs(y2 - x).max() > 10 * np.abs(y - x).max()


def test_dequantize_exact_values(orc):
    rng = np.random.default_rng(60)
    codes = rng.integers(0, 256, (3, 32), dtype=np.uint8)
    scales = rng.integers(100, 150, (3, 2), dtype=np.uint8)
    y = orc.dequantize(codes, scales, 3, 64)
    for r in range(3):
        for c in range(64):
            code = (codes[r, c // 2] >> (4 * (c & 1))) & 0xF
            assert y[r, c] == decode_f64(code) * 2.0 ** (int(scales[r, c // 32]) - 127)


# ----------------------------------------------------------------------------------------------
# 32x32 blocks: transposition invariance [P3 "The fix ..."]
# ----------------------------------------------------------------------------------------------
def test_2d_blocks_transposition_invariant(orc):
    rng = np.random.default_rng(70)
    w = (rng.standard_t(3, (96, 64)) * 0.02).astype(np.float32)
    w[:, 7] *= 100.0
    c, s, ct, st = orc.quantize_2d(w, scale_rule=1)
    wt = np.ascontiguousarray(w.T)
    c2, s2, ct2, st2 = orc.quantize_2d(wt, scale_rule=1)
    assert np.array_equal(s, s2.T) and np.array_equal(st, s2)
    assert np.array_equal(c, ct2) and np.array_equal(ct, c2)


def test_2d_scale_from_tile_max_and_codes_brute(orc):
    rng = np.random.default_rng(71)
    w = rng.standard_normal((64, 64)).astype(np.float32)
    c, s, ct, st = orc.quantize_2d(w, scale_rule=1)
    want = np.zeros((64, 64), dtype=np.uint8)
    for br in range(2):
        for bc in range(2):
            t = w[br * 32:(br + 1) * 32, bc * 32:(bc + 1) * 32].astype(np.float64)
            e = brute_ceil_e(float(np.abs(t).max()))
            assert s[br, bc] == e + 127
            for i in range(32):
                for j in range(32):
                    want[br * 32 + i, bc * 32 + j] = brute_rne_code(t[i, j] * 2.0 ** -e)
    assert np.array_equal(c, pack(want))


def test_1d_blocks_are_not_transposition_invariant(orc):
    """The inconsistency 2-D blocks remove [P3 "The aha ..."]: with 1x32 blocks an element's
    row scale and column scale differ for a large share of elements."""
    rng = np.random.default_rng(72)
    x = rng.standard_t(3, (128, 128)).astype(np.float32)
    _, srow = orc.quantize(x, axis=1, scale_rule=1)
    _, scol = orc.quantize(x, axis=0, scale_rule=1)
    row_scale = np.repeat(srow, 32, axis=1)            # [r][c]
    col_scale = np.repeat(scol, 32, axis=1).T          # scol is [c][r/32]
    assert (row_scale != col_scale).mean() > 0.2


# ----------------------------------------------------------------------------------------------
# GEMM oracle vs exact rational brute force
# ----------------------------------------------------------------------------------------------
def test_gemm_matches_rational_brute_force(orc):
    rng = np.random.default_rng(80)
    M, N, K = 3, 5, 64
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    bs = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    C, Cabs = orc.gemm(aq, as_, 1, bq, bs, 1, M, N, K, alpha_exp=-5)

    def val(q, s, r, k):
        code = (int(q[r, k // 2]) >> (4 * (k & 1))) & 0xF
        return Fraction(decode_f64(code)) * Fraction(2) ** (int(s[r, k // 32]) - 127)

    for m in range(M):
        for n in range(N):
            terms = [val(aq, as_, m, k) * val(bq, bs, n, k) for k in range(K)]
            exact = sum(terms) * Fraction(1, 32)
            assert Fraction(C[m, n]) == exact
            assert Fraction(Cabs[m, n]) == sum(abs(t) for t in terms) * Fraction(1, 32)


def test_gemm_scale_shift_doubles_output(orc):
    rng = np.random.default_rng(81)
    M, N, K = 32, 32, 128
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    bs = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    C, _ = orc.gemm(aq, as_, 1, bq, bs, 1, M, N, K)
    C2, _ = orc.gemm(aq, as_ + 1, 1, bq, bs, 1, M, N, K)
    assert np.array_equal(C2, 2 * C)
    # 2-D scales: g = 32 reads one scale row per 32 rows
    s2 = rng.integers(110, 140, (1, K // 32), dtype=np.uint8)
    C3, _ = orc.gemm(aq, s2, 32, bq, bs, 1, M, N, K)
    C4, _ = orc.gemm(aq, np.repeat(s2, 32, axis=0), 1, bq, bs, 1, M, N, K)
    assert np.array_equal(C3, C4)


@pytest.mark.parametrize("nthreads", [2, 3, 8])
def test_threaded_driver_equals_one_thread(orc, nthreads):
    """The threaded driver only splits the row range into 32-row pieces; every option set
    (1x32 along either axis, Hadamard with random signs, SR, 32x32 tiles) and a row range whose
    piece count does not divide by the thread count give the same bytes as one thread."""
    rng = np.random.default_rng(31)
    x = (rng.standard_t(3, size=(32 * 37, 96)) * 0.2).astype(np.float32)
    mask = 0x9E3779B9
    for axis in (1, 0):
        for rr in (None, (64, 32 * 30)):
            kw = dict(axis=axis, scale_rule=1, round_mode=1, hadamard=1, sign_mask=mask, seed=77,
                      row_range=rr)
            one = orc.quantize(x, nthreads=1, **kw)
            many = orc.quantize(x, nthreads=nthreads, **kw)
            for a, b in zip(one, many):
                assert np.array_equal(a, b)
    for rr in (None, (32, 32 * 33)):
        one = orc.quantize_2d(x, scale_rule=1, round_mode=1, seed=5, row_range=rr, nthreads=1)
        many = orc.quantize_2d(x, scale_rule=1, round_mode=1, seed=5, row_range=rr,
                               nthreads=nthreads)
        for a, b in zip(one, many):
            assert np.array_equal(a, b)
    # the untouched rows outside a range stay zero, and the range itself is fully written
    c, s = orc.quantize(x, axis=1, row_range=(64, 128), nthreads=nthreads)
    assert not c[:64].any() and not c[128:].any() and s[64:128].all()
