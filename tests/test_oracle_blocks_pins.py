"""Pins the oracle's block-size variants and the 1D scale-mismatch map.

"Stable FP4 Training via Transposition-Invariant Block Quantization": "The fix, and its
supporting cast" (Table 4 compares 8x8, 32x32 and 64x64 tiles) and "The aha: transposition
scrambles the blocks" (Figure 1 shows scale-difference maps, large for 1D blocks, near zero for
2D). The references: brute-force scale exponents and nearest-even codes over exact rationals,
the transposition identity, and the antisymmetry of the map on symmetric matrices.
"""
import numpy as np
import pytest

from tests.test_oracle_pins import brute_ceil_e, brute_floor_e, brute_rne_code


def unpack(codes, rows, cols):
    c = codes.reshape(rows, cols // 2)
    out = np.empty((rows, cols), dtype=np.int64)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


@pytest.mark.parametrize("B", [8, 64])
@pytest.mark.parametrize("rule", [0, 1])
def test_block_quantize_vs_brute_force(orc, B, rule):
    rng = np.random.default_rng(B + rule)
    rows, cols = 2 * B, 3 * B
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-6, 6, (rows, 1)))).astype(np.float32)
    x[:B, :B] = 0.0  # an all-zero tile
    codes, scales, codes_t, scales_t = orc.quantize_2d_block(x, B, scale_rule=rule)
    got = unpack(codes, rows, cols)
    for br in range(rows // B):
        for bc in range(cols // B):
            tile = x[br * B:(br + 1) * B, bc * B:(bc + 1) * B]
            amax = float(np.abs(tile).max())
            e = brute_floor_e(amax) if rule == 0 else brute_ceil_e(amax)
            assert scales[br, bc] == e + 127 and scales_t[bc, br] == e + 127
            for i in range(0, B, 3 if B == 64 else 1):
                for j in range(B):
                    v = float(np.float32(tile[i, j] * np.float32(2.0 ** -e)))
                    assert got[br * B + i, bc * B + j] == brute_rne_code(v)
    assert np.array_equal(unpack(codes_t, cols, rows), got.T)


@pytest.mark.parametrize("B", [8, 32, 64])
def test_block_quantize_transposition_invariant(orc, B):
    rng = np.random.default_rng(3 * B)
    x = rng.standard_normal((2 * B, 4 * B)).astype(np.float32)
    c, s, ct, st = orc.quantize_2d_block(x, B)
    c2, s2, ct2, st2 = orc.quantize_2d_block(np.ascontiguousarray(x.T), B)
    assert np.array_equal(s2, s.T) and np.array_equal(c2, ct) and np.array_equal(ct2, c)


def test_block_32_matches_the_32x32_quantizer(orc):
    rng = np.random.default_rng(8)
    x = rng.standard_t(3, (96, 160)).astype(np.float32)
    for rule, rnd in [(0, 0), (1, 1)]:
        a = orc.quantize_2d_block(x, 32, scale_rule=rule, round_mode=rnd, seed=5)
        b = orc.quantize_2d(x, scale_rule=rule, round_mode=rnd, seed=5)
        assert all(np.array_equal(p, q) for p, q in zip(a, b))


@pytest.mark.parametrize("rule", [0, 1])
def test_mismatch_map_vs_brute_force(orc, rule):
    rng = np.random.default_rng(20 + rule)
    rows, cols = 64, 96
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-4, 4, (rows, cols)))).astype(np.float32)
    m = orc.scale_mismatch_map(x, scale_rule=rule)
    e = brute_floor_e if rule == 0 else brute_ceil_e
    for i in range(rows):
        for j in range(0, cols, 5):
            row_blk = np.abs(x[i, 32 * (j // 32):32 * (j // 32) + 32]).max()
            col_blk = np.abs(x[32 * (i // 32):32 * (i // 32) + 32, j]).max()
            assert m[i, j] == e(float(row_blk)) - e(float(col_blk)), (i, j)


def test_mismatch_map_is_antisymmetric_on_symmetric_matrices(orc):
    rng = np.random.default_rng(4)
    a = rng.standard_t(3, (96, 96)).astype(np.float32)
    x = np.ascontiguousarray(np.triu(a) + np.triu(a, 1).T)
    assert np.array_equal(x, x.T)
    m = orc.scale_mismatch_map(x).astype(np.int32)
    assert np.array_equal(m, -m.T) and np.abs(m).max() > 0


def test_mismatch_map_marks_non_finite_blocks(orc):
    x = np.ones((64, 64), dtype=np.float32)
    x[5, 40] = np.inf
    m = orc.scale_mismatch_map(x)
    # the row block (row 5, columns 32-63) and the column block (rows 0-31, column 40)
    assert np.all(m[5, 32:64] == -128) and np.all(m[0:32, 40] == -128)
    assert (m == -128).sum() == 32 + 32 - 1 and np.all(m[m != -128] == 0)


def test_mismatch_map_saturates(orc):
    """Exponent differences beyond the int8 range saturate at +-127."""
    x = np.full((32, 32), 1e-30, dtype=np.float32)
    x[0, 0] = 1e30   # in the block of row 0 and in the block of column 0
    m = orc.scale_mismatch_map(x).astype(np.int32)
    assert m[0, 0] == 0 and m[5, 5] == 0
    assert m[0, 5] == 127     # row block huge, column block tiny
    assert m[5, 0] == -127    # row block tiny, column block huge
