"""8x8 / 64x64 tiles, GEMMs on 64x64 scales, and the 1D scale-mismatch map, against the oracle.

Codes, scales and map bytes must be bit-exact; GEMMs within |gpu - exact| <= 2^-20 sum|ab|
(fp32 out) or its bf16 rounding bracket. The 64x64 scales come in the GEMM layout (each tile's
byte for both of its 32-wide halves); the oracle's canonical [rows/64][cols/64] must equal
either half. The last tests run the 2-D workload's tensors at full size on sampled row slabs.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import assert_bytes_equal, check_gemm, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_hadamard32_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def tile_input(rows, cols, dtype, seed):
    x = wl.student_t3((rows, cols), seed=seed)
    wl.outlier_columns(x, max(1, cols // 64), 100.0, seed=seed)
    x[:8, :8] = 0.0
    if rows > 16 and cols > 16:
        x[8:16, 8:16] = -0.0
    return x.to(dtype)


def check_blocks(mx_out, ref, B):
    c, s, ct, st = mx_out
    rc, rs, rct, rst = ref
    assert_bytes_equal(c, rc, "codes")
    assert_bytes_equal(ct, rct, "codes_t")
    if B == 64:
        hs, hst = host(s), host(st)
        assert np.array_equal(hs[:, 0::2], rs) and np.array_equal(hs[:, 1::2], rs)
        assert np.array_equal(hst[:, 0::2], rst) and np.array_equal(hst[:, 1::2], rst)
    else:
        assert_bytes_equal(s, rs, "scales")
        assert_bytes_equal(st, rst, "scales_t")


BLOCK_CASES = [
    # B, rows, cols, dtype
    (8, 32, 32, torch.bfloat16),
    (8, 64, 96, torch.float32),
    (8, 288, 544, torch.bfloat16),    # two workgroup tiles each way, the last partial
    (64, 64, 64, torch.bfloat16),
    (64, 128, 192, torch.float32),
    (64, 320, 576, torch.bfloat16),   # partial workgroup tiles
]


@pytest.mark.parametrize("B,rows,cols,dtype", BLOCK_CASES)
@pytest.mark.parametrize("rule,rnd", [(1, 0), (0, 0), (1, 1)])
def test_block_quantize_bit_exact(mx, orc, B, rows, cols, dtype, rule, rnd):
    x = tile_input(rows, cols, dtype, seed=B + rows + cols)
    out = mx.mx_quantize_2d_blocks(x.to(DEV), block=B, scale_rule=rule, round=rnd, seed=77)
    torch.cuda.synchronize()
    ref = orc.quantize_2d_block(wl.host_input(x), B, scale_rule=rule, round_mode=rnd, seed=77)
    check_blocks(out, ref, B)


def test_block_32_is_the_32x32_quantizer(mx):
    x = tile_input(96, 160, torch.bfloat16, seed=3).to(DEV)
    a = mx.mx_quantize_2d_blocks(x, block=32, scale_rule=1, round=1, seed=5)
    b = mx.mx_quantize_2d(x, scale_rule=1, round=1, seed=5)
    torch.cuda.synchronize()
    assert all(torch.equal(p, q) for p, q in zip(a, b))


def test_block_quantize_strided_and_non_finite(mx, orc):
    full = tile_input(128, 320, torch.float32, seed=9)
    full[70, 100] = float("inf")
    x = full[:, :256]
    for B in (8, 64):
        out = mx.mx_quantize_2d_blocks(full.to(DEV)[:, :256], block=B, scale_rule=1)
        torch.cuda.synchronize()
        ref = orc.quantize_2d_block(wl.host_input(x.contiguous()), B, scale_rule=1)
        check_blocks(out, ref, B)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_with_64x64_scales(mx, orc, out_dtype):
    """Fprop with 64x64-quantized W (g = 64) and Dgrad with its transposed copy, against the
    oracle on the same codes and scales."""
    T, K, N = 192, 512, 320
    X = wl.student_t3((T, K), seed=31).to(torch.bfloat16).to(DEV)
    W = tile_input(N, K, torch.bfloat16, seed=32).to(DEV)
    dY = wl.normal((T, N), 1e-3, seed=33).to(torch.bfloat16).to(DEV)
    xq, xs = mx.mx_quantize(X, scale_rule=1)
    wq, ws, wtq, wts = mx.mx_quantize_2d_blocks(W, block=64, scale_rule=1)
    dyq, dys = mx.mx_quantize(dY, scale_rule=1)
    y = mx.mx_gemm_fprop(xq, xs, 1, wq, ws, 64, out_dtype=out_dtype)
    dx = mx.mx_gemm_dgrad(dyq, dys, 1, wtq, wts, 64, out_dtype=out_dtype)
    torch.cuda.synchronize()
    C, Cabs = orc.gemm(host(xq), host(xs), 1, host(wq), host(ws), 64, T, N, K)
    check_gemm(y, C, Cabs)
    C, Cabs = orc.gemm(host(dyq), host(dys), 1, host(wtq), host(wts), 64, T, K, N)
    check_gemm(dx, C, Cabs)


@pytest.mark.parametrize("rows,cols,dtype", [(32, 32, torch.float32), (64, 96, torch.bfloat16),
                                             (96, 160, torch.float32), (320, 416, torch.bfloat16)])
@pytest.mark.parametrize("rule", [0, 1])
def test_mismatch_map_bit_exact(mx, orc, rows, cols, dtype, rule):
    x = wl.student_t3((rows, cols), seed=rows + cols)
    x *= torch.exp2(torch.randint(-3, 4, (rows, cols), generator=torch.Generator().manual_seed(1)))
    x = x.to(dtype)
    m = mx.mx_scale_mismatch_map(x.to(DEV), scale_rule=rule)
    torch.cuda.synchronize()
    ref = orc.scale_mismatch_map(wl.host_input(x), scale_rule=rule)
    assert_bytes_equal(m, ref, "map")


def test_mismatch_map_edges(mx, orc):
    """Strided input, a non-finite block, saturation, and a symmetric matrix (antisymmetric map)."""
    full = torch.full((64, 96), 1e-30)
    full[0, 0] = 1e30
    full[40, 50] = float("nan")
    x = full[:, :64]
    m = mx.mx_scale_mismatch_map(full.to(DEV)[:, :64])
    torch.cuda.synchronize()
    assert_bytes_equal(m, orc.scale_mismatch_map(wl.host_input(x.contiguous())), "map")
    a = wl.student_t3((96, 96), seed=5)
    s = torch.triu(a) + torch.triu(a, 1).T
    ms = host(mx.mx_scale_mismatch_map(s.to(DEV))).astype(np.int32)
    torch.cuda.synchronize()
    assert np.array_equal(ms, -ms.T) and np.abs(ms).max() > 0


def test_blocks_2d_workload_full_size(mx, orc):
    """The 2-D workload's W (14336 x 4096) and dY (8192 x 14336), bf16, ceil scale: 8x8 and 64x64
    tiles and the mismatch map of X (8192 x 4096), each checked on sampled row slabs."""
    d = wl.blocks_2d(device=DEV)
    for name in ("W", "dY"):
        src = d[name]
        rows, cols = src.shape
        for B in (8, 64):
            c, s, ct, st = mx.mx_quantize_2d_blocks(src, block=B, scale_rule=1)
            torch.cuda.synchronize()
            for r0 in (0, rows // 2, rows - 64):
                slab = wl.host_input(src[r0:r0 + 64])
                rc, rs, rct, rst = orc.quantize_2d_block(slab, B, scale_rule=1)
                assert np.array_equal(host(c[r0:r0 + 64]), rc)
                hs = host(s[r0 // B:(r0 + 64) // B])
                assert np.array_equal(hs if B == 8 else hs[:, 0::2], rs)
                assert np.array_equal(host(ct[:, r0 // 2:(r0 + 64) // 2]), rct)
            del c, s, ct, st
    X = d["X"]
    m = mx.mx_scale_mismatch_map(X)
    torch.cuda.synchronize()
    for r0 in (0, 4096, X.shape[0] - 32):
        ref = orc.scale_mismatch_map(wl.host_input(X[r0:r0 + 32]))
        assert np.array_equal(host(m[r0:r0 + 32]), ref)
