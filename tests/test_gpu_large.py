"""Parity beyond 2^31 elements: 64-bit indexing of the quantizers (element indices and the
stochastic-rounding counters past 2^31) and of the GEMM's output offsets.

The quantize cases run a bf16 tensor of 65568 x 32768 = 2 148 532 224 elements (the first
element past 2^31 sits in row 65536) through the row and column kernels with the random-sign
Hadamard transform, ceil scale and stochastic rounding; the oracle checks the first rows, a middle
slab and the rows that straddle element 2^31, bit for bit. The GEMM case writes a 49152 x 49152
bf16 output (2.4 G elements) and is checked on sampled outputs that include the last rows.
"""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import assert_bytes_equal, check_gemm, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
THREADS = max(1, min(16, os.cpu_count() or 1))
ROWS, COLS = 65568, 32768
OPTS = dict(scale_rule=1, hadamard=1, sign_mask=0x2C6FE9B1, seed=1234)


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_hadamard32_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


@pytest.fixture(scope="module")
def big():
    assert ROWS * COLS > 2 ** 31 and (2 ** 31) // COLS == 65536
    x = wl.student_t3((ROWS, COLS), seed=77, device=DEV).to(torch.bfloat16)
    yield x, wl.host_input(x)
    del x
    torch.cuda.empty_cache()


SLABS = [(0, 64), (32768, 32832), (65472, 65568)]  # first rows, middle, across element 2^31


@pytest.mark.parametrize("rnd", [1, 0])
def test_quantize_rows_past_2g_elements(mx, orc, big, rnd):
    x, xh = big
    c, s = mx.mx_quantize(x, axis=1, round=rnd, **OPTS)
    torch.cuda.synchronize()
    for r0, r1 in SLABS:
        rc, rs = orc.quantize(xh, axis=1, round_mode=rnd, row_range=(r0, r1), nthreads=THREADS,
                              **OPTS)
        assert_bytes_equal(s[r0:r1], rs[r0:r1], f"scales rows {r0}:{r1}")
        assert_bytes_equal(c[r0:r1], rc[r0:r1], f"codes rows {r0}:{r1}")


def test_quantize_columns_past_2g_elements(mx, orc, big):
    x, xh = big
    c, s = mx.mx_quantize(x, axis=0, round=1, **OPTS)
    torch.cuda.synchronize()
    for r0, r1 in [(0, 64), (65504, 65568)]:  # the second range crosses element 2^31
        rc, rs = orc.quantize(xh, axis=0, round_mode=1, row_range=(r0, r1), nthreads=THREADS,
                              **OPTS)
        assert_bytes_equal(s[:, r0 // 32:r1 // 32], rs[:, r0 // 32:r1 // 32], f"scales_t {r0}:{r1}")
        assert_bytes_equal(c[:, r0 // 2:r1 // 2], rc[:, r0 // 2:r1 // 2], f"codes_t {r0}:{r1}")


def test_gemm_output_past_2g_elements(mx, orc):
    M = N = 49152
    K = 1024
    assert M * N > 2 ** 31
    a = wl.student_t3((M, K), seed=78, device=DEV).to(torch.bfloat16)
    aq, as_ = mx.mx_quantize(a, scale_rule=1, round=1, seed=5)
    del a
    b = wl.student_t3((N, K), seed=79, device=DEV).to(torch.bfloat16)
    bq, bs = mx.mx_quantize(b, scale_rule=1, round=1, seed=6)
    del b
    out = mx.mx_gemm_fprop(aq, as_, 1, bq, bs, 1, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1, M - 2, (2 ** 31) // N, (2 ** 31) // N + 1],
                                     rng.integers(0, M, 4)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 512)]))
    C, Cabs = orc.gemm(host(aq), host(as_), 1, host(bq), host(bs), 1, M, N, K, 0,
                       rows=rows, cols=cols)
    check_gemm(out, C, Cabs, rows=rows, cols=cols)
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("axis,rnd", [(0, 1), (0, 0), (1, 1)])
def test_quantize_leading_dimension_past_2g_bytes(mx, orc, axis, rnd):
    """A 32 x 64 slice of a tensor with 2^26 + 64 columns: the loads of row 28 start 3.5 GiB past
    the first (the column kernels' per-lane offsets, the row kernel's direct loads)."""
    ld = 2 ** 26 + 64
    full = torch.empty((32, ld), dtype=torch.bfloat16, device=DEV)
    src = wl.student_t3((32, 64), seed=81).to(torch.bfloat16)
    full[:, :64] = src.to(DEV)
    x = full[:, :64]
    c, s = mx.mx_quantize(x, axis=axis, round=rnd, **OPTS)
    torch.cuda.synchronize()
    rc, rs = orc.quantize(wl.host_input(src), axis=axis, round_mode=rnd, **OPTS)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")
    del full
    torch.cuda.empty_cache()


def test_quantize_mxfp8_columns_leading_dimension_past_2g_bytes(mx, orc):
    """The MXFP8 column kernel on the same 32 x 64 slice of a 2^26 + 64-column tensor."""
    ld = 2 ** 26 + 64
    full = torch.empty((32, ld), dtype=torch.bfloat16, device=DEV)
    src = wl.student_t3((32, 64), seed=82).to(torch.bfloat16)
    full[:, :64] = src.to(DEV)
    c, s = mx.mx_quantize_mxfp8(full[:, :64], fmt=0, axis=0, scale_rule=1, round=1, hadamard=1,
                                sign_mask=0x2C6FE9B1, seed=99)
    torch.cuda.synchronize()
    rc, rs = orc.quantize_fp8(wl.host_input(src), fmt=0, axis=0, scale_rule=1, round_mode=1,
                              hadamard=1, sign_mask=0x2C6FE9B1, seed=99)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")
    del full
    torch.cuda.empty_cache()
