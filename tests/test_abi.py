"""The C ABI library loads, exports every entry point declared in include/mx.h, and rejects bad
arguments with the documented status codes before touching the GPU (so these run on a host with
no GPU: validation happens before any HIP call, and no pointer here is dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from mxfp4_block_scaled_hadamard32_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmx.so not built (run __graft_entry__.build())")
    return _lib.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"mx_quantize", "mx_quantize_2d", "mx_dequantize", "mx_gemm_fprop", "mx_gemm_dgrad",
            "mx_gemm_wgrad"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.mx_version() >= 100
    from mxfp4_block_scaled_hadamard32_amd import _lib
    for s in range(6):
        assert _lib.status_string(s).startswith("MX_")


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced on the error paths below


def opts(**kw):
    from mxfp4_block_scaled_hadamard32_amd._lib import mx_quant_opts
    o = mx_quant_opts(0, 0, 0, 0, 0)
    for k, v in kw.items():
        setattr(o, k, v)
    return ctypes.byref(o)


def test_quantize_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    q = L.mx_quantize
    assert q(FAKE, 1, 64, 48, 48, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_SHAPE   # cols % 32
    assert q(FAKE, 1, 48, 64, 64, 0, opts(), FAKE, FAKE, None) == m.MX_ERR_SHAPE   # rows % 32
    assert q(FAKE, 1, 64, 64, 32, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_SHAPE   # ld < cols
    assert q(FAKE, 1, 64, 64, 68, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_SHAPE   # ld*2 % 16
    assert q(FAKE, 7, 64, 64, 64, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_ARG     # dtype
    assert q(FAKE, 1, 64, 64, 64, 2, opts(), FAKE, FAKE, None) == m.MX_ERR_ARG     # axis
    assert q(FAKE, 1, 64, 64, 64, 1, opts(round=5), FAKE, FAKE, None) == m.MX_ERR_ARG
    assert q(FAKE, 1, 64, 64, 64, 1, None, FAKE, FAKE, None) == m.MX_ERR_NULL
    assert q(None, 1, 64, 64, 64, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_NULL
    assert q(FAKE, 1, 64, 64, 64, 1, opts(), None, FAKE, None) == m.MX_ERR_NULL
    assert q(ctypes.c_void_p(0x10008), 1, 64, 64, 64, 1, opts(), FAKE, FAKE, None) == m.MX_ERR_ARG
    # codes: 16 bytes for both axes (a lane writes a block's 16 code bytes at once)
    assert q(FAKE, 1, 64, 64, 64, 1, opts(), ctypes.c_void_p(0x10008), FAKE, None) == m.MX_ERR_ARG
    assert q(FAKE, 1, 64, 64, 64, 0, opts(), ctypes.c_void_p(0x10004), FAKE, None) == m.MX_ERR_ARG
    # empty tensors are fine and launch nothing
    assert q(None, 1, 0, 64, 64, 1, opts(), None, None, None) == m.MX_OK
    assert q(None, 1, 32, 0, 0, 0, opts(), None, None, None) == m.MX_OK


def test_quantize_2d_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    q = L.mx_quantize_2d
    assert q(FAKE, 1, 64, 64, 64, opts(hadamard=1), FAKE, FAKE, None, None, None) == m.MX_ERR_UNSUPPORTED
    assert q(FAKE, 1, 48, 64, 64, opts(), FAKE, FAKE, None, None, None) == m.MX_ERR_SHAPE
    assert q(FAKE, 1, 64, 64, 64, opts(), FAKE, FAKE, FAKE, None, None) == m.MX_ERR_NULL
    assert q(None, 1, 0, 0, 0, opts(), None, None, None, None, None) == m.MX_OK


def test_dequantize_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    d = L.mx_dequantize
    assert d(FAKE, FAKE, 4, 48, 1, 0, 0, FAKE, None) == m.MX_ERR_SHAPE
    assert d(FAKE, FAKE, 64, 64, 2, 0, 0, FAKE, None) == m.MX_ERR_ARG
    assert d(FAKE, FAKE, 64, 64, 32, 1, 0, FAKE, None) == m.MX_ERR_UNSUPPORTED
    assert d(FAKE, FAKE, 40, 64, 32, 0, 0, FAKE, None) == m.MX_ERR_SHAPE
    assert d(None, FAKE, 64, 64, 1, 0, 0, FAKE, None) == m.MX_ERR_NULL
    assert d(None, None, 0, 64, 1, 0, 0, None, None) == m.MX_OK


@pytest.mark.parametrize("name", ["mx_gemm_fprop", "mx_gemm_dgrad", "mx_gemm_wgrad"])
def test_gemm_argument_errors(L, name):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    g = getattr(L, name)
    ok = dict(M=64, N=64, K=64)

    def call(M=64, N=64, K=64, ga=1, gb=1, alpha=0, dt=1, c=FAKE, ldc=64, a=FAKE):
        return g(a, FAKE, ga, FAKE, FAKE, gb, M, N, K, alpha, dt, c, ldc, None)
    assert call(M=48) == m.MX_ERR_SHAPE
    assert call(K=40) == m.MX_ERR_SHAPE
    assert call(ldc=60) == m.MX_ERR_SHAPE
    assert call(ldc=72 + 4) == m.MX_ERR_SHAPE
    assert call(ga=2) == m.MX_ERR_ARG
    assert call(dt=3) == m.MX_ERR_ARG
    assert call(alpha=200) == m.MX_ERR_ARG
    assert call(c=None) == m.MX_ERR_NULL
    assert call(a=None) == m.MX_ERR_NULL
    assert call(M=0) == m.MX_OK and call(N=0, c=None) == m.MX_OK
    del ok


def test_gemm_fprop_quant_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    g = L.mx_gemm_fprop_quant

    def call(T=64, N=64, K=128, gx=1, gw=1, alpha=0, o=None, yq=FAKE, ys=FAKE, xq=FAKE):
        return g(xq, FAKE, gx, FAKE, FAKE, gw, T, N, K, alpha, opts() if o is None else o, yq, ys,
                 None)
    assert call(T=48) == m.MX_ERR_SHAPE
    assert call(K=40) == m.MX_ERR_SHAPE
    assert call(K=96) == m.MX_ERR_UNSUPPORTED   # the epilogue runs in the 128-k streaming kernels
    assert call(gx=2) == m.MX_ERR_ARG
    assert call(alpha=-200) == m.MX_ERR_ARG
    assert call(o=opts(scale_rule=3)) == m.MX_ERR_ARG
    assert g(FAKE, FAKE, 1, FAKE, FAKE, 1, 64, 64, 128, 0, None, FAKE, FAKE, None) == m.MX_ERR_NULL
    assert call(ys=None) == m.MX_ERR_NULL
    assert call(xq=None) == m.MX_ERR_NULL
    assert call(yq=ctypes.c_void_p(0x10002)) == m.MX_ERR_ARG
    assert call(T=0, yq=None, ys=None) == m.MX_OK


def test_quantize_mxfp8_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    q = L.mx_quantize_mxfp8

    def call(x=FAKE, dt=1, rows=64, cols=64, ld=64, axis=1, fmt=0, o=None, codes=FAKE, scales=FAKE):
        return q(x, dt, rows, cols, ld, axis, fmt, opts() if o is None else o, codes, scales, None)
    assert call(cols=48, ld=48) == m.MX_ERR_SHAPE             # cols % 32 along rows
    assert call(rows=48, axis=0) == m.MX_ERR_SHAPE            # rows % 32 down columns
    assert call(rows=64, cols=36, ld=40, axis=0) == m.MX_ERR_SHAPE  # cols % 8 down columns
    assert call(fmt=2) == m.MX_ERR_ARG
    assert call(axis=3) == m.MX_ERR_ARG
    assert call(o=opts(hadamard=2)) == m.MX_ERR_ARG
    assert q(FAKE, 1, 64, 64, 64, 1, 0, None, FAKE, FAKE, None) == m.MX_ERR_NULL
    assert call(scales=None) == m.MX_ERR_NULL
    assert call(codes=ctypes.c_void_p(0x10004)) == m.MX_ERR_ARG          # 8-byte rule (rows)
    assert call(codes=ctypes.c_void_p(0x10008), axis=0) == m.MX_ERR_ARG  # 16-byte rule (cols)
    assert call(x=None, rows=0, codes=None, scales=None) == m.MX_OK


def test_gemm_mxfp8_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    g = L.mx_gemm_mxfp8

    def call(M=64, N=64, K=128, af=0, bf=1, alpha=0, dt=1, c=FAKE, ldc=64, a=FAKE):
        return g(a, FAKE, af, FAKE, FAKE, bf, M, N, K, alpha, dt, c, ldc, None)
    assert call(M=40) == m.MX_ERR_SHAPE
    assert call(K=48) == m.MX_ERR_SHAPE
    assert call(K=96) == m.MX_ERR_UNSUPPORTED   # 128-k stages
    assert call(ldc=66) == m.MX_ERR_SHAPE
    assert call(af=2) == m.MX_ERR_ARG and call(bf=-1) == m.MX_ERR_ARG
    assert call(dt=5) == m.MX_ERR_ARG
    assert call(alpha=128) == m.MX_ERR_ARG
    assert call(c=None) == m.MX_ERR_NULL
    assert call(a=None) == m.MX_ERR_NULL
    assert call(c=ctypes.c_void_p(0x10008)) == m.MX_ERR_ARG
    assert call(N=0, c=None) == m.MX_OK


def test_quantize_2d_blocks_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    q = L.mx_quantize_2d_blocks

    def call(rows=128, cols=128, ld=128, block=64, o=None, codes=FAKE, scales=FAKE, ct=None, st=None):
        return q(FAKE, 1, rows, cols, ld, block, opts() if o is None else o, codes, scales, ct, st,
                 None)
    assert call(block=16) == m.MX_ERR_ARG
    assert call(rows=96) == m.MX_ERR_SHAPE                 # 64x64 needs multiples of 64
    assert call(block=8, cols=40, ld=48) == m.MX_ERR_SHAPE  # multiples of 32 even for 8x8
    assert call(o=opts(hadamard=1)) == m.MX_ERR_UNSUPPORTED
    assert call(ct=FAKE) == m.MX_ERR_NULL
    assert call(scales=ctypes.c_void_p(0x10002)) == m.MX_ERR_ARG
    assert call(codes=None) == m.MX_ERR_NULL
    assert call(rows=0, codes=None, scales=None) == m.MX_OK


def test_scale_mismatch_map_argument_errors(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    f = L.mx_scale_mismatch_map
    assert f(FAKE, 1, 64, 48, 48, 0, FAKE, None) == m.MX_ERR_SHAPE
    assert f(FAKE, 1, 40, 64, 64, 0, FAKE, None) == m.MX_ERR_SHAPE
    assert f(FAKE, 1, 64, 64, 64, 2, FAKE, None) == m.MX_ERR_ARG
    assert f(FAKE, 3, 64, 64, 64, 0, FAKE, None) == m.MX_ERR_ARG
    assert f(FAKE, 1, 64, 64, 64, 0, None, None) == m.MX_ERR_NULL
    assert f(FAKE, 1, 64, 64, 64, 0, ctypes.c_void_p(0x10004), None) == m.MX_ERR_ARG
    assert f(None, 1, 0, 64, 64, 0, None, None) == m.MX_OK


def test_gemm_64_row_granularity_needs_whole_tiles(L):
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    g = L.mx_gemm_fprop
    assert g(FAKE, FAKE, 64, FAKE, FAKE, 1, 96, 64, 64, 0, 1, FAKE, 64, None) == m.MX_ERR_SHAPE
    assert g(FAKE, FAKE, 1, FAKE, FAKE, 64, 64, 96, 64, 0, 1, FAKE, 96, None) == m.MX_ERR_SHAPE
    assert g(FAKE, FAKE, 16, FAKE, FAKE, 1, 64, 64, 64, 0, 1, FAKE, 64, None) == m.MX_ERR_ARG


def test_gemm_rejects_operand_tiles_beyond_32_bit_offsets(L):
    """A 256-row operand tile must stay below 2 GiB (the kernels' 32-bit buffer offsets): K = 2^24
    is refused before anything is launched."""
    from mxfp4_block_scaled_hadamard32_amd import _lib as m
    K = 1 << 24
    assert L.mx_gemm_fprop(FAKE, FAKE, 1, FAKE, FAKE, 1, 256, 256, K, 0, 1, FAKE, 256,
                           None) == m.MX_ERR_LAUNCH
    assert L.mx_gemm_mxfp8(FAKE, FAKE, 0, FAKE, FAKE, 0, 256, 256, K // 2, 0, 1, FAKE, 256,
                           None) == m.MX_ERR_LAUNCH


def test_probe_library_exports_its_declaration():
    """libmx_probe.so (the matrix-core ceiling probe) exports what include/mx_probe.h declares
    and rejects bad arguments before any HIP call."""
    from mxfp4_block_scaled_hadamard32_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        pytest.skip("libmx_probe.so not built (run __graft_entry__.build())")
    P = ctypes.CDLL(hip_build.PROBE_LIB)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mx_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mx_probe_mfma_fp4"]
    for n in names:
        assert hasattr(P, n), n
    f = P.mx_probe_mfma_fp4
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int32
    assert f(0, 10, 1, FAKE, None) != 0
    assert f(4, 0, 1, FAKE, None) != 0
    assert f(4, 10, 1, None, None) != 0
