"""ctypes binding of libmx.so (the C ABI in include/mx.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels. torch is
used for device memory and the current stream. If the library is missing this module raises;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx.so")

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_UNSUPPORTED, MX_ERR_LAUNCH, MX_ERR_ARG = range(6)
MX_F32, MX_BF16 = 0, 1
MX_SCALE_FLOOR, MX_SCALE_CEIL = 0, 1
MX_ROUND_RNE, MX_ROUND_SR = 0, 1
MX_E4M3, MX_E5M2 = 0, 1

class mx_quant_opts(ctypes.Structure):
    _fields_ = [("scale_rule", ctypes.c_int32), ("round", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("sign_mask", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]


class MxError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libmx.so (build it with mxfp4_block_scaled_hadamard32_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m "
                          "mxfp4_block_scaled_hadamard32_amd.build (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    L.mx_quantize.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(mx_quant_opts), vp, vp, vp]
    L.mx_quantize_2d.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(mx_quant_opts), vp, vp, vp,
                                 vp, vp]
    L.mx_dequantize.argtypes = [vp, vp, i64, i64, i32, i32, u32, vp, vp]
    gemm_args = [vp, vp, i32, vp, vp, i32, i64, i64, i64, i32, i32, vp, i64, vp]
    for name in ("mx_gemm_fprop", "mx_gemm_dgrad", "mx_gemm_wgrad"):
        getattr(L, name).argtypes = gemm_args
    L.mx_gemm_fprop_quant.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, i32,
                                      ctypes.POINTER(mx_quant_opts), vp, vp, vp]
    L.mx_quantize_mxfp8.argtypes = [vp, i32, i64, i64, i64, i32, i32, ctypes.POINTER(mx_quant_opts),
                                    vp, vp, vp]
    L.mx_gemm_mxfp8.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, i32, i32, vp, i64, vp]
    L.mx_quantize_2d_blocks.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(mx_quant_opts),
                                        vp, vp, vp, vp, vp]
    L.mx_scale_mismatch_map.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp]
    for name in ("mx_quantize", "mx_quantize_2d", "mx_dequantize", "mx_gemm_fprop",
                 "mx_gemm_dgrad", "mx_gemm_wgrad", "mx_gemm_fprop_quant", "mx_quantize_mxfp8",
                 "mx_gemm_mxfp8", "mx_quantize_2d_blocks", "mx_scale_mismatch_map"):
        getattr(L, name).restype = ctypes.c_int
    L.mx_status_string.argtypes = [i32]
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_version.argtypes = []
    L.mx_version.restype = ctypes.c_int32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mx_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != MX_OK:
        raise MxError(status, what)
