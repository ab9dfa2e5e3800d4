"""CPU oracle for the MXFP4 block-scaled Hadamard-32 path — TEST INFRASTRUCTURE ONLY.

Only tests/, the package's smoke() check and bench.py's cpu_baseline leg may import this
module. It shares no code with the GPU library and never imports it.

Two parts:
  * the quantizer, dequantizer, Philox and Hadamard transform live in mx_oracle.c (plain
    scalar C, fp32 where the fp32 result decides a code), reached here through ctypes;
  * the GEMM is the plain definition written with numpy in float64: dequantize both operands
    exactly (E2M1 magnitude times a power of two is exact in double) and take the matrix
    product, plus the matrix product of absolute values for the error bound
    |gpu - C| <= 2^-20 * sum_k |a_k b_k|.

Pages (by title and section): "Stable FP4 Training via Transposition-Invariant Block
Quantization" — "Why FP4 training is the current frontier" (P = round(X/S), reconstruction
P*S), "The aha: transposition scrambles the blocks" (the layer's GEMMs in several
orientations), "The fix, and its supporting cast" (32x32 blocks, rounded-up scale, stochastic
rounding); "Block-Scaled MXFP4 With Stochastic Hadamard Rounding ..." paragraphs 1-2 (E8M0 per
32 E2M1 values, 32-element Walsh-Hadamard before packing); "Training LLMs with MXFP4" abstract
(stochastic rounding with a random Hadamard transform); "Pretraining large language models
with MXFP4" abstract (Fprop, Dgrad, Wgrad in FP4; deterministic Hadamard).
"""
from __future__ import annotations

import ctypes
import os
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

SCALE_FLOOR, SCALE_CEIL = 0, 1
ROUND_RNE, ROUND_SR = 0, 1
E4M3, E5M2 = 0, 1


class _Opts(ctypes.Structure):
    _fields_ = [("scale_rule", ctypes.c_int32), ("round", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("sign_mask", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build_oracle  # noqa: F401  (package-relative when imported as oracle.*)
            build_oracle.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_quantize_1d.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(_Opts), vp, vp,
                                      i64, i64]
        L.orc_quantize_2d.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(_Opts), vp, vp, vp,
                                      vp, i64, i64]
        L.orc_quantize_threaded.argtypes = [vp, i32, i64, i64, i64, i32, i32,
                                            ctypes.POINTER(_Opts), vp, vp, vp, vp, i64, i64, i32]
        L.orc_dequantize.argtypes = [vp, vp, i64, i64, i32, i32, ctypes.c_uint32, vp]
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_sr_field.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.orc_sr_field.restype = ctypes.c_uint32
        L.orc_fwht32.argtypes = [vp]
        L.orc_scale_exponent.argtypes = [ctypes.c_float, i32]
        L.orc_scale_exponent.restype = ctypes.c_int
        L.orc_e2m1_encode.argtypes = [ctypes.c_float, i32, ctypes.c_uint32]
        L.orc_e2m1_encode.restype = ctypes.c_int
        L.orc_e2m1_decode.argtypes = [i32]
        L.orc_e2m1_decode.restype = ctypes.c_float
        L.orc_e2m1_magnitude.argtypes = [i32]
        L.orc_e2m1_magnitude.restype = ctypes.c_float
        L.orc_quantize_2d_block.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(_Opts), vp,
                                            vp, vp, vp, i64, i64]
        L.orc_fp8_magnitude.argtypes = [i32, i32]
        L.orc_fp8_magnitude.restype = ctypes.c_double
        L.orc_fp8_decode.argtypes = [i32, i32]
        L.orc_fp8_decode.restype = ctypes.c_double
        L.orc_fp8_scale_exponent.argtypes = [ctypes.c_float, i32, i32]
        L.orc_fp8_scale_exponent.restype = ctypes.c_int
        L.orc_fp8_encode.argtypes = [ctypes.c_float, i32, i32, ctypes.c_uint32]
        L.orc_fp8_encode.restype = ctypes.c_int
        L.orc_quantize_fp8.argtypes = [vp, i32, i64, i64, i64, i32, i32, ctypes.POINTER(_Opts),
                                       vp, vp, i64, i64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _src(x: np.ndarray):
    """Returns (dtype code, ld) of a 2-D float32 or bf16-bit-pattern (uint16) array."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.dtype == np.float32:
        dt = 0
    elif x.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")
    if x.strides[1] != x.itemsize or x.strides[0] % x.itemsize:
        raise ValueError("rows must be contiguous")
    return dt, x.strides[0] // x.itemsize


def _opts(scale_rule, round_mode, hadamard, sign_mask, seed):
    return _Opts(int(scale_rule), int(round_mode), int(hadamard), int(sign_mask) & 0xFFFFFFFF,
                 int(seed) & 0xFFFFFFFFFFFFFFFF)


# ----------------------------------------------------------------------------------------------
# scalar primitives (exposed for the pinning tests)
# ----------------------------------------------------------------------------------------------
def e2m1_magnitude(m: int) -> float:
    return float(lib().orc_e2m1_magnitude(int(m)))


def e2m1_decode(code: int) -> float:
    return float(lib().orc_e2m1_decode(int(code)))


def e2m1_encode(v: float, round_mode: int = ROUND_RNE, r16: int = 0) -> int:
    return int(lib().orc_e2m1_encode(ctypes.c_float(v), int(round_mode), int(r16)))


def scale_exponent(amax: float, scale_rule: int) -> int:
    return int(lib().orc_scale_exponent(ctypes.c_float(amax), int(scale_rule)))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_field(seed: int, i: int) -> int:
    return int(lib().orc_sr_field(int(seed), int(i)))


def fwht32(x) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(x, dtype=np.float32).copy())
    assert y.shape == (32,)
    lib().orc_fwht32(_ptr(y))
    return y


def fp8_magnitude(m: int, fmt: int) -> float:
    return float(lib().orc_fp8_magnitude(int(m), int(fmt)))


def fp8_decode(code: int, fmt: int) -> float:
    return float(lib().orc_fp8_decode(int(code), int(fmt)))


def fp8_encode(v: float, fmt: int, round_mode: int = ROUND_RNE, r16: int = 0) -> int:
    return int(lib().orc_fp8_encode(ctypes.c_float(v), int(fmt), int(round_mode), int(r16)))


def fp8_scale_exponent(amax: float, scale_rule: int, fmt: int) -> int:
    return int(lib().orc_fp8_scale_exponent(ctypes.c_float(amax), int(scale_rule), int(fmt)))


# ----------------------------------------------------------------------------------------------
# tensor quantizers
# ----------------------------------------------------------------------------------------------
def quantize(x: np.ndarray, axis: int = 1, scale_rule: int = SCALE_FLOOR,
             round_mode: int = ROUND_RNE, hadamard: int = 0, sign_mask: int = 0, seed: int = 0,
             row_range=None, nthreads: int = 1):
    """1x32 quantize. axis=1: codes [rows][cols/2], scales [rows][cols/32].
    axis=0: codes [cols][rows/2], scales [cols][rows/32] (layout of the transpose).
    row_range=(r0, r1) restricts the work to those source rows (outputs stay full size,
    untouched entries are zero)."""
    dt, ld = _src(x)
    rows, cols = x.shape
    if axis == 1:
        if cols % 32:
            raise ValueError("cols must be a multiple of 32")
        codes = np.zeros((rows, cols // 2), dtype=np.uint8)
        scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    else:
        if rows % 32:
            raise ValueError("rows must be a multiple of 32")
        codes = np.zeros((cols, rows // 2), dtype=np.uint8)
        scales = np.zeros((cols, rows // 32), dtype=np.uint8)
    r0, r1 = (0, rows) if row_range is None else row_range
    o = _opts(scale_rule, round_mode, hadamard, sign_mask, seed)
    lib().orc_quantize_threaded(_ptr(x), dt, rows, cols, ld, axis, 0, ctypes.byref(o),
                                _ptr(codes), _ptr(scales), None, None, r0, r1, int(nthreads))
    return codes, scales


def quantize_2d(x: np.ndarray, scale_rule: int = SCALE_CEIL, round_mode: int = ROUND_RNE,
                seed: int = 0, row_range=None, nthreads: int = 1):
    """32x32 quantize: codes [rows][cols/2], scales [rows/32][cols/32], codes_t [cols][rows/2],
    scales_t [cols/32][rows/32]."""
    dt, ld = _src(x)
    rows, cols = x.shape
    if rows % 32 or cols % 32:
        raise ValueError("rows and cols must be multiples of 32")
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows // 32, cols // 32), dtype=np.uint8)
    codes_t = np.zeros((cols, rows // 2), dtype=np.uint8)
    scales_t = np.zeros((cols // 32, rows // 32), dtype=np.uint8)
    r0, r1 = (0, rows) if row_range is None else row_range
    o = _opts(scale_rule, round_mode, 0, 0, seed)
    lib().orc_quantize_threaded(_ptr(x), dt, rows, cols, ld, 1, 1, ctypes.byref(o),
                                _ptr(codes), _ptr(scales), _ptr(codes_t), _ptr(scales_t), r0, r1,
                                int(nthreads))
    return codes, scales, codes_t, scales_t


def quantize_2d_block(x: np.ndarray, block: int, scale_rule: int = SCALE_CEIL,
                      round_mode: int = ROUND_RNE, seed: int = 0, row_range=None):
    """BxB quantize (block 8, 32 or 64): codes [rows][cols/2], scales [rows/B][cols/B], codes_t
    [cols][rows/2], scales_t [cols/B][rows/B]."""
    dt, ld = _src(x)
    rows, cols = x.shape
    B = int(block)
    if B not in (8, 32, 64) or rows % B or cols % B:
        raise ValueError("block must be 8, 32 or 64 and divide both dimensions")
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows // B, cols // B), dtype=np.uint8)
    codes_t = np.zeros((cols, rows // 2), dtype=np.uint8)
    scales_t = np.zeros((cols // B, rows // B), dtype=np.uint8)
    r0, r1 = (0, rows) if row_range is None else row_range
    o = _opts(scale_rule, round_mode, 0, 0, seed)
    lib().orc_quantize_2d_block(_ptr(x), dt, rows, cols, ld, B, ctypes.byref(o), _ptr(codes),
                                _ptr(scales), _ptr(codes_t), _ptr(scales_t), r0, r1)
    return codes, scales, codes_t, scales_t


def scale_mismatch_map(x: np.ndarray, scale_rule: int = SCALE_FLOOR) -> np.ndarray:
    """Scale-difference map of 1x32 blocking ("Stable FP4 Training via Transposition-Invariant
    Block Quantization", "The aha: transposition scrambles the blocks", Figure 1): for every
    element, the scale exponent of its block along the row (how X enters the forward product)
    minus that of its block down the column (how X enters the transposed product), saturated
    to [-127, 127] as int8; -128 where either block's maximum is not finite."""
    rows, cols = x.shape
    _, s_row = quantize(x, axis=1, scale_rule=scale_rule)
    _, s_col = quantize(x, axis=0, scale_rule=scale_rule)
    er = np.repeat(s_row.astype(np.int32), 32, axis=1)          # [rows][cols]
    ec = np.repeat(s_col.astype(np.int32), 32, axis=1).T        # [cols][rows] -> [rows][cols]
    d = np.clip(er - ec, -127, 127)
    d[(er == 255) | (ec == 255)] = -128
    return d.astype(np.int8)


def dequantize(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int, block_rows: int = 1,
               inv_hadamard: int = 0, sign_mask: int = 0) -> np.ndarray:
    """fp32 reconstruction code * 2^(scale-127), optionally rotated back by (1/32) D H."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    assert codes.size == rows * cols // 2
    assert scales.size == (rows // block_rows) * (cols // 32)
    out = np.empty((rows, cols), dtype=np.float32)
    lib().orc_dequantize(_ptr(codes), _ptr(scales), rows, cols, block_rows, int(inv_hadamard),
                         int(sign_mask) & 0xFFFFFFFF, _ptr(out))
    return out


def quantize_fp8(x: np.ndarray, fmt: int = E4M3, axis: int = 1, scale_rule: int = SCALE_FLOOR,
                 round_mode: int = ROUND_RNE, hadamard: int = 0, sign_mask: int = 0,
                 seed: int = 0, row_range=None):
    """1x32 MXFP8 quantize, one code byte per element. axis=1: codes [rows][cols], scales
    [rows][cols/32]; axis=0: codes [cols][rows], scales [cols][rows/32]."""
    dt, ld = _src(x)
    rows, cols = x.shape
    if (cols if axis == 1 else rows) % 32:
        raise ValueError("the blocked dimension must be a multiple of 32")
    if axis == 1:
        codes = np.zeros((rows, cols), dtype=np.uint8)
        scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    else:
        codes = np.zeros((cols, rows), dtype=np.uint8)
        scales = np.zeros((cols, rows // 32), dtype=np.uint8)
    r0, r1 = (0, rows) if row_range is None else row_range
    o = _opts(scale_rule, round_mode, hadamard, sign_mask, seed)
    lib().orc_quantize_fp8(_ptr(x), dt, rows, cols, ld, axis, int(fmt), ctypes.byref(o),
                           _ptr(codes), _ptr(scales), r0, r1)
    return codes, scales


# ----------------------------------------------------------------------------------------------
# GEMM: plain definition in float64
# ----------------------------------------------------------------------------------------------
def _magnitudes_f64() -> np.ndarray:
    return np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)


def dequantize_f64(codes: np.ndarray, scales: np.ndarray, rows: int, k: int, g: int,
                   row_index=None) -> np.ndarray:
    """Exact float64 values of a K-major packed operand (codes [rows][k/2]). g = 1: scales
    [rows][k/32]; g = 32: scales [rows/32][k/32]. row_index selects a subset of rows."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(rows, k // 2)
    scales = np.asarray(scales, dtype=np.uint8).reshape(rows // g, k // 32)
    ridx = np.arange(rows) if row_index is None else np.asarray(row_index)
    c = codes[ridx]
    nib = np.empty((len(ridx), k), dtype=np.uint8)
    nib[:, 0::2] = c & 0x0F
    nib[:, 1::2] = c >> 4
    vals = _magnitudes_f64()[nib]
    s = scales[ridx // g].astype(np.int64)
    pw = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return vals * np.repeat(pw, 32, axis=1)


def gemm(aq, as_, ga: int, bq, bs, gb: int, M: int, N: int, K: int, alpha_exp: int = 0,
         rows=None, cols=None, timings=None):
    """C[m][n] = 2^alpha * sum_k A[m][k] B[n][k] in float64, and the matching sum of |a_k b_k|.
    rows / cols optionally select output rows / columns (sampled checks). A dict passed as
    timings receives the seconds spent dequantizing ("dequant_s") and in the two products
    ("matmul_s")."""
    t0 = time.perf_counter()
    A = dequantize_f64(aq, as_, M, K, ga, rows)
    B = dequantize_f64(bq, bs, N, K, gb, cols)
    t1 = time.perf_counter()
    f = 2.0 ** alpha_exp
    C = (A @ B.T) * f
    Cabs = (np.abs(A) @ np.abs(B).T) * f
    if timings is not None:
        timings["dequant_s"] = t1 - t0
        timings["matmul_s"] = time.perf_counter() - t1
    return C, Cabs


def _fp8_values_f64(fmt: int) -> np.ndarray:
    return np.array([fp8_decode(c, fmt) for c in range(256)], dtype=np.float64)


def dequantize_fp8_f64(codes: np.ndarray, scales: np.ndarray, rows: int, k: int, fmt: int,
                       row_index=None) -> np.ndarray:
    """Exact float64 values of a K-major MXFP8 operand: codes [rows][k], scales [rows][k/32]."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(rows, k)
    scales = np.asarray(scales, dtype=np.uint8).reshape(rows, k // 32)
    ridx = np.arange(rows) if row_index is None else np.asarray(row_index)
    vals = _fp8_values_f64(fmt)[codes[ridx]]
    s = scales[ridx].astype(np.int64)
    pw = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return vals * np.repeat(pw, 32, axis=1)


def gemm_fp8(aq, as_, afmt: int, bq, bs, bfmt: int, M: int, N: int, K: int, alpha_exp: int = 0,
             rows=None, cols=None):
    """MXFP8 C[m][n] = 2^alpha * sum_k A[m][k] B[n][k] in float64 and sum |a_k b_k| (as gemm)."""
    A = dequantize_fp8_f64(aq, as_, M, K, afmt, rows)
    B = dequantize_fp8_f64(bq, bs, N, K, bfmt, cols)
    f = 2.0 ** alpha_exp
    return (A @ B.T) * f, (np.abs(A) @ np.abs(B).T) * f
