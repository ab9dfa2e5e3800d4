"""MXFP4 block-scaled Hadamard-32 hot path for AMD MI355X (gfx950).

Python face of the C ABI in include/mx.h (libmx.so). Each function marshals torch tensors (device
memory, current HIP stream) into one library call; the quantizer, dequantizer and GEMMs all run
in the library's HIP kernels.

  mx_quantize     1x32 blocks, optional 32-point Hadamard rotation with random signs, floor or
                  ceil E8M0 scale, RNE or Philox stochastic rounding, packed E2M1 codes
  mx_quantize_2d  32x32 transposition-invariant blocks, plus the transposed K-major copy
  mx_dequantize   codes * 2^(scale-127), optional inverse rotation
  mx_gemm_fprop / mx_gemm_dgrad / mx_gemm_wgrad   block-scaled MXFP4 GEMMs, fp32 accumulate
  mx_gemm_fprop_quant   Fprop whose output tile is quantized (1x32 along N) in the epilogue
  mx_quantize_2d_blocks   8x8, 32x32 or 64x64 tiles (64x64 scales in the GEMM layout, g = 64)
  mx_scale_mismatch_map   per-element scale exponent of the row block minus the column block
  mx_quantize_mxfp8 / mx_gemm_mxfp8   MXFP8 (E4M3 / E5M2 elements, the same E8M0 block scales)
                  quantize and block-scaled GEMM, for the query / key projections
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MX_BF16, MX_E4M3, MX_E5M2, MX_F32, MX_ROUND_RNE, MX_ROUND_SR, MX_SCALE_CEIL,
                   MX_SCALE_FLOOR, MxError, check, lib, mx_quant_opts)

__all__ = ["mx_quantize", "mx_quantize_2d", "mx_dequantize", "mx_gemm_fprop", "mx_gemm_dgrad",
           "mx_gemm_wgrad", "mx_gemm_fprop_quant", "mx_quantize_mxfp8", "mx_gemm_mxfp8", "mx_quantize_2d_blocks",
           "mx_scale_mismatch_map", "MxError",
           "MX_SCALE_FLOOR", "MX_SCALE_CEIL", "MX_ROUND_RNE", "MX_ROUND_SR", "MX_E4M3", "MX_E5M2",
           "lib"]


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return MX_BF16
    if x.dtype == torch.float32:
        return MX_F32
    raise TypeError("mx_quantize takes bfloat16 or float32 input")


def _src(x: torch.Tensor):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("expected a 2-D CUDA tensor with contiguous rows")
    return x.shape[0], x.shape[1], x.stride(0)


def _buf(t, name: str, shape, dtypes, device, rows_only: bool = False):
    """Checks a caller-supplied buffer before its address goes to a kernel: a tensor on `device`
    with one of `dtypes` and exactly `shape`, contiguous (rows_only: only its rows contiguous,
    for outputs with a leading dimension). Raises ValueError / TypeError otherwise."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if rows_only:
        if t.dim() != 2 or (t.numel() > 0 and (t.stride(1) != 1 or t.stride(0) < shape[1])):
            raise ValueError(f"{name} must have contiguous rows")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_U8 = (torch.uint8,)


def _codes_out(t, name, shape, device):
    """A code or scale output: allocated when None, else checked."""
    if t is None:
        return torch.empty(shape, dtype=torch.uint8, device=device)
    return _buf(t, name, shape, _U8, device)


def _operand(q, s, g: int, name: str, k_bytes_per_elem: float = 0.5):
    """A packed GEMM operand (codes [rows][K * bytes per element], scales [rows / g][K / 32])
    on a CUDA device; returns (rows, K)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or not q.is_cuda:
        raise ValueError(f"{name} codes must be a 2-D CUDA tensor")
    rows = q.shape[0]
    K = int(round(q.shape[1] / k_bytes_per_elem))
    _buf(q, f"{name} codes", tuple(q.shape), _U8, q.device)
    if int(g) not in (1, 32, 64) or rows % int(g):
        raise ValueError(f"{name} scale granularity {g} does not divide its {rows} rows")
    _buf(s, f"{name} scales", (rows // int(g), K // 32), _U8, q.device)
    return rows, K


def _opts(scale_rule, round, hadamard, sign_mask, seed) -> mx_quant_opts:
    return mx_quant_opts(int(scale_rule), int(round), int(hadamard), int(sign_mask) & 0xFFFFFFFF,
                         int(seed) & 0xFFFFFFFFFFFFFFFF)


def mx_quantize(x: torch.Tensor, axis: int = 1, scale_rule: int = MX_SCALE_FLOOR,
                round: int = MX_ROUND_RNE, hadamard: int = 0, sign_mask: int = 0, seed: int = 0,
                codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                stream=None):
    """1x32 quantize. axis=1 -> codes [rows][cols/2], scales [rows][cols/32];
    axis=0 -> codes [cols][rows/2], scales [cols][rows/32] (K-major layout of x^T)."""
    rows, cols, ld = _src(x)
    shape_c = (rows, cols // 2) if axis == 1 else (cols, rows // 2)
    shape_s = (rows, cols // 32) if axis == 1 else (cols, rows // 32)
    codes = _codes_out(codes, "codes", shape_c, x.device)
    scales = _codes_out(scales, "scales", shape_s, x.device)
    o = _opts(scale_rule, round, hadamard, sign_mask, seed)
    check(lib().mx_quantize(_ptr(x), _dtype_code(x), rows, cols, ld, int(axis), ctypes.byref(o),
                            _ptr(codes), _ptr(scales), _stream(stream)), "mx_quantize")
    return codes, scales


def mx_quantize_2d(x: torch.Tensor, scale_rule: int = MX_SCALE_CEIL, round: int = MX_ROUND_RNE,
                   seed: int = 0, transposed: bool = True, codes=None, scales=None, codes_t=None,
                   scales_t=None, stream=None):
    """32x32 quantize -> (codes [rows][cols/2], scales [rows/32][cols/32],
    codes_t [cols][rows/2], scales_t [cols/32][rows/32]); the last two are None unless
    transposed."""
    rows, cols, ld = _src(x)
    dev = x.device
    codes = _codes_out(codes, "codes", (rows, cols // 2), dev)
    scales = _codes_out(scales, "scales", (rows // 32, cols // 32), dev)
    if transposed:
        codes_t = _codes_out(codes_t, "codes_t", (cols, rows // 2), dev)
        scales_t = _codes_out(scales_t, "scales_t", (cols // 32, rows // 32), dev)
    else:
        codes_t = scales_t = None
    o = _opts(scale_rule, round, 0, 0, seed)
    check(lib().mx_quantize_2d(_ptr(x), _dtype_code(x), rows, cols, ld, ctypes.byref(o),
                               _ptr(codes), _ptr(scales), _ptr(codes_t), _ptr(scales_t),
                               _stream(stream)), "mx_quantize_2d")
    return codes, scales, codes_t, scales_t


def mx_dequantize(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int,
                  block_rows: int = 1, inv_hadamard: int = 0, sign_mask: int = 0,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if not isinstance(codes, torch.Tensor) or not codes.is_cuda:
        raise ValueError("codes must be a CUDA tensor")
    rows, cols, block_rows = int(rows), int(cols), int(block_rows)
    if block_rows not in (1, 32) or rows % block_rows:
        raise ValueError("block_rows must be 1 or 32 and divide rows")
    dev = codes.device
    _buf(codes, "codes", (rows, cols // 2), _U8, dev)
    _buf(scales, "scales", (rows // block_rows, cols // 32), _U8, dev)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    _buf(out, "out", (rows, cols), (torch.float32,), dev)
    check(lib().mx_dequantize(_ptr(codes), _ptr(scales), rows, cols, int(block_rows),
                              int(inv_hadamard), int(sign_mask) & 0xFFFFFFFF, _ptr(out),
                              _stream(stream)), "mx_dequantize")
    return out


def _out(out, rows, cols, out_dtype, device):
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=device)
    _buf(out, "out", (rows, cols), (torch.bfloat16, torch.float32), device, rows_only=True)
    code = MX_BF16 if out.dtype == torch.bfloat16 else MX_F32
    return out, code


def _gemm(name, aq, as_, ga, bq, bs, gb, alpha_exp, out_dtype, out, stream):
    M, K = _operand(aq, as_, ga, "A")
    N, Kb = _operand(bq, bs, gb, "B")
    if Kb != K or bq.device != aq.device:
        raise ValueError("operands disagree on the reduction length or the device")
    out, code = _out(out, M, N, out_dtype, aq.device)
    check(getattr(lib(), name)(_ptr(aq), _ptr(as_), int(ga), _ptr(bq), _ptr(bs), int(gb), M, N, K,
                               int(alpha_exp), code, _ptr(out), out.stride(0), _stream(stream)),
          name)
    return out


def mx_gemm_fprop(xq, xs, gx, wq, ws, gw, alpha_exp=0, out_dtype=torch.bfloat16, out=None,
                  stream=None):
    """Y[T][N] = 2^alpha sum_k X[t][k] W[n][k]; xq [T][K/2], wq [N][K/2]."""
    return _gemm("mx_gemm_fprop", xq, xs, gx, wq, ws, gw, alpha_exp, out_dtype, out, stream)


def mx_gemm_dgrad(dyq, dys, gdy, wtq, wts, gwt, alpha_exp=0, out_dtype=torch.bfloat16, out=None,
                  stream=None):
    """dX[T][K] = 2^alpha sum_n dY[t][n] Wt[k][n]; dyq [T][N/2], wtq [K][N/2]."""
    return _gemm("mx_gemm_dgrad", dyq, dys, gdy, wtq, wts, gwt, alpha_exp, out_dtype, out, stream)


def mx_gemm_wgrad(dytq, dyts, gdy, xtq, xts, gx, alpha_exp=0, out_dtype=torch.bfloat16, out=None,
                  stream=None):
    """dW[N][K] = 2^alpha sum_t dYt[n][t] Xt[k][t]; dytq [N][T/2], xtq [K][T/2]."""
    return _gemm("mx_gemm_wgrad", dytq, dyts, gdy, xtq, xts, gx, alpha_exp, out_dtype, out, stream)


def mx_gemm_fprop_quant(xq, xs, gx, wq, ws, gw, alpha_exp=0, scale_rule=MX_SCALE_FLOOR,
                        round=MX_ROUND_RNE, hadamard=0, sign_mask=0, seed=0, codes=None,
                        scales=None, stream=None):
    """Y = 2^alpha X W^T in fp32, quantized in the GEMM epilogue along its rows (1x32 blocks
    along N, options as for mx_quantize) -> (codes [T][N/2], scales [T][N/32])."""
    T, K = _operand(xq, xs, gx, "X")
    N, Kw = _operand(wq, ws, gw, "W")
    if Kw != K or wq.device != xq.device:
        raise ValueError("operands disagree on the reduction length or the device")
    codes = _codes_out(codes, "codes", (T, N // 2), xq.device)
    scales = _codes_out(scales, "scales", (T, N // 32), xq.device)
    o = _opts(scale_rule, round, hadamard, sign_mask, seed)
    check(lib().mx_gemm_fprop_quant(_ptr(xq), _ptr(xs), int(gx), _ptr(wq), _ptr(ws), int(gw), T, N,
                                    K, int(alpha_exp), ctypes.byref(o), _ptr(codes), _ptr(scales),
                                    _stream(stream)), "mx_gemm_fprop_quant")
    return codes, scales


def mx_quantize_mxfp8(x: torch.Tensor, fmt: int = MX_E4M3, axis: int = 1,
                      scale_rule: int = MX_SCALE_FLOOR, round: int = MX_ROUND_RNE,
                      hadamard: int = 0, sign_mask: int = 0, seed: int = 0,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                      stream=None):
    """1x32 MXFP8 quantize (fmt MX_E4M3 or MX_E5M2). axis=1 -> codes [rows][cols] (one byte per
    element), scales [rows][cols/32]; axis=0 -> codes [cols][rows], scales [cols][rows/32]."""
    rows, cols, ld = _src(x)
    shape_c = (rows, cols) if axis == 1 else (cols, rows)
    shape_s = (rows, cols // 32) if axis == 1 else (cols, rows // 32)
    codes = _codes_out(codes, "codes", shape_c, x.device)
    scales = _codes_out(scales, "scales", shape_s, x.device)
    o = _opts(scale_rule, round, hadamard, sign_mask, seed)
    check(lib().mx_quantize_mxfp8(_ptr(x), _dtype_code(x), rows, cols, ld, int(axis), int(fmt),
                                  ctypes.byref(o), _ptr(codes), _ptr(scales), _stream(stream)),
          "mx_quantize_mxfp8")
    return codes, scales


def mx_gemm_mxfp8(aq, as_, afmt, bq, bs, bfmt, alpha_exp=0, out_dtype=torch.bfloat16, out=None,
                  stream=None):
    """C[M][N] = 2^alpha sum_k A[m][k] B[n][k]; aq [M][K], bq [N][K] MXFP8 codes of formats
    afmt / bfmt, scales [M][K/32], [N][K/32]."""
    M, K = _operand(aq, as_, 1, "A", 1.0)
    N, Kb = _operand(bq, bs, 1, "B", 1.0)
    if Kb != K or bq.device != aq.device:
        raise ValueError("operands disagree on the reduction length or the device")
    out, code = _out(out, M, N, out_dtype, aq.device)
    check(lib().mx_gemm_mxfp8(_ptr(aq), _ptr(as_), int(afmt), _ptr(bq), _ptr(bs), int(bfmt), M, N,
                              K, int(alpha_exp), code, _ptr(out), out.stride(0), _stream(stream)),
          "mx_gemm_mxfp8")
    return out


def mx_quantize_2d_blocks(x: torch.Tensor, block: int = 32, scale_rule: int = MX_SCALE_CEIL,
                          round: int = MX_ROUND_RNE, seed: int = 0, transposed: bool = True,
                          codes=None, scales=None, codes_t=None, scales_t=None, stream=None):
    """BxB tiles (block 8, 32 or 64) -> (codes, scales, codes_t, scales_t); scales [rows/8]
    [cols/8] for 8, [rows/32][cols/32] for 32, [rows/64][cols/32] (GEMM layout) for 64; the
    transposed pair is None unless transposed."""
    rows, cols, ld = _src(x)
    dev = x.device
    B = int(block)
    shape_s = {8: (rows // 8, cols // 8), 32: (rows // 32, cols // 32), 64: (rows // 64, cols // 32)}
    shape_st = {8: (cols // 8, rows // 8), 32: (cols // 32, rows // 32), 64: (cols // 64, rows // 32)}
    if B not in shape_s:
        raise ValueError("block must be 8, 32 or 64")
    codes = _codes_out(codes, "codes", (rows, cols // 2), dev)
    scales = _codes_out(scales, "scales", shape_s[B], dev)
    if not transposed:
        codes_t = scales_t = None
    else:
        codes_t = _codes_out(codes_t, "codes_t", (cols, rows // 2), dev)
        scales_t = _codes_out(scales_t, "scales_t", shape_st[B], dev)
    o = _opts(scale_rule, round, 0, 0, seed)
    check(lib().mx_quantize_2d_blocks(_ptr(x), _dtype_code(x), rows, cols, ld, B, ctypes.byref(o),
                                      _ptr(codes), _ptr(scales), _ptr(codes_t), _ptr(scales_t),
                                      _stream(stream)), "mx_quantize_2d_blocks")
    return codes, scales, codes_t, scales_t


def mx_scale_mismatch_map(x: torch.Tensor, scale_rule: int = MX_SCALE_FLOOR, out=None,
                          stream=None) -> torch.Tensor:
    """int8 [rows][cols]: scale exponent of each element's 1x32 row block minus that of its 1x32
    column block (saturated; -128 for non-finite blocks)."""
    rows, cols, ld = _src(x)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    _buf(out, "out", (rows, cols), (torch.int8,), x.device)
    check(lib().mx_scale_mismatch_map(_ptr(x), _dtype_code(x), rows, cols, ld, int(scale_rule),
                                      _ptr(out), _stream(stream)), "mx_scale_mismatch_map")
    return out
