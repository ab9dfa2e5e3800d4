// mx_api.hip — the extern "C" entry points declared in include/mx.h: argument validation and
// dispatch to the kernel launchers. No allocation, no synchronisation, no global state.
#include "mx.h"
#include "mx_launch.h"

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mx_status launch_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH; }

// scale row granularity of a GEMM operand: per row, per 32x32 tile or per 64x64 tile
bool granularity_ok(int32_t g) { return g == 1 || g == 32 || g == 64; }

mx_status check_opts(const mx_quant_opts* o) {
  if (!o) return MX_ERR_NULL;
  if (o->scale_rule != MX_SCALE_FLOOR && o->scale_rule != MX_SCALE_CEIL) return MX_ERR_ARG;
  if (o->round != MX_ROUND_RNE && o->round != MX_ROUND_SR) return MX_ERR_ARG;
  if (o->hadamard != 0 && o->hadamard != 1) return MX_ERR_ARG;
  return MX_OK;
}

// Source tensor checks shared by both quantizers: rows 16-byte aligned (8 elements per lane).
mx_status check_source(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld) {
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_ERR_ARG;
  if (rows < 0 || cols < 0 || ld < cols) return MX_ERR_SHAPE;
  const int64_t esize = dtype == MX_BF16 ? 2 : 4;
  if ((ld * esize) % 16 != 0) return MX_ERR_SHAPE;
  if (!aligned(x, 16)) return MX_ERR_ARG;
  return MX_OK;
}

mx_status gemm(const uint8_t* a, const uint8_t* as, int32_t ga, const uint8_t* b,
               const uint8_t* bs, int32_t gb, int64_t M, int64_t N, int64_t K, int32_t alpha_exp,
               int32_t out_dtype, void* c, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return MX_ERR_SHAPE;
  if (M % 32 || N % 32 || K % 32) return MX_ERR_SHAPE;
  if (ldc < N || ldc % 8 != 0) return MX_ERR_SHAPE;
  if (!granularity_ok(ga) || !granularity_ok(gb)) return MX_ERR_ARG;
  if (M % ga || N % gb) return MX_ERR_SHAPE;
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_ARG;
  if (alpha_exp < -126 || alpha_exp > 127) return MX_ERR_ARG;
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return MX_ERR_NULL;
  if (!aligned(c, 16)) return MX_ERR_ARG;
  if (K > 0) {
    if (!a || !as || !b || !bs) return MX_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16)) return MX_ERR_ARG;
  }
  GemmArgs g{a, as, ga, b, bs, gb, M, N, K, alpha_exp, out_dtype == MX_BF16, c, ldc, stream};
  return launch_status(mx_launch_gemm(g));
}

}  // namespace

extern "C" {

mx_status mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                      int32_t axis, const mx_quant_opts* opts, uint8_t* codes, uint8_t* scales,
                      void* stream) {
  mx_status s = check_opts(opts);
  if (s != MX_OK) return s;
  if (axis != 0 && axis != 1) return MX_ERR_ARG;
  if ((s = check_source(x, dtype, rows, cols, ld)) != MX_OK) return s;
  if (axis == 1 && cols % 32 != 0) return MX_ERR_SHAPE;
  if (axis == 0 && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  // rows: the 16 code bytes of a block per lane; columns: 16-byte pieces of transposed code rows
  if (!aligned(codes, 16)) return MX_ERR_ARG;
  QuantArgs a{x, dtype == MX_BF16, rows, cols, ld, axis, opts->scale_rule == MX_SCALE_CEIL,
              opts->round == MX_ROUND_SR, opts->hadamard == 1, opts->sign_mask, opts->seed,
              codes, scales, nullptr, nullptr, stream};
  return launch_status(mx_launch_quantize(a));
}

mx_status mx_quantize_2d(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                         const mx_quant_opts* opts, uint8_t* codes, uint8_t* scales,
                         uint8_t* codes_t, uint8_t* scales_t, void* stream) {
  mx_status s = check_opts(opts);
  if (s != MX_OK) return s;
  if (opts->hadamard) return MX_ERR_UNSUPPORTED;
  if ((s = check_source(x, dtype, rows, cols, ld)) != MX_OK) return s;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if ((codes_t == nullptr) != (scales_t == nullptr)) return MX_ERR_NULL;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned(codes, 16) || (codes_t && !aligned(codes_t, 16))) return MX_ERR_ARG;
  QuantArgs a{x, dtype == MX_BF16, rows, cols, ld, 1, opts->scale_rule == MX_SCALE_CEIL,
              opts->round == MX_ROUND_SR, false, 0u, opts->seed, codes, scales, codes_t,
              scales_t, stream};
  return launch_status(mx_launch_quantize_2d(a));
}

mx_status mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        int32_t block_rows, int32_t inv_hadamard, uint32_t sign_mask, float* out,
                        void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if (block_rows != 1 && block_rows != 32) return MX_ERR_ARG;
  if (inv_hadamard != 0 && inv_hadamard != 1) return MX_ERR_ARG;
  if (inv_hadamard && block_rows != 1) return MX_ERR_UNSUPPORTED;
  if (block_rows == 32 && rows % 32 != 0) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!codes || !scales || !out) return MX_ERR_NULL;
  if (!aligned(codes, 4) || !aligned(out, 16)) return MX_ERR_ARG;
  return launch_status(mx_launch_dequantize(codes, scales, rows, cols, block_rows, inv_hadamard,
                                            sign_mask, out, stream));
}

mx_status mx_gemm_fprop_quant(const uint8_t* xq, const uint8_t* xs, int32_t gx, const uint8_t* wq,
                              const uint8_t* ws, int32_t gw, int64_t T, int64_t N, int64_t K,
                              int32_t alpha_exp, const mx_quant_opts* opts, uint8_t* yq,
                              uint8_t* ys, void* stream) {
  mx_status s = check_opts(opts);
  if (s != MX_OK) return s;
  if (T < 0 || N < 0 || K < 0) return MX_ERR_SHAPE;
  if (T % 32 || N % 32 || K % 32) return MX_ERR_SHAPE;
  if (!granularity_ok(gx) || !granularity_ok(gw)) return MX_ERR_ARG;
  if (T % gx || N % gw) return MX_ERR_SHAPE;
  if (alpha_exp < -126 || alpha_exp > 127) return MX_ERR_ARG;
  if (T == 0 || N == 0) return MX_OK;
  if (K == 0 || K % 128 != 0) return MX_ERR_UNSUPPORTED;  // the streaming kernels only
  if (!xq || !xs || !wq || !ws || !yq || !ys) return MX_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(yq, 4)) return MX_ERR_ARG;
  GemmArgs g{xq, xs, gx, wq, ws, gw, T, N, K, alpha_exp, false, nullptr, N, stream};
  GemmQuantOut q{yq, ys, opts->hadamard == 1, opts->round == MX_ROUND_SR,
                 opts->scale_rule == MX_SCALE_CEIL, opts->sign_mask, opts->seed};
  return launch_status(mx_launch_gemm_quant(g, q));
}

mx_status mx_gemm_fprop(const uint8_t* xq, const uint8_t* xs, int32_t gx, const uint8_t* wq,
                        const uint8_t* ws, int32_t gw, int64_t T, int64_t N, int64_t K,
                        int32_t alpha_exp, int32_t out_dtype, void* y, int64_t ldy, void* stream) {
  return gemm(xq, xs, gx, wq, ws, gw, T, N, K, alpha_exp, out_dtype, y, ldy, stream);
}

mx_status mx_gemm_dgrad(const uint8_t* dyq, const uint8_t* dys, int32_t gdy, const uint8_t* wtq,
                        const uint8_t* wts, int32_t gwt, int64_t T, int64_t K, int64_t N,
                        int32_t alpha_exp, int32_t out_dtype, void* dx, int64_t ldx, void* stream) {
  return gemm(dyq, dys, gdy, wtq, wts, gwt, T, K, N, alpha_exp, out_dtype, dx, ldx, stream);
}

mx_status mx_gemm_wgrad(const uint8_t* dytq, const uint8_t* dyts, int32_t gdy, const uint8_t* xtq,
                        const uint8_t* xts, int32_t gx, int64_t N, int64_t K, int64_t T,
                        int32_t alpha_exp, int32_t out_dtype, void* dw, int64_t ldw, void* stream) {
  return gemm(dytq, dyts, gdy, xtq, xts, gx, N, K, T, alpha_exp, out_dtype, dw, ldw, stream);
}

mx_status mx_quantize_mxfp8(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            int32_t axis, int32_t fmt, const mx_quant_opts* opts, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  mx_status s = check_opts(opts);
  if (s != MX_OK) return s;
  if (axis != 0 && axis != 1) return MX_ERR_ARG;
  if (fmt != MX_E4M3 && fmt != MX_E5M2) return MX_ERR_ARG;
  if ((s = check_source(x, dtype, rows, cols, ld)) != MX_OK) return s;
  if (axis == 1 && cols % 32 != 0) return MX_ERR_SHAPE;
  if (axis == 0 && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  // rows: 8 code bytes per lane; columns: 16-byte pieces of transposed code rows
  if (!aligned(codes, axis == 1 ? 8 : 16)) return MX_ERR_ARG;
  QuantArgs a{x, dtype == MX_BF16, rows, cols, ld, axis, opts->scale_rule == MX_SCALE_CEIL,
              opts->round == MX_ROUND_SR, opts->hadamard == 1, opts->sign_mask, opts->seed,
              codes, scales, nullptr, nullptr, stream};
  return launch_status(mx_launch_quantize_fp8(a, fmt));
}

mx_status mx_gemm_mxfp8(const uint8_t* aq, const uint8_t* as, int32_t afmt, const uint8_t* bq,
                        const uint8_t* bs, int32_t bfmt, int64_t M, int64_t N, int64_t K,
                        int32_t alpha_exp, int32_t out_dtype, void* c, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return MX_ERR_SHAPE;
  if (M % 32 || N % 32 || K % 32) return MX_ERR_SHAPE;
  if (ldc < N || ldc % 8 != 0) return MX_ERR_SHAPE;
  if ((afmt != MX_E4M3 && afmt != MX_E5M2) || (bfmt != MX_E4M3 && bfmt != MX_E5M2)) return MX_ERR_ARG;
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_ARG;
  if (alpha_exp < -126 || alpha_exp > 127) return MX_ERR_ARG;
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return MX_ERR_NULL;
  if (!aligned(c, 16)) return MX_ERR_ARG;
  GemmArgs g{aq, as, 1, bq, bs, 1, M, N, K, alpha_exp, out_dtype == MX_BF16, c, ldc, stream};
  if (K == 0) return launch_status(mx_launch_gemm(g));  // an empty sum: the output is zero
  if (K % 128 != 0) return MX_ERR_UNSUPPORTED;
  if (!aq || !as || !bq || !bs) return MX_ERR_NULL;
  if (!aligned(aq, 16) || !aligned(bq, 16)) return MX_ERR_ARG;
  return launch_status(mx_launch_gemm_fp8(g, afmt, bfmt));
}

mx_status mx_quantize_2d_blocks(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ld, int32_t block, const mx_quant_opts* opts,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, void* stream) {
  mx_status s = check_opts(opts);
  if (s != MX_OK) return s;
  if (block != 8 && block != 32 && block != 64) return MX_ERR_ARG;
  if (opts->hadamard) return MX_ERR_UNSUPPORTED;
  if ((s = check_source(x, dtype, rows, cols, ld)) != MX_OK) return s;
  const int64_t unit = block > 32 ? block : 32;
  if (rows % unit != 0 || cols % unit != 0) return MX_ERR_SHAPE;
  if ((codes_t == nullptr) != (scales_t == nullptr)) return MX_ERR_NULL;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned(codes, 16) || (codes_t && !aligned(codes_t, 16))) return MX_ERR_ARG;
  if (!aligned(scales, 4) || (scales_t && !aligned(scales_t, 4))) return MX_ERR_ARG;
  QuantArgs a{x, dtype == MX_BF16, rows, cols, ld, 1, opts->scale_rule == MX_SCALE_CEIL,
              opts->round == MX_ROUND_SR, false, 0u, opts->seed, codes, scales, codes_t,
              scales_t, stream};
  return launch_status(mx_launch_quantize_2d_blocks(a, block));
}

mx_status mx_scale_mismatch_map(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ld, int32_t scale_rule, int8_t* map, void* stream) {
  if (scale_rule != MX_SCALE_FLOOR && scale_rule != MX_SCALE_CEIL) return MX_ERR_ARG;
  mx_status s = check_source(x, dtype, rows, cols, ld);
  if (s != MX_OK) return s;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !map) return MX_ERR_NULL;
  if (!aligned(map, 8)) return MX_ERR_ARG;
  return launch_status(mx_launch_scale_mismatch(x, dtype == MX_BF16, rows, cols, ld,
                                                scale_rule == MX_SCALE_CEIL, map, stream));
}

const char* mx_status_string(int32_t status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: bad dimension, multiple-of-32 rule or leading dimension";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED: option combination not defined";
    case MX_ERR_LAUNCH: return "MX_ERR_LAUNCH: the HIP runtime refused the launch";
    case MX_ERR_ARG: return "MX_ERR_ARG: option value out of range or misaligned pointer";
    default: return "unknown mx_status";
  }
}

int32_t mx_version(void) { return kVersion; }

}  // extern "C"
