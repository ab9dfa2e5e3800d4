/*
 * mx.h — C ABI of the MXFP4 block-scaled Hadamard-32 hot path for AMD MI355X (gfx950).
 *
 * The library (libmx.so) quantizes bf16/fp32 tensors into MXFP4 (E2M1 elements sharing one
 * E8M0 power-of-two scale per block of 32 elements, or per 32x32 tile) with an optional
 * 32-point Walsh-Hadamard rotation, and multiplies MXFP4 operands with gfx950's block-scaled
 * matrix cores for the three GEMMs of a linear layer (forward, input gradient, weight
 * gradient).
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "Block-Scaled MXFP4 With Stochastic Hadamard Rounding Matches BF16 Convergence on 70B
 *       Pre-Training" (lazytensor.com news item), paragraphs 1-2: one shared 8-bit power-of-two
 *       exponent (E8M0) per block of 32 4-bit E2M1 values; a 32-element block-diagonal
 *       Walsh-Hadamard transform applied in registers before the values are packed to 4 bits.
 *  [P2] "Pretraining large language models with MXFP4" (arXiv 2605.09825, abstract): FP4 in
 *       Fprop, Dgrad and Wgrad; deterministic Hadamard rotations stabilise the Wgrad path.
 *  [P3] "Stable FP4 Training via Transposition-Invariant Block Quantization" (arXiv 2607.24953
 *       review): section "Why FP4 training is the current frontier" (E2M1 bits, per-block scale
 *       from the block max, P = round(X/S), reconstruction P*S); section "The aha: transposition
 *       scrambles the blocks" (the GEMM orientations, 1-D re-blocking under transposition);
 *       section "The fix, and its supporting cast" (32x32 blocks, scale rounded up to a power of
 *       two so nothing clips, stochastic rounding with E[round(x)] = x).
 *  [P4] "Training LLMs with MXFP4" (arXiv 2502.20586, abstract): stochastic rounding plus a
 *       random Hadamard transform (random +/-1 signs) to bound its variance.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller. The library allocates no
 *    device memory, keeps no global state and never synchronises; all work is enqueued on
 *    `stream` (a hipStream_t passed as void*, NULL = the null stream).
 *  - `opts` is a HOST pointer, read during the call only.
 *  - The return value reports argument validation and launch errors. A non-OK status means
 *    nothing was enqueued. Faults during execution surface at the caller's next
 *    synchronisation of `stream`.
 *  - Dimensions are element counts; every dimension along which blocks are formed must be a
 *    positive multiple of 32 (MX_ERR_SHAPE otherwise). A zero-sized tensor is MX_OK and
 *    enqueues nothing.
 *  - Packed codes: two E2M1 codes per byte, the element with the even index along the packed
 *    (block) axis in the low nibble. A code is (sign << 3) | m, m in 0..7 indexing the
 *    magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. The sign bit is copied from the value, so a
 *    negative value that rounds to zero is code 0x8.
 *  - Scales: one byte per block, value 2^(byte-127); byte 0xFF (NaN) marks a block whose
 *    maximum was not finite (its codes are then all zero).
 */
#ifndef MX_H
#define MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,        /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,       /* a dimension is negative, not a multiple of 32, or ld too small */
  MX_ERR_UNSUPPORTED = 3, /* an option combination the path does not define */
  MX_ERR_LAUNCH = 4,      /* the HIP runtime refused the launch */
  MX_ERR_ARG = 5          /* an enum/option value out of range */
} mx_status;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;

/* Scale exponent e of a block with maximum magnitude amax = m * 2^E, m in [1, 2):
 *  MX_SCALE_FLOOR: e = E - 2 (the OCP rule: floor(log2 amax) minus E2M1's largest exponent);
 *                  elements whose scaled magnitude exceeds 6 saturate to 6.
 *  MX_SCALE_CEIL : the least e with amax <= 6 * 2^e ("truncation-free": the scale is rounded
 *                  up to a power of two, so no element clips) [P3, "The fix ..."].
 * amax = 0 gives e = -127. e is clamped to [-127, 127]; the scale byte is e + 127. */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_CEIL = 1 } mx_scale_rule;

/* Rounding of v = x * 2^-e to E2M1:
 *  MX_ROUND_RNE: nearest grid point, ties to the even code, |v| >= 6 saturates to 6.
 *  MX_ROUND_SR : with lo <= |v| < hi adjacent grid points and f = (|v| - lo) / (hi - lo), the
 *                magnitude rounds up to hi iff r < f * 2^16, where r is the 16-bit random field
 *                of the element; so E[round(v)] = v up to 2^-16 of a grid step [P3, "The fix
 *                ..."; P4]. r comes from Philox4x32-10 (Salmon et al., SC'11) keyed by
 *                (seed & 0xffffffff, seed >> 32) at counter (i >> 3 as two 32-bit words, 0, 0);
 *                element i takes 16-bit field (i & 7) of the 128-bit output: word (i & 7) >> 1,
 *                low half for even i. i is the row-major index r * cols + c of the element in
 *                the SOURCE tensor, whatever the block shape or output layout. */
typedef enum { MX_ROUND_RNE = 0, MX_ROUND_SR = 1 } mx_round;

typedef struct {
  int32_t scale_rule; /* mx_scale_rule */
  int32_t round;      /* mx_round */
  int32_t hadamard;   /* 0 or 1: rotate every 32-block before scaling [P1 paragraph 2] */
  uint32_t sign_mask; /* random +/-1 diagonal D: bit j set negates block position j before the
                         transform [P4]; 0 = the deterministic transform [P2] */
  uint64_t seed;      /* Philox key for MX_ROUND_SR; ignored for MX_ROUND_RNE */
} mx_quant_opts;

/* 1x32 blocks [P1 paragraph 1; P3 "Why FP4 ..."].
 * x: [rows][ld] row-major, dtype MX_BF16 or MX_F32, ld >= cols (elements).
 * axis = 1: blocks run along a row (the common case).      codes [rows][cols/2],
 *           scales [rows][cols/32]; needs cols % 32 == 0.
 * axis = 0: blocks run down a column (e.g. along tokens for the weight gradient); the output
 *           is the K-major layout of the transpose: codes [cols][rows/2],
 *           scales [cols][rows/32]; needs rows % 32 == 0.
 * Per block, in this order: widen to fp32; if opts->hadamard, negate the positions selected by
 * sign_mask and apply the unnormalised 32-point Sylvester-Hadamard transform
 * H[i][j] = (-1)^popcount(i & j) as five fp32 butterfly stages of span 1, 2, 4, 8, 16;
 * block maximum; scale exponent; v = x * 2^-e in fp32; round; pack.
 * Alignment: x and every source row (ld * element size) 16 bytes; codes 16 bytes (a code row
 * is a multiple of 16 bytes, so any row slice of an aligned buffer qualifies); axis = 0 also
 * needs cols % 8 == 0.
 * Errors (nothing is launched): MX_ERR_NULL for a NULL x, codes, scales or opts;
 * MX_ERR_SHAPE for negative sizes, ld < cols or a multiple-of-32 / row-alignment rule;
 * MX_ERR_ARG for a bad dtype, axis or option value, or a misaligned pointer;
 * MX_ERR_LAUNCH if the kernel launch fails. rows == 0 or cols == 0 is a no-op. */
mx_status mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                      int32_t axis, const mx_quant_opts* opts, uint8_t* codes, uint8_t* scales,
                      void* stream);

/* 32x32 blocks, transposition invariant [P3, "The fix ...": block (i, j) of X is block (j, i)
 * of X^T with the same values, maximum and scale]. rows and cols must be multiples of 32;
 * opts->hadamard must be 0 (MX_ERR_UNSUPPORTED otherwise).
 * codes  [rows][cols/2], scales   [rows/32][cols/32]      (required)
 * codes_t[cols][rows/2], scales_t [cols/32][rows/32]      (optional, may be NULL)
 * codes_t/scales_t hold the SAME rounding decisions in the K-major layout of X^T, so the
 * transposed GEMM consumes them without re-quantization.
 * Alignment: x and every source row 16 bytes, codes and codes_t 16 bytes. Errors as for
 * mx_quantize, plus MX_ERR_NULL when exactly one of codes_t / scales_t is NULL. */
mx_status mx_quantize_2d(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                         const mx_quant_opts* opts, uint8_t* codes, uint8_t* scales,
                         uint8_t* codes_t, uint8_t* scales_t, void* stream);

/* out[r][c] = E2M1(code) * 2^(scale - 127) in fp32 ("reconstructed as P*S", [P3 "Why FP4
 * ..."]); out is [rows][cols] contiguous. block_rows = 1 reads scales [rows][cols/32];
 * block_rows = 32 reads 2-D scales [rows/32][cols/32]. If inv_hadamard (block_rows == 1 only),
 * each 32-block is then mapped back by (1/32) * D * H: the same five fp32 butterfly stages,
 * a multiply by 1/32, and the sign flips of sign_mask.
 * Alignment: codes 4 bytes, out 16 bytes; cols % 32 == 0 (rows % 32 == 0 for block_rows = 32).
 * MX_ERR_UNSUPPORTED for inv_hadamard with block_rows = 32. */
mx_status mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        int32_t block_rows, int32_t inv_hadamard, uint32_t sign_mask, float* out,
                        void* stream);

/* Block-scaled MXFP4 GEMMs [P2 abstract; P3 "The aha ..."; P4 abstract].
 * All three compute C[m][n] = 2^alpha_exp * sum_k A[m][k] * B[n][k] with both operands packed
 * K-major (codes [rows][K/2]) and fp32 accumulation. A scale granularity g of 1 means scales
 * [rows][K/32]; g = 32 means 2-D scales [rows/32][K/32] (from mx_quantize_2d); g = 64 means
 * [rows/64][K/32] (64x64 tiles from mx_quantize_2d_blocks, each byte covering two 32-k blocks).
 * The operand's row count must be a multiple of g. alpha_exp = -5
 * undoes the factor 32 of two unnormalised Hadamard rotations along K (the caller guarantees
 * both operands used the same sign_mask); otherwise 0. out_dtype MX_BF16 (round to nearest
 * even) or MX_F32; ldc >= the output row length, in elements.
 *   fprop: Y  [T][N] = X  [T][K] . W [N][K]^T   (reduce over K)
 *   dgrad: dX [T][K] = dY [T][N] . Wt[K][N]^T   (reduce over N; Wt = W blocked along N)
 *   wgrad: dW [N][K] = dYt[N][T] . Xt[K][T]^T   (reduce over tokens T)
 * M, N multiples of 32, K a multiple of 32; the operand codes and C 16-byte aligned, ldc a
 * multiple of 8 elements. One 256-row operand tile must stay below 2 GiB (256 * K / 2 < 2^31).
 * Errors (nothing is launched): MX_ERR_SHAPE, MX_ERR_ARG (granularity, out_dtype, alpha_exp
 * outside [-126, 127], alignment), MX_ERR_NULL; MX_ERR_LAUNCH if the launch fails or the shape
 * exceeds the 32-bit offsets above. M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 * Accuracy: the E2M1 x E2M1 products with their scales are summed exactly within one 64-k
 * matrix instruction, and the K/64 instruction results are added in fp32, one accumulator per
 * output: the error is that of those additions, at worst (K/64) * 2^-24 * sum_k |a_k b_k|, and
 * within the tolerance |C - exact| <= 2^-20 * sum_k |a_k b_k| on the tested workloads (K up to
 * 28672) for fp32 output; bf16 output is the rounding of such a value. */
mx_status mx_gemm_fprop(const uint8_t* xq, const uint8_t* xs, int32_t gx, const uint8_t* wq,
                        const uint8_t* ws, int32_t gw, int64_t T, int64_t N, int64_t K,
                        int32_t alpha_exp, int32_t out_dtype, void* y, int64_t ldy, void* stream);
mx_status mx_gemm_dgrad(const uint8_t* dyq, const uint8_t* dys, int32_t gdy, const uint8_t* wtq,
                        const uint8_t* wts, int32_t gwt, int64_t T, int64_t K, int64_t N,
                        int32_t alpha_exp, int32_t out_dtype, void* dx, int64_t ldx, void* stream);
mx_status mx_gemm_wgrad(const uint8_t* dytq, const uint8_t* dyts, int32_t gdy, const uint8_t* xtq,
                        const uint8_t* xts, int32_t gx, int64_t N, int64_t K, int64_t T,
                        int32_t alpha_exp, int32_t out_dtype, void* dw, int64_t ldw, void* stream);

/* Fprop with the output quantized in the epilogue [P1 paragraph 1: the Walsh-Hadamard rotation
 * and stochastic rounding run inside the GEMM epilogue, before the output tile is packed to
 * 4 bits]. Y = 2^alpha_exp * X . W^T is formed in fp32 exactly as mx_gemm_fprop forms it and,
 * instead of being stored, quantized as mx_quantize(Y, axis = 1, opts) would quantize that fp32
 * tensor: 1x32 blocks along N, yq [T][N/2], ys [T][N/32], stochastic-rounding index t * N + n.
 * Arguments as for mx_gemm_fprop; opts as for mx_quantize. K must be a positive multiple of 128
 * (MX_ERR_UNSUPPORTED otherwise); yq 4-byte aligned. The fp32 values are not bit-identical to
 * those of a separate fp32 GEMM with a different accumulation order, so the codes equal the
 * quantization of some fp32 Y within the GEMM bound of mx_gemm_fprop. */
mx_status mx_gemm_fprop_quant(const uint8_t* xq, const uint8_t* xs, int32_t gx, const uint8_t* wq,
                              const uint8_t* ws, int32_t gw, int64_t T, int64_t N, int64_t K,
                              int32_t alpha_exp, const mx_quant_opts* opts, uint8_t* yq,
                              uint8_t* ys, void* stream);

/* MXFP8 [P3, "The fix, and its supporting cast": the query and key projections are quantized
 * in MXFP8 rather than FP4]. Blocks, scales, options and stochastic-rounding fields are those
 * of the MXFP4 path; the elements are 8-bit OCP floating point (the pages do not fix the
 * encoding):
 *  MX_E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 15 with mantissa 7 is
 *           NaN and there is no infinity, so the largest magnitude is 448 = 1.75 * 2^8;
 *  MX_E5M2: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent 31 is inf / NaN, the
 *           largest magnitude is 57344 = 1.75 * 2^15.
 * Exponent field 0 is subnormal. A code is one byte, the sign in bit 7 (copied from the value).
 * Scale exponent, with amax = m * 2^E, m in [1, 2): MX_SCALE_FLOOR e = E - emax (emax = 8 or
 * 15, the exponent of the largest magnitude; values beyond it saturate); MX_SCALE_CEIL the
 * least e with amax <= largest * 2^e. MX_ROUND_RNE rounds to the nearest representable value
 * with ties to the even code; MX_ROUND_SR rounds up iff r < f * 2^16 as for E2M1; |v| >= the
 * largest magnitude gives the largest code. */
typedef enum { MX_E4M3 = 0, MX_E5M2 = 1 } mx_fp8_format;

/* 1x32 MXFP8 quantize; arguments as for mx_quantize plus fmt (mx_fp8_format).
 * axis = 1: codes [rows][cols] (one byte per element), scales [rows][cols/32];
 * axis = 0: codes [cols][rows], scales [cols][rows/32] (the K-major layout of the transpose).
 * Alignment: x and source rows 16 bytes; codes 8 bytes (axis = 1) or 16 bytes (axis = 0);
 * axis = 0 also needs cols % 8 == 0. Errors as for mx_quantize; MX_ERR_ARG for a bad fmt. */
mx_status mx_quantize_mxfp8(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            int32_t axis, int32_t fmt, const mx_quant_opts* opts, uint8_t* codes,
                            uint8_t* scales, void* stream);

/* MXFP8 GEMM on gfx950's block-scaled matrix cores: C[m][n] = 2^alpha_exp * sum_k A[m][k] *
 * B[n][k], fp32 accumulation, with A codes [M][K] of format afmt and B codes [N][K] of format
 * bfmt (one byte per element, K-major), scales [M][K/32] and [N][K/32]. Fprop, Dgrad and Wgrad
 * are this call on the operands of the respective orientation (as for the MXFP4 calls).
 * M, N multiples of 32; K a positive multiple of 128 (MX_ERR_UNSUPPORTED otherwise, except
 * K == 0, which writes zeros); operand codes and C 16-byte aligned; ldc a multiple of 8
 * elements; 256 * K < 2^31. out_dtype, alpha_exp and errors as for mx_gemm_fprop.
 * Accuracy: |C - exact| <= 2^-10 * sum_k |a_k b_k| for fp32 output (K <= 65536), and bf16
 * output is the rounding of a value within that bound. The bound is the matrix core's: within
 * each group of 8 consecutive products of one 64-k instruction, every product is truncated
 * toward zero to a multiple of 2^(E - 13), 2^E the leading power of two of the group's largest
 * product, and the truncated products are summed exactly and rounded to fp32 once (derived
 * from single-instruction measurements on gfx950). A group loses less than 7 * 2^-13 of its
 * largest product, and the K/64 fp32 additions of the instruction results add at most
 * (K/64) 2^-24 sum |a_k b_k|. (MXFP4 products are summed exactly: the 2^-20 rule of
 * mx_gemm_fprop.) */
mx_status mx_gemm_mxfp8(const uint8_t* aq, const uint8_t* as, int32_t afmt, const uint8_t* bq,
                        const uint8_t* bs, int32_t bfmt, int64_t M, int64_t N, int64_t K,
                        int32_t alpha_exp, int32_t out_dtype, void* c, int64_t ldc, void* stream);

/* Square tiles of other sizes [P3, "The fix ...": Table 4 compares 8x8, 32x32 and 64x64
 * blocks, the smaller with more scale metadata]. As mx_quantize_2d with tile edge block = 8, 32
 * or 64: one scale per tile from the tile maximum, every element rounded once and written to
 * both code layouts (codes [rows][cols/2], codes_t [cols][rows/2], as for mx_quantize_2d).
 * Scales: block = 8: scales [rows/8][cols/8], scales_t [cols/8][rows/8];
 *         block = 32: exactly mx_quantize_2d;
 *         block = 64: in the layout the GEMMs read with g = 64, scales [rows/64][cols/32] and
 *                     scales_t [cols/64][rows/32], each tile's byte stored for both of its
 *                     32-wide halves.
 * 8x8 tiles cannot feed the block-scaled matrix cores, whose scale blocks are 32 elements along
 * K; they are a quantization (and mismatch) format here. rows and cols must be multiples of
 * max(block, 32); opts->hadamard must be 0. Alignment: x and source rows 16 bytes, codes and
 * codes_t 16 bytes, scales and scales_t 4 bytes. Errors as for mx_quantize_2d, plus MX_ERR_ARG
 * for another block. */
mx_status mx_quantize_2d_blocks(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ld, int32_t block, const mx_quant_opts* opts,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, void* stream);

/* Scale-difference map of 1x32 blocking [P3, "The aha: transposition scrambles the blocks",
 * Figure 1]: map[r][c] = e_row - e_col, where e_row is the scale exponent (scale_rule, as for
 * mx_quantize) of the 1x32 block along row r that holds element (r, c), how X enters the forward
 * product, and e_col that of the 1x32 block down column c, how X enters the transposed product.
 * int8, saturated to [-127, 127]; -128 where either block's maximum is not finite. With 32x32
 * tiles the two exponents are one and the same, so the map of that quantizer is zero.
 * x: [rows][ld] bf16 or fp32, rows and cols multiples of 32; map [rows][cols] contiguous, 8-byte
 * aligned. Errors: MX_ERR_SHAPE, MX_ERR_ARG (dtype, scale_rule, alignment), MX_ERR_NULL. */
mx_status mx_scale_mismatch_map(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                int64_t ld, int32_t scale_rule, int8_t* map, void* stream);

/* Human-readable name of a status code (static storage). */
const char* mx_status_string(int32_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
