// mx_launch.h — internal interface between the C ABI layer (mx_api.hip) and the kernel
// launchers (quant.hip, gemm.hip). Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct QuantArgs {
  const void* x;
  bool bf16;
  int64_t rows, cols, ld;
  int axis;          // 1D only
  bool ceil, sr, hadamard;
  uint32_t sign_mask;
  uint64_t seed;
  uint8_t* codes;    // axis 1 / 2-D: [rows][cols/2];  axis 0: [cols][rows/2]
  uint8_t* scales;
  uint8_t* codes_t;  // 2-D only, nullable
  uint8_t* scales_t; // 2-D only, nullable
  void* stream;
};

hipError_t mx_launch_quantize(const QuantArgs& a);
hipError_t mx_launch_quantize_2d(const QuantArgs& a);
// MXFP8 1x32 quantize (fmt 0 = E4M3, 1 = E5M2): codes one byte per element,
// axis 1: [rows][cols], axis 0: [cols][rows]; scales as for MXFP4
hipError_t mx_launch_quantize_fp8(const QuantArgs& a, int fmt);
// B x B tiles (block 8, 32 or 64; rows and cols multiples of max(block, 32)); for 64 the scales
// are in the GEMM layout [rows/64][cols/32] / [cols/64][rows/32] (each byte twice)
hipError_t mx_launch_quantize_2d_blocks(const QuantArgs& a, int block);
// map[r][c] = scale byte of the row block of (r, c) minus that of its column block (int8,
// saturated; -128 for a non-finite block); rows, cols multiples of 32
hipError_t mx_launch_scale_mismatch(const void* x, bool bf16, int64_t rows, int64_t cols,
                                    int64_t ld, bool ceil, int8_t* map, void* stream);
hipError_t mx_launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, int block_rows, int inv_had, uint32_t sign_mask,
                                float* out, void* stream);

// C[m][n] = 2^alpha * sum_k A[m][k] * B[n][k]; A [M][K/2], B [N][K/2] packed E2M1, scales
// [M/ga][K/32] and [N/gb][K/32].
struct GemmArgs {
  const uint8_t* a;
  const uint8_t* as;
  int ga;
  const uint8_t* b;
  const uint8_t* bs;
  int gb;
  int64_t M, N, K;
  int alpha;
  bool out_bf16;
  void* c;
  int64_t ldc;
  void* stream;
};

hipError_t mx_launch_gemm(const GemmArgs& g);

// Epilogue quantization of C along its rows (1x32 blocks along N), instead of storing C:
// codes [M][N/2], scales [M][N/32]; the random-field index of C[m][n] is m * N + n.
struct GemmQuantOut {
  uint8_t* codes;
  uint8_t* scales;
  bool hadamard, sr, ceil;
  uint32_t sign_mask;
  uint64_t seed;
};

// K must be a multiple of 128 (the streaming kernels); returns hipErrorInvalidValue otherwise.
hipError_t mx_launch_gemm_quant(const GemmArgs& g, const GemmQuantOut& q);

// MXFP8 GEMM: A [M][K], B [N][K] one code byte per element (afmt / bfmt: 0 = E4M3, 1 = E5M2),
// scales [M][K/32] and [N][K/32] (ga = gb = 1). K must be a positive multiple of 128.
hipError_t mx_launch_gemm_fp8(const GemmArgs& g, int afmt, int bfmt);
