// mfma_probe.hip — measured ceiling of gfx950's block-scaled FP4 matrix instruction, for the
// roofline of the GEMMs (a measurement aid, not part of the quantize/GEMM path).
//
// Each wave keeps 16 independent 32x32 accumulators (the 4x4 MFMA tiles a GEMM wave owns) and
// issues V_MFMA_SCALE_F32_32X32X64_F8F6F4 on them back to back with FP4 operands of random
// bits and random E8M0 scales near 1, so the matrix cores toggle as they do on real data
// (constant operand bits draw less power and clock higher, which overstates the ceiling). No
// memory traffic in the loop; one float per lane is written at the end so nothing is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// integer hash (xorshift-multiply), only to spread operand bits
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_fp4_probe_kernel(int iters, uint32_t seed, float* __restrict__ sink) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  v8i a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      a[i][w] = w < 4 ? (int)mix32(seed ^ (t * 64u + 8u * i + w)) : 0;
      b[i][w] = w < 4 ? (int)mix32(~seed ^ (t * 64u + 8u * i + w)) : 0;
    }
  // scale bytes 126 or 127 (factors 1/2 or 1): the sums stay far from overflow
  const int sa = (int)(0x7F7F7F7Fu ^ (mix32(seed + 3u * t) & 0x01010101u));
  const int sb = (int)(0x7F7F7F7Fu ^ (mix32(seed + 3u * t + 1u) & 0x01010101u));
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 4, 4,
                                                                    0, sb, 0, sa);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  sink[t] = s;
}

}  // namespace

extern "C" int32_t mx_probe_mfma_fp4(int32_t workgroups, int32_t iters, uint32_t seed, float* sink,
                                     void* stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_fp4_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     (hipStream_t)stream, iters, seed, sink);
  return (int32_t)hipGetLastError();
}
