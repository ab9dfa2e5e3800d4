// gemm.hip — block-scaled MXFP4 GEMM on gfx950 matrix cores.
//
// C[m][n] = 2^alpha * sum_k A[m][k] * B[n][k], both operands packed E2M1 in K-major rows with
// one E8M0 scale per 32 consecutive k (per row, or per 32x32 tile). This single kernel serves
// the forward, input-gradient and weight-gradient products of a linear layer: every one of
// them reduces along the axis its operands were blocked on ("Stable FP4 Training via
// Transposition-Invariant Block Quantization", section "The aha: transposition scrambles the
// blocks"; "Pretraining large language models with MXFP4", abstract: FP4 in Fprop, Dgrad and
// Wgrad; "Training LLMs with MXFP4", abstract: MXFP4 GEMMs).
//
// Matrix-core facts used (gfx950 V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands):
//  * operand lane l holds row (l % 32) and k = 32 * (l / 32) .. +31 of a 32x64 slice, as 16
//    bytes, element 2i in the low nibble of byte i;
//  * the 32-bit scale operand of lane l carries the E8M0 byte of exactly that 32-element
//    k-block; the op_sel immediate picks which byte of the register is used;
//  * output register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
// Because every lane's 32 k-values form one scale block, the block scales enter the product
// directly and the fp32 accumulation sees exact products.
//
// Tiling: a 256-thread workgroup computes a 256x256 tile; each of the 4 waves owns 128x128 =
// 4x4 MFMA tiles (256 fp32 accumulators per lane). K advances 128 at a time (64 bytes per row);
// packed tiles and their scale words are staged in LDS, double-buffered, with a 16-byte chunk
// swizzle so the MFMA fragment reads of 16 consecutive rows hit distinct banks. The B tile
// feeds the MFMA's first operand so that a lane's 4 consecutive output registers are 4
// consecutive columns of C (one 8- or 16-byte store).
#include "mx_device.h"
#include "mx_launch.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 128;                 // k elements per step
constexpr int kRowBytes = kBK / 2;       // 64 bytes of codes per row per step
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kRowBytes;           // 16 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes + 2 * kBM * 4;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One k-step of global loads for one operand: 4 chunks of 16 bytes per thread plus the 4
// scale bytes of one row.
struct StepRegs {
  uint4 a[4], b[4];
  uint32_t sa, sb;
};

__device__ __forceinline__ uint4 load_chunk(const uint8_t* __restrict__ base, int64_t rows,
                                            int64_t kbytes, int64_t row, int64_t kbyte) {
  if (row < rows && kbyte < kbytes)
    return *reinterpret_cast<const uint4*>(base + row * kbytes + kbyte);
  return make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ uint32_t load_scales4(const uint8_t* __restrict__ s, int g, int64_t rows,
                                                 int64_t nkb, int64_t row, int64_t kb0) {
  uint32_t w = 0x7F7F7F7Fu;  // unit scale for k beyond K (their codes are zero)
  if (row < rows) {
    const uint8_t* p = s + (row / g) * nkb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kb0 + i < nkb) w = (w & ~(0xFFu << (8 * i))) | ((uint32_t)p[kb0 + i] << (8 * i));
    }
  }
  return w;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, int ga,
                    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int gb,
                    int64_t M, int64_t N, int64_t K, float alpha_f, int out_bf16,
                    void* __restrict__ C, int64_t ldc, int nbm, int nbn) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  // ---- tile schedule: XCD-contiguous ranges, then groups of 8 tile-rows ----
  const int nblocks = nbm * nbn;
  int bid = blockIdx.x;
  const int per_xcd = nblocks / 8;
  if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
  constexpr int kGroup = 8;
  const int group = bid / (kGroup * nbn);
  const int first_m = group * kGroup;
  const int gsize = min(nbm - first_m, kGroup);
  const int in_group = bid - group * kGroup * nbn;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t kbytes = K / 2, nkb = K / 32;
  const int nk = (int)((K + kBK - 1) / kBK);

  // global-load assignment: rows (t >> 2) + 64 i, chunk t & 3
  const int lrow = t >> 2, lchunk = t & 3;

  auto gload = [&](int ks, StepRegs& r) {
    const int64_t kb = (int64_t)ks * kRowBytes + lchunk * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.a[i] = load_chunk(A, M, kbytes, m0 + lrow + 64 * i, kb);
      r.b[i] = load_chunk(B, N, kbytes, n0 + lrow + 64 * i, kb);
    }
    r.sa = load_scales4(As, ga, M, nkb, m0 + t, (int64_t)ks * 4);
    r.sb = load_scales4(Bs, gb, N, nkb, n0 + t, (int64_t)ks * 4);
  };
  auto lstore = [&](int stage, const StepRegs& r) {
    uint8_t* st = smem + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 64 * i;
      *reinterpret_cast<uint4*>(st + swz(row, lchunk)) = r.a[i];
      *reinterpret_cast<uint4*>(st + kTileBytes + swz(row, lchunk)) = r.b[i];
    }
    reinterpret_cast<uint32_t*>(st + 2 * kTileBytes)[t] = r.sa;
    reinterpret_cast<uint32_t*>(st + 2 * kTileBytes + kBM * 4)[t] = r.sb;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  StepRegs regs;
  gload(0, regs);
  lstore(0, regs);
  __syncthreads();

  const int frow = lane & 31, fhalf = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) gload(ks + 1, regs);
    const uint8_t* st = smem + (ks & 1) * kStageBytes;
    const uint32_t* sA = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
    const uint32_t* sB = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + kBM * 4);
    uint32_t sca[4], scb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sca[i] = sA[wm * 128 + 32 * i + frow] >> (8 * fhalf);
      scb[i] = sB[wn * 128 + 32 * i + frow] >> (8 * fhalf);
    }
#pragma unroll
    for (int ki = 0; ki < 2; ++ki) {
      v8i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * 128 + 32 * i + frow;
        const int rb = wn * 128 + 32 * i + frow;
        const uint4 va = *reinterpret_cast<const uint4*>(st + swz(ra, 2 * ki + fhalf));
        const uint4 vb = *reinterpret_cast<const uint4*>(st + kTileBytes + swz(rb, 2 * ki + fhalf));
        af[i] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        bf[i] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ki == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[j], af[i], acc[i][j], 4, 4, 0, scb[j], 0, sca[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[j], af[i], acc[i][j], 4, 4, 2, scb[j], 2, sca[i]);
        }
    }
    if (ks + 1 < nk) lstore((ks + 1) & 1, regs);
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][r] = C[m][n], m = wm*128 + 32 i + (lane % 32),
  //      n = wn*128 + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4 ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + 32 * i + frow;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int64_t n = n0 + wn * 128 + 32 * j + 8 * rq + 4 * fhalf;
        if (n >= N) continue;
        const float v0 = acc[i][j][4 * rq + 0] * alpha_f;
        const float v1 = acc[i][j][4 * rq + 1] * alpha_f;
        const float v2 = acc[i][j][4 * rq + 2] * alpha_f;
        const float v3 = acc[i][j][4 * rq + 3] * alpha_f;
        if (out_bf16) {
          uint2 w;
          w.x = bf16_rne(v0) | (bf16_rne(v1) << 16);
          w.y = bf16_rne(v2) | (bf16_rne(v3) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + m * ldc + n) = w;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + m * ldc + n) =
              make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
}

}  // namespace

hipError_t mx_launch_gemm(const GemmArgs& g) {
  const int64_t nbm = (g.M + kBM - 1) / kBM, nbn = (g.N + kBN - 1) / kBN;
  if (nbm * nbn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float alpha_f = __builtin_bit_cast(float, (uint32_t)(g.alpha + 127) << 23);
  hipLaunchKernelGGL(gemm_mx_kernel, dim3((unsigned)(nbm * nbn)), dim3(kThreads), 0,
                     (hipStream_t)g.stream, g.a, g.as, g.ga, g.b, g.bs, g.gb, g.M, g.N, g.K,
                     alpha_f, g.out_bf16 ? 1 : 0, g.c, g.ldc, (int)nbm, (int)nbn);
  return hipGetLastError();
}
