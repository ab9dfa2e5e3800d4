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
// 4x4 MFMA tiles (256 fp32 accumulators per lane, in AGPRs). K advances 128 per step (64 bytes
// per row). Global loads (buffer loads over the operand tile; rows past the end read as zero)
// run two steps ahead in registers; LDS holds two stages of packed tiles plus their scale
// words, with a 16-byte chunk swizzle so that the fragment reads of 16 consecutive rows hit
// distinct banks. The barrier of a step sits between its two 64-wide k-halves so that LDS
// fragment reads overlap MFMAs on both sides of it. The B tile feeds the MFMA's first operand
// so a lane's 4 consecutive output registers are 4 consecutive columns of C.
#include "mx_device.h"
#include "mx_launch.h"

#include <type_traits>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 128;                 // k elements per step
constexpr int kRowBytes = kBK / 2;       // 64 bytes of codes per row per step
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kRowBytes;           // 16 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes + 2 * kBM * 4;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Buffer resource over bytes [base, base + bytes): loads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One k-step of global loads: 4 chunks of 16 bytes of A and of B per thread (rows
// (t >> 2) + 64 i, chunk t & 3) and the 4 scale bytes of row t of each operand.
struct StepRegs {
  u32x4 a[4], b[4];
  uint32_t sa, sb;
};

struct Frags {
  u32x4 a[4], b[4];  // 16 bytes = 32 FP4 values per lane (the MFMA reads 4 registers for FP4)
};

__device__ __forceinline__ v8i as_operand(const u32x4& v) {
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// Generic kernel (any K that is a multiple of 32): register-staged global loads. With
// KFULL (K a multiple of 128) every step is complete and each row's 4 scale bytes of a step
// form one aligned word; otherwise the last step is partial: its codes past K are zeroed and
// its missing scale bytes read as 127 (unit).
template <bool KFULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_generic_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, int lga,
                    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int lgb,
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
  const int lrow = t >> 2, lchunk = t & 3;
  const int frow = lane & 31, fhalf = lane >> 5;

  // operand tiles and their scale rows as buffer resources (32-bit offsets within a tile)
  const int64_t rows_a = min((int64_t)kBM, M - m0), rows_b = min((int64_t)kBN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + m0 * kbytes, rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + n0 * kbytes, rows_b * kbytes);
  const int64_t s0a = m0 >> lga, s0b = n0 >> lgb;
  const int64_t sbytes_a = (((m0 + rows_a - 1) >> lga) - s0a + 1) * nkb;
  const int64_t sbytes_b = (((n0 + rows_b - 1) >> lgb) - s0b + 1) * nkb;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(As + s0a * nkb, sbytes_a);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(Bs + s0b * nkb, sbytes_b);
  const int voff = (int)(lrow * kbytes) + 16 * lchunk;  // + i * 64 rows for chunk load i
  const int row_step = (int)(64 * kbytes);
  // scale row of thread t; rows past the operand point past the resource (read as zero)
  const int soff_a = t < rows_a ? (int)((((m0 + t) >> lga) - s0a) * nkb) : (int)sbytes_a;
  const int soff_b = t < rows_b ? (int)((((n0 + t) >> lgb) - s0b) * nkb) : (int)sbytes_b;

  auto scale4 = [&](__amdgpu_buffer_rsrc_t r, int off, int ks) -> uint32_t {
    if (KFULL) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 4 * ks, 0);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(r, off + i, 4 * ks, 0);
      byte = (4 * ks + i < nkb) ? byte : 0x7Fu;
      w |= byte << (8 * i);
    }
    return w;
  };
  auto gload = [&](int ks, StepRegs& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff + i * row_step, ks * kRowBytes, 0);
      r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff + i * row_step, ks * kRowBytes, 0);
    }
    if (!KFULL) {
      const bool past = 16 * lchunk + (int64_t)ks * kRowBytes >= kbytes;  // chunk beyond K
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r.a[i] = past ? u32x4{0u, 0u, 0u, 0u} : r.a[i];
        r.b[i] = past ? u32x4{0u, 0u, 0u, 0u} : r.b[i];
      }
    }
    r.sa = scale4(rsa, soff_a, ks);
    r.sb = scale4(rsb, soff_b, ks);
  };
  auto lstore = [&](int stage, const StepRegs& r) {
    uint8_t* st = smem + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 64 * i;
      *reinterpret_cast<u32x4*>(st + swz(row, lchunk)) = r.a[i];
      *reinterpret_cast<u32x4*>(st + kTileBytes + swz(row, lchunk)) = r.b[i];
    }
    reinterpret_cast<uint32_t*>(st + 2 * kTileBytes)[t] = r.sa;
    reinterpret_cast<uint32_t*>(st + 2 * kTileBytes + kBM * 4)[t] = r.sb;
  };
  // fragments of k-half ki (64 k values) of a stage
  auto lread = [&](int stage, int ki, Frags& f) {
    const uint8_t* st = smem + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = *reinterpret_cast<const u32x4*>(st + swz(wm * 128 + 32 * i + frow, 2 * ki + fhalf));
      f.b[i] = *reinterpret_cast<const u32x4*>(st + kTileBytes +
                                               swz(wn * 128 + 32 * i + frow, 2 * ki + fhalf));
    }
  };
  // per-lane scale words: lanes 0-31 use k-blocks 0 and 2 of the step, lanes 32-63 k-blocks
  // 1 and 3, so shift the word by one byte on the upper half; op_sel 0 / 2 then picks the
  // byte of the first / second k-half
  auto sread = [&](int stage, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
    const uint8_t* st = smem + stage * kStageBytes;
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + kBM * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = pa[wm * 128 + 32 * i + frow] >> (8 * fhalf);
      sb[i] = pb[wn * 128 + 32 * i + frow] >> (8 * fhalf);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mma = [&](const Frags& f, const uint32_t (&sa)[4], const uint32_t (&sb)[4], auto opsel) {
    constexpr int OP = decltype(opsel)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_operand(f.b[j]), as_operand(f.a[i]), acc[i][j], 4, 4, OP, sb[j], OP, sa[i]);
  };
  using Op0 = std::integral_constant<int, 0>;
  using Op2 = std::integral_constant<int, 2>;

  // Step ks: issue loads for ks+2; read the second k-half of stage ks; MFMAs of the first half;
  // store step ks+1 (loaded during step ks-1) into the other stage; barrier; read scales and
  // the first half of stage ks+1; MFMAs of the second half of ks.
  StepRegs Rn, Rf;  // Rn: step ks+1 in flight/landed; Rf: free for step ks+2
  Frags F0, F1;
  uint32_t saC[4], sbC[4], saN[4], sbN[4];
  gload(0, Rf);
  if (nk > 1) gload(1, Rn);
  lstore(0, Rf);
  __syncthreads();
  sread(0, saC, sbC);
  lread(0, 0, F0);

#pragma unroll 1
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 2 < nk) gload(ks + 2, Rf);
    lread(ks & 1, 1, F1);
    mma(F0, saC, sbC, Op0{});
    if (ks + 1 < nk) lstore((ks + 1) & 1, Rn);
    __syncthreads();
    if (ks + 1 < nk) {
      sread((ks + 1) & 1, saN, sbN);
      lread((ks + 1) & 1, 0, F0);
    }
    mma(F1, saC, sbC, Op2{});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      saC[i] = saN[i];
      sbC[i] = sbN[i];
    }
    const StepRegs tmp = Rn;  // the set loaded for ks+2 becomes the next "in flight" set
    Rn = Rf;
    Rf = tmp;
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

// ---------------------------------------------------------------------------------------------
// Streaming kernel for K a multiple of 128: a 4-stage LDS ring filled by direct-to-LDS buffer
// loads (no register staging). Each wave issues 10 loads per step (4 + 4 code chunks of 1 KiB,
// 2 scale words of 256 B); loads run two steps ahead of use. The code tiles land in LDS in the
// swizzled order: lane l of load i of wave w fills 16-byte slot s = 64 (4 i + w) + l, i.e. row
// s / 4, position s % 4, which holds k-chunk (s % 4) ^ ((row / 4) & 3) of that row.
// ---------------------------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (base, stride 0, num_records, CDNA data-format word).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, (int)bytes, 0x00020000};
}

// Direct-to-LDS buffer loads: lane l's 16 (or 4) bytes land at LDS address lds + 16 l (4 l).
// Issued through asm so that the compiler inserts no waits for them; the kernel waits on
// vmcnt explicitly before each barrier.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_b32(i32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_stream_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, int lga,
                           const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int lgb,
                           int64_t M, int64_t N, int64_t K, float alpha_f, int out_bf16,
                           void* __restrict__ C, int64_t ldc, int nbm, int nbn) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStageBytes];

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
  const int nk = (int)(K / kBK);
  const int frow = lane & 31, fhalf = lane >> 5;

  const int64_t rows_a = min((int64_t)kBM, M - m0), rows_b = min((int64_t)kBN, N - n0);
  const i32x4 ra = rsrc_words(A + m0 * kbytes, rows_a * kbytes);
  const i32x4 rb = rsrc_words(B + n0 * kbytes, rows_b * kbytes);
  const int64_t s0a = m0 >> lga, s0b = n0 >> lgb;
  const int64_t sbytes_a = (((m0 + rows_a - 1) >> lga) - s0a + 1) * nkb;
  const int64_t sbytes_b = (((n0 + rows_b - 1) >> lgb) - s0b + 1) * nkb;
  const i32x4 rsa = rsrc_words(As + s0a * nkb, sbytes_a);
  const i32x4 rsb = rsrc_words(Bs + s0b * nkb, sbytes_b);
  // code slot of this lane in load i: row 16 (4 i + wave) + lane / 4, k-chunk as in swz()
  const int crow = 16 * wave + (lane >> 2);
  const int cchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int voff = (int)(crow * kbytes) + 16 * cchunk;  // + i * 64 rows for load i
  const int row_step = (int)(64 * kbytes);
  // scale word of row 64 wave + lane
  const int srow = 64 * wave + lane;
  const int soff_a = srow < rows_a ? (int)((((m0 + srow) >> lga) - s0a) * nkb) : (int)sbytes_a;
  const int soff_b = srow < rows_b ? (int)((((n0 + srow) >> lgb) - s0b) * nkb) : (int)sbytes_b;

  auto issue = [&](uint8_t* st, int ks) {
    const int kofs = ks * kRowBytes;
    const uint32_t base = lds_addr(st + 1024 * wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma_b128(ra, base + 4096 * i, voff + i * row_step, kofs);
      dma_b128(rb, base + 4096 * i + kTileBytes, voff + i * row_step, kofs);
    }
    const uint32_t sbase = lds_addr(st + 2 * kTileBytes + 256 * wave);
    dma_b32(rsa, sbase, soff_a, 4 * ks);
    dma_b32(rsb, sbase + kBM * 4, soff_b, 4 * ks);
  };
  auto lread = [&](const uint8_t* st, int ki, Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = *reinterpret_cast<const u32x4*>(st + swz(wm * 128 + 32 * i + frow, 2 * ki + fhalf));
      f.b[i] = *reinterpret_cast<const u32x4*>(st + kTileBytes +
                                               swz(wn * 128 + 32 * i + frow, 2 * ki + fhalf));
    }
  };
  auto sread = [&](const uint8_t* st, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
    const uint32_t* pa = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
    const uint32_t* pb = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + kBM * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = pa[wm * 128 + 32 * i + frow] >> (8 * fhalf);
      sb[i] = pb[wn * 128 + 32 * i + frow] >> (8 * fhalf);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mma = [&](const Frags& f, const uint32_t (&sa)[4], const uint32_t (&sb)[4], auto opsel) {
    constexpr int OP = decltype(opsel)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_operand(f.b[j]), as_operand(f.a[i]), acc[i][j], 4, 4, OP, sb[j], OP, sa[i]);
  };
  using Op0 = std::integral_constant<int, 0>;
  using Op2 = std::integral_constant<int, 2>;

  Frags F0, F1;
  uint32_t saC[4], sbC[4], saN[4], sbN[4];

  // Every step issues exactly 10 loads per wave (steps past the end re-read step nk-1 into a
  // stage nobody reads again), so the wait before each barrier is always "all but the newest
  // 10", i.e. the step about to be read has landed, and the loop body has no branches.
  auto issue_step = [&](uint8_t* st, int ks) { issue(st, min(ks, nk - 1)); };

  // prologue: steps 0, 1, 2 in flight; wait for step 0 everywhere
  issue_step(st0, 0);
  issue_step(st1, 1);
  issue_step(st2, 2);
  wait_vmcnt<20>();
  __builtin_amdgcn_s_barrier();
  sread(st0, saC, sbC);
  lread(st0, 0, F0);

  // step ks on stage cur: read its second k-half; MFMAs of the first half; wait until step ks+1
  // has landed (own loads; the barrier covers the other waves) and every wave has finished
  // reading stage ks-1; refill that stage with step ks+3; read the first half and scales of
  // ks+1; MFMAs of the second half of ks.
  auto body = [&](int ks, const uint8_t* cur, const uint8_t* nxt, uint8_t* refill) {
    lread(cur, 1, F1);
    mma(F0, saC, sbC, Op0{});
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<10>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage ks are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_step(refill, ks + 3);
    sread(nxt, saN, sbN);
    lread(nxt, 0, F0);
    mma(F1, saC, sbC, Op2{});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      saC[i] = saN[i];
      sbC[i] = sbN[i];
    }
  };
  int ks = 0;
#pragma unroll 1
  for (; ks + 4 <= nk; ks += 4) {
    body(ks, st0, st1, st3);
    body(ks + 1, st1, st2, st0);
    body(ks + 2, st2, st3, st1);
    body(ks + 3, st3, st0, st2);
  }
  if (ks < nk) body(ks, st0, st1, st3);
  if (ks + 1 < nk) body(ks + 1, st1, st2, st0);
  if (ks + 2 < nk) body(ks + 2, st2, st3, st1);
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

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
  // buffer offsets are 32-bit: one 256-row operand tile must stay below 2 GiB
  if ((int64_t)kBM * (g.K / 2) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const float alpha_f = __builtin_bit_cast(float, (uint32_t)(g.alpha + 127) << 23);
  const int lga = g.ga == 32 ? 5 : 0, lgb = g.gb == 32 ? 5 : 0;
  const dim3 grid((unsigned)(nbm * nbn));
  if (g.K % kBK == 0 && g.K > 0)
    hipLaunchKernelGGL(gemm_mx_stream_kernel, grid, dim3(kThreads), 0, (hipStream_t)g.stream, g.a,
                       g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0, g.c,
                       g.ldc, (int)nbm, (int)nbn);
  else
    hipLaunchKernelGGL(gemm_mx_generic_kernel<false>, grid, dim3(kThreads), 0, (hipStream_t)g.stream, g.a,
                       g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0, g.c,
                       g.ldc, (int)nbm, (int)nbn);
  return hipGetLastError();
}
