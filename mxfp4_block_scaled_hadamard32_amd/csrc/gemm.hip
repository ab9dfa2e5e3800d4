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
// Matrix-core facts used (gfx950 V_MFMA_SCALE_F32_32X32X64_F8F6F4; pinned on hardware by
// single-instruction probes with random operands and scales):
//  * FP4 operands: lane l holds row (l % 32) and k = 32 * (l / 32) .. +31 of a 32x64 slice,
//    as 16 bytes, element 2i in the low nibble of byte i;
//  * FP8 operands: lane l holds 32 bytes of row (l % 32): bytes 0-15 are 16 values of k-block
//    0 and bytes 16-31 16 values of k-block 1 (which half of each block a lane holds only has
//    to agree between the two operands; here lane half h holds k 16h .. 16h+15 of each);
//  * the 32-bit scale operand of lane l carries the E8M0 byte of k-block (l / 32) of row
//    l % 32; the op_sel immediate picks which byte of the register is used;
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 128;                 // k elements per step
constexpr int kRowBytes = kBK / 2;       // 64 bytes of codes per row per step
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kRowBytes;           // 16 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes + 2 * kBM * 4;
constexpr int kStreamWaves = 4;  // waves per workgroup of the streaming kernel (4 or 8)

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

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

__device__ __forceinline__ v8i as_operand(const u32x4& v) {
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8i as_operand(const u32x8& v) { return __builtin_bit_cast(v8i, v); }

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

  // ---- tile schedule: XCD-contiguous ranges, then groups of 4 tile-rows ----
  const int nblocks = nbm * nbn;
  int bid = blockIdx.x;
  const int per_xcd = nblocks / 8;
  if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
  constexpr int kGroup = 4;
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

// Streaming kernel, templated on the k-extent of one LDS stage. BKS = number of 64-wide k
// sub-steps per stage: 2 (128 k = 64 bytes per row) with 4 stages, or 4 (256 k = 128 bytes per
// row) with 2 stages. With 128-byte rows every direct load instruction covers whole 128-byte
// lines (8 rows x 128 B), which quarters the number of L1->L2 requests per byte compared with
// 64-byte row pieces; the L2 request rate, not its bandwidth, is what bounds this kernel.
// WAVES = 4: one wave per SIMD, each wave owns 128x128 (4x4 MFMA tiles, 256 accumulators).
// WAVES = 8: two waves per SIMD, each wave owns 64x128 (2x4 MFMA tiles).
template <int WAVES, int BKS, int STAGES, bool F8 = false>
struct StreamCfg {
  static constexpr int kRow = 32 * BKS;                         // code bytes per row per stage
  static constexpr int kTile = kBM * kRow;                      // per operand
  static constexpr int kKStage = F8 ? kRow : 2 * kRow;          // k elements per stage
  static constexpr int kSub = kKStage / 64;                     // 64-wide MFMA k sub-steps
  static constexpr int kScaleRow = kKStage / 32;                // scale bytes per row per stage
  // BKS == 4: scales do not travel with the stage. A separate double-buffered area holds 4
  // steps (32 bytes) of scales per row, fetched as 32-byte pieces (one L2 request per row per
  // 4 steps instead of one per step); each step brings in one quarter of the next group.
  static constexpr bool kGroupScales = BKS == 4;
  static constexpr int kGroupSteps = 4;
  static constexpr int kGroupRow = kGroupSteps * kScaleRow;     // 32 bytes
  static constexpr int kGroupBytes = 2 * kBM * kGroupRow;       // both operands, 16 KiB
  static constexpr int kStage = 2 * kTile + (kGroupScales ? 0 : 2 * kBM * kScaleRow);
  static constexpr int kLds = STAGES * kStage + (kGroupScales ? 2 * kGroupBytes : 0);
  static constexpr int kRowsPerBlock = 1024 / kRow;             // rows per 1 KiB code load
  static constexpr int kCodeLoads = kBM / kRowsPerBlock / WAVES;  // per operand per wave
  // a group quarter (128 rows x kGroupRow bytes) is split evenly over the waves: one 16-byte
  // load per lane for 32-byte FP4 rows with 4 waves, otherwise 4-byte loads (there is no
  // 8-byte direct load)
  static constexpr int kGroupLaneBytes = (WAVES == 4 && !F8) ? 16 : 4;
  static constexpr int kGroupLoads = kGroupBytes / 4 / WAVES / (64 * kGroupLaneBytes);
  static constexpr int kScaleLoads = kGroupScales ? kGroupLoads
                                                  : 2 * (kBM * kScaleRow / 256) / WAVES;
  static constexpr int kLoads = 2 * kCodeLoads + kScaleLoads;
  // FP4 scale groups (32-byte rows, two 16-byte halves of two steps each): row r keeps its
  // halves swapped when bit 3 of r is set. A step's scale reads hit 32 consecutive rows at one
  // offset; with plain 32-byte rows every 8th row shares a bank (4-way conflicts), with the swap
  // rows r and r + 8 use different banks (2-way), and each direct load still moves whole halves.
  static constexpr bool kScaleSwap = kGroupScales && kGroupRow == 32;
  __device__ static __forceinline__ int scale_swap(int row) {
    return kScaleSwap ? ((row >> 3) & 1) << 4 : 0;
  }
  static constexpr int kSwzShift = BKS == 2 ? 2 : 1;            // rows sharing a bank phase
  // byte offset of 16-byte chunk `chunk` of row `row` in a stage's code tile: the chunk
  // position is XOR-ed with a row phase so that 16 consecutive rows hit distinct bank groups
  __device__ static __forceinline__ int swz(int row, int chunk) {
    return row * kRow + ((chunk ^ ((row >> kSwzShift) & (2 * BKS - 1))) << 4);
  }
};

// AF, BF: matrix-core element formats of A and B (4 = E2M1, packed two per byte; 0 = E4M3,
// 1 = E5M2, one per byte). Both operands have the same width. With 8-bit elements a stage
// holds half the k of the FP4 stage in the same bytes, and one MFMA (64 k) reads 32 bytes per
// lane instead of 16 but takes twice as many cycles, so the bytes per MFMA cycle, the load
// schedule and the LDS layout stay those of the FP4 kernel.
template <int WAVES, int BKS, int STAGES, int SPLIT3 = 0, int SPLIT0 = 0, int SPLIT1 = 0,
          bool QOUT = false, int AF = 4, int BF = 4>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void gemm_mx_stream_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, int lga,
                           const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int lgb,
                           int64_t M, int64_t N, int64_t K, float alpha_f, int out_bf16,
                           void* __restrict__ C, int64_t ldc, int nbm, int nbn,
                           GemmQuantOut qo) {
  constexpr bool F8 = AF != 4;
  static_assert(F8 == (BF != 4), "both operands 4-bit or both 8-bit");
  using Cfg = StreamCfg<WAVES, BKS, STAGES, F8>;
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  static_assert((BKS == 2 && STAGES == 4) || (BKS == 4 && STAGES == 2), "stage shapes");
  static_assert(!F8 || (BKS == 4 && !QOUT), "8-bit operands: 128-byte stages, plain output");
  constexpr int FA = WAVES == 4 ? 4 : 2;   // 32-row A fragments per wave
  constexpr int FB = 4;                    // 32-row B fragments per wave
  constexpr int WM = kBM / (32 * FA);      // waves along M
  constexpr int SW = Cfg::kScaleRow / 4;   // scale words per row per stage
  constexpr int NSUB = Cfg::kSub;          // MFMA k sub-steps per stage
  using Frag = std::conditional_t<F8, u32x8, u32x4>;
  constexpr int LOADS = Cfg::kLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::kLds];
  uint8_t* const sgroup = smem + STAGES * Cfg::kStage;  // scale groups (BKS == 4)

  const int nblocks = nbm * nbn;
  // Tiles blockIdx.x, blockIdx.x + gridDim.x, ...: a resident grid (one workgroup per CU, a
  // multiple of 8, so tile t stays on XCD t % 8 as the ordering below assumes) walks the tiles
  // in the same order as a grid of one workgroup per tile, without a dispatch gap between them.
  for (int tile = blockIdx.x; tile < nblocks; tile += gridDim.x) {
    int bid = tile;
    const int per_xcd = nblocks / 8;
    if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
    constexpr int kGroup = 4;
    const int group = bid / (kGroup * nbn);
    const int first_m = group * kGroup;
    const int gsize = min(nbm - first_m, kGroup);
    const int in_group = bid - group * kGroup * nbn;
    const int tm = first_m + in_group % gsize;
    const int tn = in_group / gsize;
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

    int t = threadIdx.x;
    asm volatile("" : "+v"(t));  // per tile: keep lane setup out of the loop-carried state
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int64_t kbytes = F8 ? K : K / 2, nkb = K / 32;
    const int nk = (int)(K / Cfg::kKStage);
    const int frow = lane & 31, fhalf = lane >> 5;

    const int64_t rows_a = min((int64_t)kBM, M - m0), rows_b = min((int64_t)kBN, N - n0);
    const i32x4 ra = rsrc_words(A + m0 * kbytes, rows_a * kbytes);
    const i32x4 rb = rsrc_words(B + n0 * kbytes, rows_b * kbytes);
    const int64_t s0a = m0 >> lga, s0b = n0 >> lgb;
    const int64_t sbytes_a = (((m0 + rows_a - 1) >> lga) - s0a + 1) * nkb;
    const int64_t sbytes_b = (((n0 + rows_b - 1) >> lgb) - s0b + 1) * nkb;
    const i32x4 rsa = rsrc_words(As + s0a * nkb, sbytes_a);
    const i32x4 rsb = rsrc_words(Bs + s0b * nkb, sbytes_b);

    // code load i of this wave fills 1 KiB block b = i * WAVES + wave of the tile: rows
    // kRowsPerBlock * b + lane / (2 BKS), position lane % (2 BKS), i.e. chunk position ^ phase
    int voff[Cfg::kCodeLoads];
#pragma unroll
    for (int i = 0; i < Cfg::kCodeLoads; ++i) {
      const int b = i * WAVES + wave;
      const int row = Cfg::kRowsPerBlock * b + lane / (2 * BKS);
      const int pos = lane % (2 * BKS);
      const int chunk = pos ^ ((row >> Cfg::kSwzShift) & (2 * BKS - 1));
      voff[i] = (int)(row * kbytes) + 16 * chunk;
    }
    // scale load j of this wave: 256-byte piece q of operand o (rows of 2 BKS bytes, lane ->
    // row piece * (128 / BKS) + lane / SW, word lane % SW); rows past the operand read zero
    constexpr int kPieces = kBM * Cfg::kScaleRow / 256;  // per operand
    int soff[Cfg::kGroupScales ? 1 : Cfg::kScaleLoads];
    if constexpr (!Cfg::kGroupScales) {
      if constexpr (!Cfg::kGroupScales)
#pragma unroll
      for (int j = 0; j < Cfg::kScaleLoads; ++j) {
        const int sidx = wave + j * WAVES;
        const int o = sidx / kPieces, q = sidx % kPieces;
        const int row = q * (128 / BKS) + lane / SW;
        const int word = lane % SW;
        if (o == 0)
          soff[j] = row < rows_a ? (int)((((m0 + row) >> lga) - s0a) * nkb) + 4 * word : (int)sbytes_a;
        else
          soff[j] = row < rows_b ? (int)((((n0 + row) >> lgb) - s0b) * nkb) + 4 * word : (int)sbytes_b;
      }
    }
    // group mode: quarter p of a group holds rows 128 p .. 128 p + 127 of the 512 scale rows
    // (A rows 0-255, then B), 32 bytes each. Load h of wave w covers bytes
    // (w G + h) 64 LB .. +64 LB of the quarter (G loads per wave, LB bytes per lane), so lane l
    // fetches byte (q % 32) ^ scale_swap(row) of row 128 p + q / 32 for q = ((w G + h) 64 + l) LB.
    // Quarters 0-1 are A rows, 2-3 are B rows, so the operand depends on p only.
    constexpr int kGL = Cfg::kGroupLoads, kLB = Cfg::kGroupLaneBytes;
    int goff[4][Cfg::kGroupScales ? kGL : 1];
    if constexpr (Cfg::kGroupScales) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int h = 0; h < kGL; ++h) {
          const int q = ((wave * kGL + h) * 64 + lane) * kLB;
          const int row = (128 * p + q / Cfg::kGroupRow) & (kBM - 1);
          const int byte = (q % Cfg::kGroupRow) ^ Cfg::scale_swap(row);
          if (p < 2)
            goff[p][h] = row < rows_a ? (int)((((m0 + row) >> lga) - s0a) * nkb) + byte : (int)sbytes_a;
          else
            goff[p][h] = row < rows_b ? (int)((((n0 + row) >> lgb) - s0b) * nkb) + byte : (int)sbytes_b;
        }
    }
    const int ngroups = (nk + Cfg::kGroupSteps - 1) / Cfg::kGroupSteps;
    // load h of quarter p of scale group g into buffer g % 2 (groups past the end re-read the
    // last one)
    auto issue_group_load = [&](int g, int p, int h) {
      const int gs = min(g, ngroups - 1);
      const uint32_t dst = lds_addr(sgroup + (g & 1) * Cfg::kGroupBytes + 128 * p * Cfg::kGroupRow +
                                    (wave * kGL + h) * 64 * kLB);
      const i32x4 sel = p < 2 ? rsa : rsb;
      if constexpr (kLB == 16) dma_b128(sel, dst, goff[p][h], gs * Cfg::kGroupRow);
      else dma_b32(sel, dst, goff[p][h], gs * Cfg::kGroupRow);
    };
    auto issue_group_part = [&](int g, int p) {
#pragma unroll
      for (int h = 0; h < kGL; ++h) issue_group_load(g, p, h);
    };

    auto stage_ptr = [&](int st) { return smem + st * Cfg::kStage; };
    auto issue = [&](uint8_t* st, int ks) {
      const int kofs = ks * Cfg::kRow;
#pragma unroll
      for (int i = 0; i < Cfg::kCodeLoads; ++i) {
        const uint32_t dst = lds_addr(st + 1024 * (i * WAVES + wave));
        dma_b128(ra, dst, voff[i], kofs);
        dma_b128(rb, dst + Cfg::kTile, voff[i], kofs);
      }
      if constexpr (!Cfg::kGroupScales)
#pragma unroll
      for (int j = 0; j < Cfg::kScaleLoads; ++j) {
        const int sidx = wave + j * WAVES;
        const int o = sidx / kPieces, q = sidx % kPieces;
        const uint32_t dst = lds_addr(st + 2 * Cfg::kTile + o * kBM * Cfg::kScaleRow + 256 * q);
        const i32x4 sel = o == 0 ? rsa : rsb;  // wave-uniform; pin it to scalar registers
        const i32x4 rs = {__builtin_amdgcn_readfirstlane(sel.x), __builtin_amdgcn_readfirstlane(sel.y),
                          __builtin_amdgcn_readfirstlane(sel.z), __builtin_amdgcn_readfirstlane(sel.w)};
        dma_b32(rs, dst, soff[j], ks * Cfg::kScaleRow);
      }
    };
    // a lane's fragment of sub-step sub (64 k values of one row): FP4, the 32 values of k-block
    // fhalf (16 bytes, chunk 2 sub + fhalf); FP8, 16 values of each k-block, the half fhalf of
    // block 0 in bytes 0-15 and of block 1 in bytes 16-31 (chunks 4 sub + fhalf and
    // 4 sub + 2 + fhalf)
    auto frag = [&](const uint8_t* tile, int row, int sub) -> Frag {
      if constexpr (F8) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + Cfg::swz(row, 4 * sub + fhalf));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + Cfg::swz(row, 4 * sub + 2 + fhalf));
        return u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        return *reinterpret_cast<const u32x4*>(tile + Cfg::swz(row, 2 * sub + fhalf));
      }
    };
    auto lread = [&](const uint8_t* st, int sub, Frag (&fa)[FA], Frag (&fb)[FB]) {
#pragma unroll
      for (int i = 0; i < FA; ++i) fa[i] = frag(st, wm * 32 * FA + 32 * i + frow, sub);
#pragma unroll
      for (int j = 0; j < FB; ++j) fb[j] = frag(st + Cfg::kTile, wn * 32 * FB + 32 * j + frow, sub);
    };
    // per-lane scale words of a stage: word w holds k-blocks 4w..4w+3 of the row; lanes 0-31
    // use the even blocks, lanes 32-63 the odd ones, so shift by one byte on the upper half and
    // let op_sel 0 / 2 pick sub-step 2w / 2w+1
    auto sread = [&](const uint8_t* st, int ks, uint32_t (&sa)[FA][SW], uint32_t (&sb)[FB][SW]) {
      const uint32_t* pa;
      const uint32_t* pb;
      int stride;  // words per row
      if constexpr (Cfg::kGroupScales) {
        // rows wm * 32 FA + 32 i + frow all have bit 3 of frow, so the half swap is per lane
        const int soff = ((ks % Cfg::kGroupSteps) * Cfg::kScaleRow) ^ Cfg::scale_swap(frow);
        const uint8_t* gb = sgroup + ((ks / Cfg::kGroupSteps) & 1) * Cfg::kGroupBytes + soff;
        pa = reinterpret_cast<const uint32_t*>(gb);
        pb = reinterpret_cast<const uint32_t*>(gb + kBM * Cfg::kGroupRow);
        stride = Cfg::kGroupRow / 4;
      } else {
        pa = reinterpret_cast<const uint32_t*>(st + 2 * Cfg::kTile);
        pb = reinterpret_cast<const uint32_t*>(st + 2 * Cfg::kTile + kBM * Cfg::kScaleRow);
        stride = SW;
      }
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int w = 0; w < SW; ++w) sa[i][w] = pa[(wm * 32 * FA + 32 * i + frow) * stride + w] >> (8 * fhalf);
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int w = 0; w < SW; ++w) sb[j][w] = pb[(wn * 32 * FB + 32 * j + frow) * stride + w] >> (8 * fhalf);
    };

    v16f acc[FA][FB];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // MFMAs of sub-step SUB: scale word SUB / 2, byte pair selected by op_sel 2 * (SUB % 2)
    auto mma = [&](const Frag (&fa)[FA], const Frag (&fb)[FB], const uint32_t (&sa)[FA][SW],
                   const uint32_t (&sb)[FB][SW], auto sub) {
      constexpr int SUB = decltype(sub)::value;
      constexpr int OP = 2 * (SUB % 2), W = SUB / 2;
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              as_operand(fb[j]), as_operand(fa[i]), acc[i][j], BF, AF, OP, sb[j][W], OP, sa[i][W]);
    };

    Frag fa0[FA], fb0[FB], fa1[FA], fb1[FB];
    uint32_t saC[FA][SW], sbC[FB][SW], saN[FA][SW], sbN[FB][SW];

    // Every step issues exactly LOADS loads per wave (steps past the end re-read step nk-1 into
    // a stage nobody reads again), so each wait is a constant count and the loop has no branches.
    auto issue_step = [&](uint8_t* st, int ks) { issue(st, min(ks, nk - 1)); };

    // Group mode schedule: the load bundle of step j (its code loads, issued two steps ahead)
    // also carries quarter (j + 3) % 4 of scale group (j + 3) / 4, so group G arrives with the
    // bundles of steps 4G-3 .. 4G. That makes it complete (loads retire in order) when the
    // scales of step 4G are first read, at the barrier of step 4G-1, and its first quarter is
    // requested only after the barrier of step 4G-5, after which nobody reads the previous
    // occupant of its buffer (group G-2) any more. Quarters 0-2 of group 0 go out on their own.
    auto issue_bundle = [&](uint8_t* st, int j) {
      issue_step(st, j);
      if constexpr (Cfg::kGroupScales) issue_group_part((j + 3) / 4, (j + 3) % 4);
    };
    // Spread schedule (2 stages): load L of bundle j (L < S: load L of its scale quarter, S the
    // number of scale loads per step; L = S + q: code load q / 2 of operand q % 2) is issued
    // between MFMAs instead of in one burst after the
    // barrier, so that a full address queue stalls a single load rather than the whole sub-step.
    // Loads 0 .. kP3-1 go out during the last sub-step of step j-2 (right after its barrier),
    // the rest during sub-steps 0 .. 2 of step j-1; all of them land by the barrier of step j-1.
    // FP4: at most one load per pair of MFMAs; FP8 (MFMAs twice as long): one per MFMA
    constexpr int kPer = F8 ? 1 : 2;
    constexpr int kP3 = SPLIT3, kP0 = SPLIT0, kP1 = SPLIT1, kP2 = LOADS - kP3 - kP0 - kP1;
    static_assert(STAGES != 2 || (kP2 >= 0 && kPer * kP3 <= FA * FB && kPer * kP0 <= FA * FB &&
                  kPer * kP1 <= FA * FB && kPer * kP2 <= FA * FB), "loads per sub-step");
    static_assert(STAGES != 2 || NSUB == 4 || (NSUB == 2 && kP1 == 0 && kP2 == 0),
                  "two sub-steps: all loads in sub-steps 1 and 0");
    auto issue_load = [&](uint8_t* st, int j, int L) {
      if (L < Cfg::kScaleLoads) {
        issue_group_load((j + 3) / 4, (j + 3) % 4, L);
      } else {
        const int q = L - Cfg::kScaleLoads, i = q >> 1;
        const uint32_t dst = lds_addr(st + 1024 * (i * WAVES + wave)) + ((q & 1) ? Cfg::kTile : 0);
        dma_b128((q & 1) ? rb : ra, dst, voff[i], min(j, nk - 1) * Cfg::kRow);
      }
    };
    // the same MFMAs with loads FIRST .. FIRST+CNT-1 of bundle j (into stage st) issued after
    // every second MFMA
    auto mma_mix = [&](const Frag (&fa)[FA], const Frag (&fb)[FB], const uint32_t (&sa)[FA][SW],
                       const uint32_t (&sb)[FB][SW], auto sub, uint8_t* st, int j, auto first,
                       auto count) {
      constexpr int SUB = decltype(sub)::value;
      constexpr int OP = 2 * (SUB % 2), W = SUB / 2;
      constexpr int FIRST = decltype(first)::value, CNT = decltype(count)::value;
      static_for<FA * FB>([&](auto nn) {
        constexpr int n = decltype(nn)::value, i = n / FB, jj = n % FB;
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_operand(fb[jj]), as_operand(fa[i]), acc[i][jj], BF, AF, OP, sb[jj][W], OP, sa[i][W]);
        if constexpr (n % kPer == kPer - 1 && n / kPer < CNT) {
          issue_load(st, j, FIRST + n / kPer);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };

    if constexpr (Cfg::kGroupScales) {
      issue_group_part(0, 0);
      issue_group_part(0, 1);
      issue_group_part(0, 2);
    }
    if constexpr (STAGES == 2) {
      static_for<LOADS>([&](auto L) { issue_load(stage_ptr(0), 0, decltype(L)::value); });
      static_for<kP3>([&](auto L) { issue_load(stage_ptr(1), 1, decltype(L)::value); });
      wait_vmcnt<kP3>();
    } else {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue_bundle(stage_ptr(s), s);
      wait_vmcnt<(STAGES - 1) * LOADS>();
    }
    __builtin_amdgcn_s_barrier();
    sread(stage_ptr(0), 0, saC, sbC);
    lread(stage_ptr(0), 0, fa0, fb0);

    // Step ks on stage cur: sub-steps 0 .. BKS-1, fragments read one sub-step ahead (ping-pong
    // fa0/fb0, fa1/fb1). Before the MFMAs of the last sub-step: wait until step ks+1 has landed
    // (own loads; the barrier covers the other waves; steps ks+2 .. ks+STAGES-1 may still be in
    // flight); every wave then holds all of stage ks in registers, so the stage is refilled at
    // once with step ks+STAGES; the scales and first sub-step of ks+1 are read meanwhile.
    auto body = [&](int ks, uint8_t* cur, const uint8_t* nxt) {
      static_for<NSUB>([&](auto sub) {
        constexpr int S = decltype(sub)::value;
        if constexpr (S + 1 < NSUB) {
          if constexpr (S % 2 == 0) lread(cur, S + 1, fa1, fb1);
          else lread(cur, S + 1, fa0, fb0);
        } else {
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<(STAGES - 2) * LOADS>();
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage ks are done
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          issue_bundle(cur, ks + STAGES);
          sread(nxt, ks + 1, saN, sbN);
          lread(nxt, 0, fa0, fb0);  // the last sub-step (odd) uses fa1/fb1
        }
        if constexpr (S % 2 == 0) mma(fa0, fb0, saC, sbC, sub);
        else mma(fa1, fb1, saC, sbC, sub);
        __builtin_amdgcn_sched_barrier(0);  // keep one sub-step of fragments live at a time
      });
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int w = 0; w < SW; ++w) saC[i][w] = saN[i][w];
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int w = 0; w < SW; ++w) sbC[j][w] = sbN[j][w];
    };
    // Two-stage step ks on stage cur with the spread schedule: sub-steps 0 .. 2 carry the rest of
    // bundle ks+1 (into nxt), the last sub-step starts bundle ks+2 (into cur) after the barrier.
    auto body2 = [&](int ks, uint8_t* cur, uint8_t* nxt) {
      static_for<NSUB>([&](auto sub) {
        constexpr int S = decltype(sub)::value;
        if constexpr (S + 1 < NSUB) {
          constexpr int first = S == 0 ? kP3 : S == 1 ? kP3 + kP0 : kP3 + kP0 + kP1;
          constexpr int cnt = S == 0 ? kP0 : S == 1 ? kP1 : kP2;
          if constexpr (S % 2 == 0) {
            lread(cur, S + 1, fa1, fb1);
            mma_mix(fa0, fb0, saC, sbC, sub, nxt, ks + 1, std::integral_constant<int, first>{},
                    std::integral_constant<int, cnt>{});
          } else {
            lread(cur, S + 1, fa0, fb0);
            mma_mix(fa1, fb1, saC, sbC, sub, nxt, ks + 1, std::integral_constant<int, first>{},
                    std::integral_constant<int, cnt>{});
          }
        } else {
          static_assert(NSUB % 2 == 0, "last sub-step uses fa1/fb1");
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<0>();
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage ks are done
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          sread(nxt, ks + 1, saN, sbN);
          lread(nxt, 0, fa0, fb0);
          mma_mix(fa1, fb1, saC, sbC, sub, cur, ks + 2, std::integral_constant<int, 0>{},
                  std::integral_constant<int, kP3>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int w = 0; w < SW; ++w) saC[i][w] = saN[i][w];
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int w = 0; w < SW; ++w) sbC[j][w] = sbN[j][w];
    };
    int ks = 0;
    if constexpr (STAGES == 4) {
#pragma unroll 1
      for (; ks + 4 <= nk; ks += 4) {
        body(ks, stage_ptr(0), stage_ptr(1));
        body(ks + 1, stage_ptr(1), stage_ptr(2));
        body(ks + 2, stage_ptr(2), stage_ptr(3));
        body(ks + 3, stage_ptr(3), stage_ptr(0));
      }
      if (ks < nk) body(ks, stage_ptr(0), stage_ptr(1));
      if (ks + 1 < nk) body(ks + 1, stage_ptr(1), stage_ptr(2));
      if (ks + 2 < nk) body(ks + 2, stage_ptr(2), stage_ptr(3));
    } else {
      // one step per iteration with computed stage pointers: unrolling two steps here doubles
      // the live fragment registers and spills
#pragma unroll 1
      for (; ks < nk; ++ks) body2(ks, stage_ptr(ks & 1), stage_ptr((ks + 1) & 1));
    }
    wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

    // Epilogue: acc[i][j][r] = C[m][n], m = wm*32FA + 32 i + (lane % 32),
    //                                   n = wn*32FB + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4.
    // A store straight from that layout writes 16 or 32 bytes into each of 32 rows, and the L2
    // write-request rate then bounds the kernel's tail. The tile goes through LDS instead (free
    // now: every wave has passed its last stage read): each wave writes its sub-tile row-major,
    // then each store instruction writes whole rows (512 or 1024 contiguous bytes). bf16 results
    // use the hardware round-to-nearest-even pair conversion, which equals rounding the fp32 bit
    // pattern for every non-NaN input. Rows are padded by 16 bytes so that the 32 rows a write
    // instruction touches spread over all banks.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if constexpr (QOUT) {
      // Quantized output [P1 paragraph 1: rotate, scale, round and pack the output tile before
      // it is stored]: the fp32 tile (times 2^alpha) goes to LDS in two halves of 128 rows;
      // then every quad of lanes takes one 32-column block of a row, as the row quantizer does.
      constexpr int kPitch = kBN * 4 + 16;
      constexpr int kPassRows = kBM / 2;
      static_assert(kPassRows * kPitch <= Cfg::kLds, "fp32 half tile fits in LDS");
      const int q = t & 3;
      const int mode = (qo.hadamard ? 1 : 0) | (qo.sr ? 2 : 0) | (qo.ceil ? 4 : 0);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if ((wm * 32 * FA) / kPassRows == p) {
#pragma unroll
          for (int i = 0; i < FA; ++i)
#pragma unroll
            for (int j = 0; j < FB; ++j)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) {
                const int r = wm * 32 * FA + 32 * i + frow - p * kPassRows;
                const int c = wn * 32 * FB + 32 * j + 8 * rq + 4 * fhalf;
                *reinterpret_cast<f32x4*>(smem + r * kPitch + 4 * c) =
                    f32x4{acc[i][j][4 * rq + 0] * alpha_f, acc[i][j][4 * rq + 1] * alpha_f,
                          acc[i][j][4 * rq + 2] * alpha_f, acc[i][j][4 * rq + 3] * alpha_f};
              }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        // round rnd: block b = 64 rnd + t / 4 of the half (row b / 8, 32-column block b % 8)
        constexpr int kRounds = kPassRows * (kBN / 32) / (64 * WAVES / 4);
#pragma unroll 1
        for (int rnd = 0; rnd < kRounds; ++rnd) {
          const int b = rnd * (16 * WAVES) + (t >> 2);
          const int r = b >> 3, bc = b & 7;
          const int64_t m = m0 + p * kPassRows + r, nb = n0 + 32 * bc;
          if (m >= M || nb >= N) continue;  // whole quads leave together
          const f32x4 lo = *reinterpret_cast<const f32x4*>(smem + r * kPitch + 4 * (32 * bc + 8 * q));
          const f32x4 hi = *reinterpret_cast<const f32x4*>(smem + r * kPitch + 4 * (32 * bc + 8 * q) + 16);
          float w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int64_t e0 = m * N + nb + 8 * q;  // row-major index of value 0 in C
          const uint64_t g = (uint64_t)e0 >> 3;
          uint32_t sb = 0, word = 0;
          switch (mode) {
            case 0: word = mxd::quant_chunk8<false, false, false>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 1: word = mxd::quant_chunk8<true, false, false>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 2: word = mxd::quant_chunk8<false, true, false>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 3: word = mxd::quant_chunk8<true, true, false>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 4: word = mxd::quant_chunk8<false, false, true>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 5: word = mxd::quant_chunk8<true, false, true>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            case 6: word = mxd::quant_chunk8<false, true, true>(w, q, qo.sign_mask, qo.seed, g, sb); break;
            default: word = mxd::quant_chunk8<true, true, true>(w, q, qo.sign_mask, qo.seed, g, sb); break;
          }
          *reinterpret_cast<uint32_t*>(qo.codes + e0 / 2) = word;
          if (q == 0) qo.scales[m * (N / 32) + nb / 32] = (uint8_t)sb;
        }
        if (p == 0) {
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __builtin_amdgcn_s_barrier();
        }
      }
    } else {
      const bool full = m0 + kBM <= M && n0 + kBN <= N;
      if (out_bf16) {
        constexpr int kPitch = kBN * 2 + 16;
        static_assert(kBM * kPitch <= Cfg::kLds, "bf16 tile fits in LDS");
#pragma unroll
        for (int i = 0; i < FA; ++i)
#pragma unroll
          for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int r = wm * 32 * FA + 32 * i + frow;
              const int c = wn * 32 * FB + 32 * j + 8 * rq + 4 * fhalf;
              f32x2 lo = {acc[i][j][4 * rq + 0] * alpha_f, acc[i][j][4 * rq + 1] * alpha_f};
              f32x2 hi = {acc[i][j][4 * rq + 2] * alpha_f, acc[i][j][4 * rq + 3] * alpha_f};
              uint2 w;
              w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
              w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
              *reinterpret_cast<uint2*>(smem + r * kPitch + 2 * c) = w;
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        // instruction q of wave w: rows 2 (q WAVES + w) + lane / 32, 16-byte chunk lane % 32
        constexpr int kReads = kBM / 2 / WAVES;
#pragma unroll 8
        for (int q = 0; q < kReads; ++q) {
          const int r = 2 * (q * WAVES + wave) + fhalf;
          const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * kPitch + 16 * frow);
          const int64_t m = m0 + r, n = n0 + 8 * frow;
          // non-temporal: the output streams past L2 instead of displacing the operand panels the
          // XCD's other tiles are still reading there
          if (full || (m < M && n < N))
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + m * ldc + n));
        }
      } else {
        // fp32: two passes of 128 rows (the waves with wm == p fill pass p)
        constexpr int kPitch = kBN * 4 + 16;
        constexpr int kPassRows = kBM / 2;
        static_assert(kPassRows * kPitch <= Cfg::kLds, "fp32 half tile fits in LDS");
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if ((wm * 32 * FA) / kPassRows == p) {
#pragma unroll
            for (int i = 0; i < FA; ++i)
#pragma unroll
              for (int j = 0; j < FB; ++j)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                  const int r = wm * 32 * FA + 32 * i + frow - p * kPassRows;
                  const int c = wn * 32 * FB + 32 * j + 8 * rq + 4 * fhalf;
                  *reinterpret_cast<f32x4*>(smem + r * kPitch + 4 * c) =
                      f32x4{acc[i][j][4 * rq + 0] * alpha_f, acc[i][j][4 * rq + 1] * alpha_f,
                            acc[i][j][4 * rq + 2] * alpha_f, acc[i][j][4 * rq + 3] * alpha_f};
                }
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __builtin_amdgcn_s_barrier();
          // instruction q of wave w: row q WAVES + w, 16-byte chunk lane
          constexpr int kReads = kPassRows / WAVES;
#pragma unroll 8
          for (int q = 0; q < kReads; ++q) {
            const int r = q * WAVES + wave;
            const f32x4 v = *reinterpret_cast<const f32x4*>(smem + r * kPitch + 16 * lane);
            const int64_t m = m0 + p * kPassRows + r, n = n0 + 4 * lane;
            if (full || (m < M && n < N))
              __builtin_nontemporal_store(
                  v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + m * ldc + n));
          }
          if (p == 0) {
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
          }
        }
      }
    }
    // every wave is done with the LDS (the epilogue staging) before the next tile loads into it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
}


// ---------------------------------------------------------------------------------------------
// Ping-pong kernel (FP4 operands, K a multiple of 1024). Eight waves, two per SIMD: waves w and
// w + 4 share a SIMD (the hardware places a workgroup's waves 0-3 on four different SIMDs and
// waves 4-7 on the same four), and wave w belongs to group g = w / 4. Wave (g, s = w % 4) owns
// rows 128g .. 128g+127 and columns 64s .. 64s+63 of the 256x256 tile (4 x 2 MFMA tiles, 128
// fp32 accumulators), so every 64-row block of B is read by one wave of each group and every
// 128-row half of A by one group only. The two waves of a SIMD take turns: while one
// issues the 32 MFMAs of a 256-k step from registers (compute phase), the other reads its
// fragments and scales of its next step from LDS and, in group 0, issues the direct-to-LDS loads
// of the step after (memory phase). Every phase ends with a workgroup barrier, so the matrix
// core of a SIMD always has one wave feeding it while the other waits on LDS or memory; a single
// wave per SIMD would idle the matrix core whenever it waits.
//
// Step k lives in LDS stage k % 2 (A then B, 128-byte rows, 16-byte chunk c of row r at position
// c ^ ((r >> 1) & 7), so 16 consecutive rows read at one chunk hit all 64 banks). Its scales come
// from scale group k / 4 (buffer (k / 4) % 2: 32 bytes per row = 4 steps of 8 E8M0 bytes; the
// two 16-byte halves of a row swap places when bit 3 of the row is set, which keeps 16
// consecutive rows on distinct banks).
//
// Which k-blocks one MFMA covers is free as long as both operands agree: sub-step s (0..3) of a
// step uses k-block 4h + s on lane half h. A lane's fragment of sub-step s is then chunk 4h + s
// of its row, and its four scale bytes of a step are one aligned word (bytes 4h .. 4h+3 of the
// row's 8), whose byte s the MFMA selects with op_sel = s.
//
// Timeline per tile (n steps; M = memory phase, C = compute phase, | = barrier):
//   group 0:   M0 | C0 | M1 | C1 | ... | M(n-1) | C(n-1) | (idle)   |
//   group 1: (idle) | M0 | C0 | M1 | ... | C(n-2) | M(n-1) | C(n-1) |
// A step's direct loads (64 KiB of codes) take the load path about half a phase; issued by one
// group in one phase they would outlast the partner's compute phase. So each group loads one
// operand: group 0's M(k) issues A of step k+1 into stage (k+1) % 2 (whose last reader was
// group 1's M(k-1)) and one quarter of a scale group, waited for at the end of its C(k); wave s
// of group 1, once its own M(k) reads of stage k % 2 are complete, issues the 64 B rows it and
// wave s of group 0 read (group 0's M(k) is a phase older), for step k+2 into that stage, and
// waits for them at the end of its M(k+1). Steps 0 and 1 and scale group 0 are loaded up front:
// for a workgroup's first tile before it, for each later tile at the end of the tile before.
// There step 0 and scale group 0 go out as soon as the last compute phase is done, the epilogue
// stages the output through stage 1 only, and step 1 and the first quarter of scale group 1 go
// out after it, ahead of the output stores. The next tile's first waits count those stores as
// still in flight (a wave's vector memory operations complete in issue order), so the stores
// drain under its first compute phase instead of ahead of it.
// ---------------------------------------------------------------------------------------------
namespace pp {
constexpr int kThreads = 512;
constexpr int kRow = 128;                    // code bytes per row per step (256 FP4 values)
constexpr int kTile = 256 * kRow;            // one operand's codes of a step: 32 KiB
constexpr int kStage = 2 * kTile;            // A then B
constexpr int kGrpRow = 32;                  // scale bytes per row per group (4 steps)
constexpr int kGrpOp = 256 * kGrpRow;        // 8 KiB per operand
constexpr int kGrp = 2 * kGrpOp;             // A then B
constexpr int kLds = 2 * kStage + 2 * kGrp;  // 160 KiB
// epilogue staging in stage 1: 128-row passes of bf16 rows (512 B) or 64-row passes of fp32
// rows (1 KiB); the 16-byte chunks of row r sit at chunk ^ (r % 32), so that a column of rows
// written by one instruction and a row read by one instruction both spread over all banks
static_assert(kStage == 128 * 512 && kStage == 64 * 1024, "staging passes");
__device__ __forceinline__ uint32_t stage_chunk(int row, int chunk) {
  return (uint32_t)(chunk ^ (row & 31)) * 16u;
}

// s_waitcnt vmcnt with a count known only at run time (uniform), from the values used below
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 25: wait_vmcnt<25>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 8: wait_vmcnt<8>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// tile index -> first row of A and of B, in the order of the streaming kernel: each XCD gets a
// contiguous range of tiles, walked in groups of 4 tile rows
__device__ __forceinline__ void tile_origin(int tile, int nbm, int nbn, int64_t& m0, int64_t& n0) {
  const int nblocks = nbm * nbn;
  int bid = tile;
  const int per_xcd = nblocks / 8;
  if (bid < per_xcd * 8) bid = (bid % 8) * per_xcd + bid / 8;
  constexpr int kGroup = 4;
  const int group = bid / (kGroup * nbn);
  const int first_m = group * kGroup;
  const int gsize = min(nbm - first_m, kGroup);
  const int in_group = bid - group * kGroup * nbn;
  m0 = (int64_t)(first_m + in_group % gsize) * 256;
  n0 = (int64_t)(in_group / gsize) * 256;
}

// buffer descriptors of one tile's operands: 256-row code panels and their scale rows; loads
// past the operand's last row read zero
struct TileRes {
  i32x4 ra, rb, rsa, rsb;
};
__device__ __forceinline__ TileRes tile_res(const uint8_t* A, const uint8_t* As, int lga,
                                            const uint8_t* B, const uint8_t* Bs, int lgb,
                                            int64_t M, int64_t N, int64_t K, int64_t m0,
                                            int64_t n0, int64_t kbytes) {
  const int64_t nkb = K / 32;
  const int64_t rows_a = min((int64_t)256, M - m0), rows_b = min((int64_t)256, N - n0);
  TileRes r;
  r.ra = rsrc_words(A + m0 * kbytes, rows_a * kbytes);
  r.rb = rsrc_words(B + n0 * kbytes, rows_b * kbytes);
  // rows_a and rows_b are multiples of the scale granularity, so the scale rows of rows past
  // the operand start at or beyond the end of these ranges
  r.rsa = rsrc_words(As + (m0 >> lga) * nkb, (rows_a >> lga) * nkb);
  r.rsb = rsrc_words(Bs + (n0 >> lgb) * nkb, (rows_b >> lgb) * nkb);
  return r;
}
}  // namespace pp

// AF, BF: operand formats as the matrix instruction numbers them (4 = E2M1; 0 = E4M3 and
// 1 = E5M2 for MXFP8). A step is 128 code bytes of each row either way: 256 FP4 values in four
// 64-k sub-steps, or 128 FP8 values in two. A scale group holds a row's 32 scale bytes of 4
// FP4 steps (8 per step) or of 8 FP8 steps (4 per step). QOUT: the output is quantized in the
// epilogue (1x32 blocks along N, qo) instead of stored.
template <int AF, int BF, bool QOUT = false>
__global__ __launch_bounds__(pp::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_mx_pp_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, int lga,
                       const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int lgb,
                       int64_t M, int64_t N, int64_t K, float alpha_f, int out_bf16,
                       void* __restrict__ C, int64_t ldc, int nbm, int nbn, GemmQuantOut qo) {
  using namespace pp;
  constexpr bool F8 = AF != 4;
  static_assert(F8 == (BF != 4), "both operands FP4 or both FP8");
  static_assert(!(F8 && QOUT), "the quantizing epilogue takes FP4 operands");
  constexpr int kSub = F8 ? 2 : 4;   // 64-k sub-steps per step
  constexpr int kGS = F8 ? 8 : 4;    // steps per scale group
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
  const int nblocks = nbm * nbn;
  const int64_t kbytes = F8 ? K : K / 2, nkb = K / 32;
  const int n = (int)(kbytes / kRow);  // steps per tile, a multiple of 4
  __builtin_assume(n >= 4);

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int s = w & 3, g = w >> 2;           // index within the group, and the group
  const int wm = g, wn = s;
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  // output stores the previous tile issued after the last loads of this tile (0 for the first
  // tile, and after a partial tile, whose stores are not all issued), and the loads and stores
  // that may still be in flight when this tile starts (0 for the first tile)
  int nst_prev = 0, in_flight = 0;

  // Direct-to-LDS loads of wave s of a group (lane-dependent parts; the rest is scalar):
  //  * A code load q (0..7, group 0) of a step fills 1 KiB block b = s + 4q of the A stage tile:
  //    rows 8b + lane / 8, position lane % 8, i.e. chunk (lane % 8) ^ ((row >> 1) & 7), whose
  //    phase depends on the lane only: byte row * kbytes + 16 chunk of the operand panel, with
  //    32 q * kbytes of it a per-load constant;
  //  * B code load q (0..7, group 1) fills block b = 8s + q (rows 64s + 8q + lane / 8), whose
  //    chunk phase (4q + lane / 16) % 8 alternates with the parity of q;
  //  * scale quarter p (0..3, group 0 only) is load u = 4p + s: operand p / 2, rows
  //    128 (p % 2) + 32 s + lane / 2, position lane % 2, i.e. half (lane % 2) ^ bit 3 of the
  //    row = bit 4 of the lane.
  auto dma_lane_offsets = [&](int lane, int& voff0, int& goff0) {
    const int row = 8 * s + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    voff0 = row * (int)kbytes + 16 * chunk;
    const int half = (lane & 1) ^ ((lane >> 4) & 1);
    goff0 = 16 * half;  // + the row's scale offset, added per operand below
  };

  for (int tile = blockIdx.x; tile < nblocks; tile += gridDim.x) {
    // the lane index from the execution mask (not threadIdx, which would have to be kept in a
    // register through the tile loop); per tile, so that the lane setup stays out of the
    // loop-carried state
    uint32_t zero = 0;
    asm volatile("" : "+s"(zero));
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, zero));
    const int frow = lane & 31, h = lane >> 5;
    int64_t m0, n0;
    tile_origin(tile, nbm, nbn, m0, n0);
    const TileRes R = tile_res(A, As, lga, B, Bs, lgb, M, N, K, m0, n0, kbytes);

    int voff0, goff_half;
    dma_lane_offsets(lane, voff0, goff_half);
    // B loads of group 1: rows 64s + 8q + lane / 8; q even / odd have chunk phases differing in
    // bit 2
    const int bchunk = (lane & 7) ^ ((lane >> 4) & 7);
    const int voffb0 = (64 * s + (lane >> 3)) * (int)kbytes + 16 * bchunk;
    const int voffb1 = (64 * s + (lane >> 3)) * (int)kbytes + 16 * (bchunk ^ 4);
    // scale row offset of quarter p's row for lane: (row >> lg) * nkb, row = 128 (p % 2) + 32 w
    // + lane / 2; the scalar part goes in soffset, the lane part here (zero for g = 32 and 64,
    // where the lane's row stays inside one scale row)
    const int goff_a = (lga == 0 ? (lane >> 1) * (int)nkb : 0) + goff_half;
    const int goff_b = (lgb == 0 ? (lane >> 1) * (int)nkb : 0) + goff_half;

    // Step j's code loads by wave s of group op (0: A, all 256 rows over the group; 1: B rows
    // 64s .. 64s+63): 8 blocks of 1 KiB into stage j % 2. The row offsets stay in the lane
    // offset (the buffer range check, which zeroes rows past the operand, applies to it); only
    // the k offset is scalar.
    // (The lane offsets pass through an empty asm at each use, so that the eight per-load
    // offsets are recomputed there instead of being held in registers across the loop.)
    // (The wave's LDS base also passes through an empty asm, so that the eight destinations are
    // formed at each use rather than held in scalar registers.)
    auto issue_codes = [&](const TileRes& r, int j, int op) {
      if (op == 0) {
        uint32_t st = lds0 + 1024 * s;
        int v0 = voff0;
        asm volatile("" : "+v"(v0), "+s"(st));
        st += (j & 1) * kStage;
#pragma unroll
        for (int q = 0; q < 8; ++q) dma_b128(r.ra, st + 4096 * q, v0 + q * 32 * (int)kbytes, j * kRow);
      } else {
        uint32_t st = lds0 + kTile + 8192 * s;
        int v0 = voffb0, v1 = voffb1;
        asm volatile("" : "+v"(v0), "+v"(v1), "+s"(st));
        st += (j & 1) * kStage;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          dma_b128(r.rb, st + 1024 * q, ((q & 1) ? v1 : v0) + 8 * q * (int)kbytes, j * kRow);
      }
    };
    auto issue_quarter = [&](const TileRes& r, int G, int p) {
      const int op = p >> 1;
      const int row0 = 128 * (p & 1) + 32 * s;  // first row of this wave's piece
      const int lg = op ? lgb : lga;
      const uint32_t dst = lds0 + 2 * kStage + (G & 1) * kGrp + op * kGrpOp + 1024 * (4 * (p & 1) + s);
      int voff = op ? goff_b : goff_a;
      asm volatile("" : "+v"(voff));
      voff += (row0 >> lg) * (int)nkb;
      dma_b128(op ? r.rsb : r.rsa, dst, voff, G * kGrpRow);
    };

    // Steps 0 and 1 of a tile, scale group 0 and the first quarter of group 1: group 0 loads
    // A and the scales, group 1 loads B. The first tile of a workgroup issues them here, later
    // tiles at the end of the previous tile (step 0 and group 0 before its epilogue, the rest
    // after it).
    auto prologue0 = [&](const TileRes& r) {
      issue_codes(r, 0, g);
      if (g == 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) issue_quarter(r, 0, p);
      }
    };
    auto prologue1 = [&](const TileRes& r) {
      issue_codes(r, 1, g);
      if (g == 0 && kGS < n) issue_quarter(r, 1, 0);
    };
    const bool first = tile == (int)blockIdx.x;
    if (first) {
      prologue0(R);
      prologue1(R);
    }

    // per-lane LDS offsets of the fragment and scale reads
    const int phi = (frow >> 1) & 7;
    const int cb = (4 * h) ^ phi;  // chunk 4h + c of the row sits at cb ^ c
    const uint32_t a_row = (uint32_t)(128 * wm + frow) * kRow;
    const uint32_t b_row = kTile + (uint32_t)(64 * wn + frow) * kRow;
    const int sw = (frow >> 3) & 1;
    // FP4: the lane half's 4 scale bytes of a step are a word of their own; FP8: both halves
    // read the step's word and the upper half shifts its two bytes down
    const uint32_t sa_row = 2 * kStage + (uint32_t)(128 * wm + frow) * kGrpRow + (F8 ? 0 : 4 * h);
    const uint32_t sb_row =
        2 * kStage + kGrpOp + (uint32_t)(64 * wn + frow) * kGrpRow + (F8 ? 0 : 4 * h);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    using Frag = std::conditional_t<F8, u32x8, u32x4>;  // 32 values of a row per lane
    Frag fa[kSub][4], fb[kSub][2];                      // [sub-step][fragment]
    uint32_t sa[4], sb[2];

    // memory phase of step k: fragments and scale words into registers (plus, in group 0, the
    // loads of step k + 1); ends with this wave's reads complete
    auto mem_phase = [&](int k, auto step0, auto grp) {
      constexpr int G = decltype(grp)::value;
      const uint8_t* st = smem + (k & 1) * kStage;
      auto frag = [&](uint32_t row, int ss) {
        if constexpr (F8) {
          // the matrix instruction's 8-bit layout: lane half h holds values 16h .. 16h+15 of
          // each of the sub-step's two k-blocks, i.e. chunks 4ss + h and 4ss + 2 + h
          const uint32_t c = 16u * (uint32_t)((4 * ss + h) ^ phi);
          const u32x4 lo = *reinterpret_cast<const u32x4*>(st + row + c);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(st + row + (c ^ 32u));
          return Frag{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        } else {  // chunk 4h + ss
          return *reinterpret_cast<const Frag*>(st + row + 16u * (uint32_t)(cb ^ ss));
        }
      };
#pragma unroll
      for (int ss = 0; ss < kSub; ++ss) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[ss][i] = frag(a_row + 4096 * i, ss);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[ss][j] = frag(b_row + 4096 * j, ss);
      }
      // step k's scale bytes: FP4 8 per row (word 4h + ...), FP8 4 per row
      const int t = k & (kGS - 1);
      const uint32_t sofs =
          F8 ? ((k >> 3) & 1) * kGrp + 16 * ((t >> 2) ^ sw) + 4 * (t & 3)
             : ((k >> 2) & 1) * kGrp + 16 * ((t >> 1) ^ sw) + 8 * (t & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sa[i] = *reinterpret_cast<const uint32_t*>(smem + sa_row + 1024 * i + sofs);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        sb[j] = *reinterpret_cast<const uint32_t*>(smem + sb_row + 1024 * j + sofs);
      if (G == 0 && k >= 1 && k + 1 < n) {
        issue_codes(R, k + 1, 0);
        // quarter p of scale group G' goes out at step kGS (G' - 1) + p (groups of this tile
        // only)
        const int v = k + kGS;
        if ((v & (kGS - 1)) < 4 && (v & ~(kGS - 1)) < n) issue_quarter(R, v / kGS, v & (kGS - 1));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage k are done
      if constexpr (F8) {
        // the scale of a sub-step's k-block b comes from lane half b: byte 2ss + h of the
        // step's word, i.e. byte 2ss after a shift by one byte on the upper half
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] >>= 8 * h;
#pragma unroll
        for (int j = 0; j < 2; ++j) sb[j] >>= 8 * h;
      }
      if constexpr (G == 1) {
        // B of step k + 1 has landed (at k = 0 the previous tile's output stores, issued after
        // it, may still be in flight)
        if constexpr (decltype(step0)::value) wait_vmcnt_upto(nst_prev);
        else wait_vmcnt<0>();
        if (k + 2 < n) issue_codes(R, k + 2, 1);
      }
    };
    auto compute_phase = [&]() {
      __builtin_amdgcn_s_setprio(1);
      static_for<kSub>([&](auto ssc) {
        constexpr int SS = decltype(ssc)::value;
        constexpr int OP = F8 ? 2 * SS : SS;  // scale byte of the sub-step
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                as_operand(fb[SS][j]), as_operand(fa[SS][i]), acc[i][j], BF, AF, OP, sb[j], OP, sa[i]);
      });
      __builtin_amdgcn_s_setprio(0);
    };

    // this tile's step 0 and scale group 0 have landed: everything of a first tile; for a
    // later tile all but step 1 (8 loads), the quarter of group 1 (group 0, one load) and the
    // stores after them
    wait_vmcnt_upto(in_flight);
    barrier();
    // step 0 is peeled off the loops: its waits let the previous tile's stores stay in flight
    using Step0 = std::integral_constant<bool, true>;
    using StepK = std::integral_constant<bool, false>;
    using Grp0 = std::integral_constant<int, 0>;
    using Grp1 = std::integral_constant<int, 1>;
    if (g == 0) {
      mem_phase(0, Step0{}, Grp0{});
      barrier();
      compute_phase();
      wait_vmcnt_upto(nst_prev);  // A of step 1 and the scale quarter, not the stores after them
      barrier();
#pragma unroll 1
      for (int k = 1; k < n; ++k) {
        mem_phase(k, StepK{}, Grp0{});
        barrier();
        compute_phase();
        wait_vmcnt<0>();  // A of step k + 1 and the scale quarter have landed
        barrier();
      }
      barrier();  // group 1 computes step n - 1
    } else {
      barrier();  // group 0 reads step 0
      mem_phase(0, Step0{}, Grp1{});
      barrier();
      compute_phase();
      barrier();
#pragma unroll 1
      for (int k = 1; k < n; ++k) {
        mem_phase(k, StepK{}, Grp1{});
        barrier();
        compute_phase();
        barrier();
      }
    }
    // both groups are past their last reads of the stages and scale groups: the next tile's
    // step 0 and scale group 0 go out now
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < nblocks;
    if (has_next) {
      int64_t nm0, nn0;
      tile_origin(next, nbm, nbn, nm0, nn0);
      prologue0(tile_res(A, As, lga, B, Bs, lgb, M, N, K, nm0, nn0, kbytes));
    }

    // Epilogue: acc[i][j][r] = C[m][n], m = 128 wm + 32 i + (lane % 32),
    //                                   n = 64 wn + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4.
    // The tile goes through stage 1 so that stores write whole rows; the row values are read
    // back into registers first, so that the next tile's step 1 can go out before the stores.
    uint8_t* const stg = smem + kStage;
    auto step1_next = [&]() {
      if (has_next) {
        int64_t nm0, nn0;
        tile_origin(next, nbm, nbn, nm0, nn0);
        prologue1(tile_res(A, As, lga, B, Bs, lgb, M, N, K, nm0, nn0, kbytes));
      }
    };
    const bool full = m0 + 256 <= M && n0 + 256 <= N;
    int bf16_out = out_bf16, wme = wm;
    asm volatile("" : "+s"(bf16_out), "+s"(wme));  // tested here, not held as masks
    if constexpr (QOUT) {
      // Quantized output [P1 paragraph 1: rotate, scale, round and pack the output tile before
      // it is stored]: four passes of 64 rows of the fp32 tile (times 2^alpha) through stage 1,
      // as the fp32 output does; then thread t takes the 32-column block t % 8 of pass row t / 8
      // whole, as the row quantizer does (random-field index of C[m][n]: m * N + n)
      const int t = 64 * w + lane;
      const int rr = t >> 3, bc = t & 7;
      // accumulator rows 32 i, i = 2 (p % 2) + 0, 1, of the waves with wm == p / 2 (the
      // accumulator index must be a constant, so the pass loop dispatches on p % 2)
      auto write_pass = [&](auto half) {
        constexpr int P1 = decltype(half)::value;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              constexpr int kI0 = 2 * P1;
              const int r = 32 * ii + frow;
              const int c = 64 * wn + 32 * j + 8 * rq + 4 * h;
              *reinterpret_cast<f32x4*>(stg + r * 1024 + stage_chunk(r, c >> 2)) =
                  f32x4{acc[kI0 + ii][j][4 * rq + 0] * alpha_f, acc[kI0 + ii][j][4 * rq + 1] * alpha_f,
                        acc[kI0 + ii][j][4 * rq + 2] * alpha_f, acc[kI0 + ii][j][4 * rq + 3] * alpha_f};
            }
      };
#pragma unroll 1
      for (int p = 0; p < 4; ++p) {
        if (wme == (p >> 1)) {
          if (p & 1) write_pass(std::integral_constant<int, 1>{});
          else write_pass(std::integral_constant<int, 0>{});
        }
        barrier();
        float x[32];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rr * 1024 + stage_chunk(rr, 8 * bc + c));
          x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier();  // the next pass may write stage 1
        const int64_t m = m0 + 64 * p + rr, nb = n0 + 32 * bc;
        if (m < M && nb < N) {
          if (qo.hadamard) {
#pragma unroll
            for (int j = 0; j < 32; ++j)
              x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((qo.sign_mask >> j) & 1u) << 31));
            mxd::hadamard32_inlane(x);
          }
          const int64_t e0 = m * N + nb;
          uint32_t sb;
          u32x4 code;
          if (qo.sr) code = qo.ceil ? mxd::quant_block32<true, true>(x, qo.seed, (uint64_t)e0 >> 3, sb)
                                    : mxd::quant_block32<true, false>(x, qo.seed, (uint64_t)e0 >> 3, sb);
          else code = qo.ceil ? mxd::quant_block32<false, true>(x, qo.seed, (uint64_t)e0 >> 3, sb)
                              : mxd::quant_block32<false, false>(x, qo.seed, (uint64_t)e0 >> 3, sb);
          __builtin_nontemporal_store(code, reinterpret_cast<u32x4*>(qo.codes + e0 / 2));
          qo.scales[e0 / 32] = (uint8_t)sb;
        }
      }
      step1_next();
      nst_prev = 0;
    } else if (bf16_out) {
      // two passes of 128 rows: the waves with wm == p write pass p
      u32x4 v[2][8];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (wme == p) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) {
                const int r = 32 * i + frow;
                const int c = 64 * wn + 32 * j + 8 * rq + 4 * h;  // first of 4 bf16 columns
                f32x2 lo = {acc[i][j][4 * rq + 0] * alpha_f, acc[i][j][4 * rq + 1] * alpha_f};
                f32x2 hi = {acc[i][j][4 * rq + 2] * alpha_f, acc[i][j][4 * rq + 3] * alpha_f};
                uint2 u;
                u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                *reinterpret_cast<uint2*>(stg + r * 512 + stage_chunk(r, c >> 3) + 8 * h) = u;
              }
        }
        barrier();
        // read q of wave w: row 16 q + 2 w + lane / 32, 16-byte chunk lane % 32
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 16 * q + 2 * w + h;
          v[p][q] = *reinterpret_cast<const u32x4*>(stg + r * 512 + stage_chunk(r, frow));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier();
      }
      step1_next();
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t m = m0 + 128 * p + 16 * q + 2 * w + h, nn = n0 + 8 * frow;
          if (full || (m < M && nn < N))
            __builtin_nontemporal_store(
                v[p][q], reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(C) + m * ldc + nn));
        }
      nst_prev = full ? 16 : 0;
    } else {
      // fp32: four passes of 64 rows (the waves with wm == p / 2 fill pass p with their
      // accumulator rows 32 i, i = 2 (p % 2), 2 (p % 2) + 1); each pass stores as it goes
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (wme == (p >> 1)) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) {
                const int i = 2 * (p & 1) + ii;
                const int r = 32 * ii + frow;
                const int c = 64 * wn + 32 * j + 8 * rq + 4 * h;  // first of 4 fp32 columns
                *reinterpret_cast<f32x4*>(stg + r * 1024 + stage_chunk(r, c >> 2)) =
                    f32x4{acc[i][j][4 * rq + 0] * alpha_f, acc[i][j][4 * rq + 1] * alpha_f,
                          acc[i][j][4 * rq + 2] * alpha_f, acc[i][j][4 * rq + 3] * alpha_f};
              }
        }
        barrier();
        // read q of wave w: row 8 q + w, 16-byte chunk lane
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 8 * q + w;
          v[q] = *reinterpret_cast<const f32x4*>(stg + r * 1024 + stage_chunk(r, lane));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t m = m0 + 64 * p + 8 * q + w, nn = n0 + 4 * lane;
          if (full || (m < M && nn < N))
            __builtin_nontemporal_store(
                v[q], reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + m * ldc + nn));
        }
      }
      step1_next();
      nst_prev = 0;
    }
    // the next tile starts once all but its step 1 (8 loads), the quarter of scale group 1
    // (group 0's waves, one load) and these stores have landed
    int gq = g, nq = n;
    asm volatile("" : "+s"(gq), "+s"(nq));
    in_flight = 8 + (gq == 0 && kGS < nq ? 1 : 0) + nst_prev;
  }

  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends
}

}  // namespace

// Grid of the streaming kernel: one workgroup per CU (a workgroup holds a whole CU's LDS), each
// walking tiles, when there are more tiles than CUs; the CU count is rounded down to a multiple
// of 8 (the XCDs). Without the attribute, one workgroup per tile.
static int stream_grid(int64_t nblocks) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    return (int)nblocks;
  cus -= cus % 8;
  return (int)min(nblocks, (int64_t)cus);
}

hipError_t mx_launch_gemm(const GemmArgs& g) {
  const int64_t nbm = (g.M + kBM - 1) / kBM, nbn = (g.N + kBN - 1) / kBN;
  if (nbm * nbn > 0x7FFFFFFF) return hipErrorInvalidValue;
  // buffer offsets are 32-bit: one 256-row operand tile must stay below 2 GiB
  if ((int64_t)kBM * (g.K / 2) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const float alpha_f = __builtin_bit_cast(float, (uint32_t)(g.alpha + 127) << 23);
  const int lga = g.ga == 64 ? 6 : g.ga == 32 ? 5 : 0, lgb = g.gb == 64 ? 6 : g.gb == 32 ? 5 : 0;
  const dim3 grid((unsigned)(nbm * nbn));
  const dim3 resident((unsigned)stream_grid(nbm * nbn));
  // loads of a step issued during sub-steps 3, 0, 1 (the rest during sub-step 2): as early as
  // the at-most-one-load-per-MFMA-pair rule allows
  constexpr int kS3 = kStreamWaves == 4 ? 8 : 4, kS0 = kStreamWaves == 4 ? 8 : 4;
  constexpr int kS1 = kStreamWaves == 4 ? 1 : 2;
  if (g.K % 1024 == 0 && g.K > 0)
    hipLaunchKernelGGL((gemm_mx_pp_kernel<4, 4>), resident, dim3(pp::kThreads), 0, (hipStream_t)g.stream,
                       g.a, g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0,
                       g.c, g.ldc, (int)nbm, (int)nbn, GemmQuantOut{});
  else if (g.K % 512 == 0 && g.K > 0)
    hipLaunchKernelGGL((gemm_mx_stream_kernel<kStreamWaves, 4, 2, kS3, kS0, kS1>), resident,
                       dim3(64 * kStreamWaves), 0, (hipStream_t)g.stream, g.a,
                       g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0, g.c,
                       g.ldc, (int)nbm, (int)nbn, GemmQuantOut{});
  else if (g.K % kBK == 0 && g.K > 0)
    hipLaunchKernelGGL((gemm_mx_stream_kernel<kStreamWaves, 2, 4>), resident, dim3(64 * kStreamWaves),
                       0, (hipStream_t)g.stream, g.a,
                       g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0, g.c,
                       g.ldc, (int)nbm, (int)nbn, GemmQuantOut{});
  else
    hipLaunchKernelGGL(gemm_mx_generic_kernel<false>, grid, dim3(kThreads), 0, (hipStream_t)g.stream, g.a,
                       g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f, g.out_bf16 ? 1 : 0, g.c,
                       g.ldc, (int)nbm, (int)nbn);
  return hipGetLastError();
}

hipError_t mx_launch_gemm_quant(const GemmArgs& g, const GemmQuantOut& q) {
  const int64_t nbm = (g.M + kBM - 1) / kBM, nbn = (g.N + kBN - 1) / kBN;
  if (nbm * nbn > 0x7FFFFFFF) return hipErrorInvalidValue;
  if ((int64_t)kBM * (g.K / 2) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  if (g.K <= 0 || g.K % kBK != 0) return hipErrorInvalidValue;
  const float alpha_f = __builtin_bit_cast(float, (uint32_t)(g.alpha + 127) << 23);
  const int lga = g.ga == 64 ? 6 : g.ga == 32 ? 5 : 0, lgb = g.gb == 64 ? 6 : g.gb == 32 ? 5 : 0;
  const dim3 resident((unsigned)stream_grid(nbm * nbn));
  constexpr int kS3 = kStreamWaves == 4 ? 8 : 4, kS0 = kStreamWaves == 4 ? 8 : 4;
  constexpr int kS1 = kStreamWaves == 4 ? 1 : 2;
  if (g.K % 1024 == 0 && (reinterpret_cast<uintptr_t>(q.codes) & 15) == 0)
    hipLaunchKernelGGL((gemm_mx_pp_kernel<4, 4, true>), resident, dim3(pp::kThreads), 0,
                       (hipStream_t)g.stream, g.a, g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K,
                       alpha_f, 0, nullptr, 0, (int)nbm, (int)nbn, q);
  else if (g.K % 512 == 0)
    hipLaunchKernelGGL((gemm_mx_stream_kernel<kStreamWaves, 4, 2, kS3, kS0, kS1, true>), resident,
                       dim3(64 * kStreamWaves), 0, (hipStream_t)g.stream, g.a, g.as, lga, g.b,
                       g.bs, lgb, g.M, g.N, g.K, alpha_f, 0, nullptr, 0, (int)nbm, (int)nbn, q);
  else
    hipLaunchKernelGGL((gemm_mx_stream_kernel<kStreamWaves, 2, 4, 0, 0, 0, true>), resident,
                       dim3(64 * kStreamWaves), 0, (hipStream_t)g.stream, g.a, g.as, lga, g.b,
                       g.bs, lgb, g.M, g.N, g.K, alpha_f, 0, nullptr, 0, (int)nbm, (int)nbn, q);
  return hipGetLastError();
}

// MXFP8 operands (K a multiple of 128): the streaming kernel with 128-k stages; all but two
// loads of a bundle go out during the last sub-step of the step before (one per MFMA)
template <int AF, int BF>
static hipError_t launch_gemm_fp8(const GemmArgs& g, const dim3 grid, float alpha_f, int lga,
                                  int lgb, int nbm, int nbn) {
  hipLaunchKernelGGL((gemm_mx_stream_kernel<4, 4, 2, 16, 2, 0, false, AF, BF>), grid, dim3(256), 0,
                     (hipStream_t)g.stream, g.a, g.as, lga, g.b, g.bs, lgb, g.M, g.N, g.K, alpha_f,
                     g.out_bf16 ? 1 : 0, g.c, g.ldc, nbm, nbn, GemmQuantOut{});
  return hipGetLastError();
}

// MXFP8 with K a multiple of 512: the two-waves-per-SIMD kernel
template <int AF, int BF>
static hipError_t launch_gemm_fp8_pp(const GemmArgs& g, const dim3 grid, float alpha_f, int nbm,
                                     int nbn) {
  hipLaunchKernelGGL((gemm_mx_pp_kernel<AF, BF>), grid, dim3(pp::kThreads), 0,
                     (hipStream_t)g.stream, g.a, g.as, 0, g.b, g.bs, 0, g.M, g.N, g.K, alpha_f,
                     g.out_bf16 ? 1 : 0, g.c, g.ldc, nbm, nbn, GemmQuantOut{});
  return hipGetLastError();
}

hipError_t mx_launch_gemm_fp8(const GemmArgs& g, int afmt, int bfmt) {
  const int64_t nbm = (g.M + kBM - 1) / kBM, nbn = (g.N + kBN - 1) / kBN;
  if (nbm * nbn > 0x7FFFFFFF) return hipErrorInvalidValue;
  if ((int64_t)kBM * g.K >= (int64_t)1 << 31) return hipErrorInvalidValue;
  if (g.K <= 0 || g.K % 128 != 0) return hipErrorInvalidValue;
  const float alpha_f = __builtin_bit_cast(float, (uint32_t)(g.alpha + 127) << 23);
  const dim3 grid((unsigned)stream_grid(nbm * nbn));
  const int b = (afmt ? 2 : 0) | (bfmt ? 1 : 0);
  if (g.K % 512 == 0) {
    switch (b) {
      case 0: return launch_gemm_fp8_pp<0, 0>(g, grid, alpha_f, (int)nbm, (int)nbn);
      case 1: return launch_gemm_fp8_pp<0, 1>(g, grid, alpha_f, (int)nbm, (int)nbn);
      case 2: return launch_gemm_fp8_pp<1, 0>(g, grid, alpha_f, (int)nbm, (int)nbn);
      default: return launch_gemm_fp8_pp<1, 1>(g, grid, alpha_f, (int)nbm, (int)nbn);
    }
  }
  switch (b) {
    case 0: return launch_gemm_fp8<0, 0>(g, grid, alpha_f, 0, 0, (int)nbm, (int)nbn);
    case 1: return launch_gemm_fp8<0, 1>(g, grid, alpha_f, 0, 0, (int)nbm, (int)nbn);
    case 2: return launch_gemm_fp8<1, 0>(g, grid, alpha_f, 0, 0, (int)nbm, (int)nbn);
    default: return launch_gemm_fp8<1, 1>(g, grid, alpha_f, 0, 0, (int)nbm, (int)nbn);
  }
}
