// quant.hip — MXFP4 quantize (1x32 along rows, 1x32 along columns, 32x32 tiles) and dequantize
// kernels for gfx950, plus their host-side launchers.
//
// Pages, cited by title and section:
//  [P1] "Block-Scaled MXFP4 With Stochastic Hadamard Rounding Matches BF16 Convergence on 70B
//       Pre-Training", paragraphs 1-2: one E8M0 exponent per 32 E2M1 values; the 32-element
//       Walsh-Hadamard rotation runs in registers before the codes are packed.
//  [P3] "Stable FP4 Training via Transposition-Invariant Block Quantization": "Why FP4 training
//       is the current frontier" (P = round(X/S), reconstruction P*S), "The aha: transposition
//       scrambles the blocks" (a transposed operand is re-blocked along the other axis), "The
//       fix, and its supporting cast" (32x32 tiles shared by X and X^T, scale rounded up so
//       nothing clips, stochastic rounding).
//  [P4] "Training LLMs with MXFP4", abstract: random Hadamard signs with stochastic rounding.
//
// Work mapping (all kernels are HBM streams):
//  * Along rows (MXFP4), a lane owns one whole 32-block: all five butterfly stages, the block
//    maximum and the scale stay in its registers. Loads are coalesced across the wave and
//    regrouped per block through the wave's LDS area.
//  * Along rows (MXFP8), a lane owns 8 consecutive elements (one 16-byte bf16 load) and a quad
//    of 4 lanes holds a block: butterfly spans 1, 2, 4 stay in the lane, spans 8 and 16 use DPP
//    quad permutes; the block maximum reduces the same way.
//  * Along columns and for square tiles, a lane owns an 8x8 patch (8 rows of 16 bytes). A quad
//    stacks 4 patches into 32 rows, so the same in-lane + quad structure runs down the columns;
//    16 lanes (4 quads side by side) make one 32x32 tile.
//  * Stochastic rounding draws one Philox4x32-10 call per 8 consecutive source elements.
#include "mx_device.h"
#include "mx_launch.h"

namespace {

using namespace mxd;

constexpr int kThreads = 256;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRowChunksPerThread = 4;

template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t off, float (&v)[8]) {
  if (BF16) {
    const u32x4 raw = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off));
    widen_bf16x8(raw, v);
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + off);
    const f32x4 a = __builtin_nontemporal_load(p);
    const f32x4 b = __builtin_nontemporal_load(p + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ---------------------------------------------------------------------------------------------
// 1x32 blocks along rows: one lane per block. Block b = row * (cols / 32) + column block is
// source elements 32 b .. 32 b + 31 of the logical tensor, so its 8-element groups have the
// stochastic-rounding chunk indices 4 b .. 4 b + 3. With the whole block in one lane, every
// butterfly stage, the maximum and the scale stay in registers (no lane exchanges, one scale
// computation per block); a wave reads 64 whole blocks and writes 1 KiB of codes and 64 scale
// bytes, each a contiguous piece.
// ---------------------------------------------------------------------------------------------
// Widen 8 bf16 values (one 16-byte load) and apply the random signs of block positions
// p0 .. p0+7: the sign of position j is bit j of sign_mask (the same for every lane). Adding
// 2^31 toggles bit 31 exactly as a XOR does, so the low value takes one shift-add and the high
// value one and-xor.
template <bool HAD>
__device__ __forceinline__ void widen_signed8(const u32x4 raw, uint32_t sign_mask, int p0,
                                              float* v) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t s0 = HAD ? ((sign_mask >> (p0 + 2 * i)) & 1u) << 31 : 0u;
    const uint32_t s1 = HAD ? ((sign_mask >> (p0 + 2 * i + 1)) & 1u) << 31 : 0u;
    v[2 * i] = __uint_as_float((w[i] << 16) + s0);
    v[2 * i + 1] = __uint_as_float((w[i] & 0xFFFF0000u) ^ s1);
  }
}

// The 16-byte pieces of a block are loaded with consecutive lanes on consecutive pieces (whole
// lines per instruction) and regrouped per block through the wave's own LDS area: piece c of
// block B sits at slot C B + (c ^ ((B >> log2(16 / C)) % C)), C pieces per block, so that both
// the writes (16 consecutive pieces) and the reads (piece j of 16 consecutive blocks) cover all
// banks. With a leading dimension other than cols the blocks are loaded directly per lane.
template <bool BF16>
__device__ __forceinline__ int row_slot(int blk, int c) {
  constexpr int C = BF16 ? 4 : 8, SH = BF16 ? 2 : 1;
  return C * blk + (c ^ ((blk >> SH) & (C - 1)));
}

template <bool BF16, bool HAD, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const void* __restrict__ x, int64_t nblk, int64_t bpr, int64_t ld, int contiguous,
    uint32_t sign_mask, uint64_t seed, u32x4* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int C = BF16 ? 4 : 8;  // 16-byte pieces per block
  __shared__ __attribute__((aligned(16))) u32x4 stage[kThreads * C];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wb = (int64_t)blockIdx.x * kThreads + wave * 64;  // the wave's first block
  const int64_t b = wb + lane;
  u32x4 raw[C];
  if (wb >= nblk) return;  // uniform per wave
  if (contiguous) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(x) + wb * 32 * (BF16 ? 2 : 4));
    u32x4* st = stage + wave * 64 * C;
    // all loads first (pieces of blocks past the end re-read the wave's first piece; their
    // slots are never read back), then the LDS writes
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int pc = 64 * i + lane;  // piece of the wave's range
      raw[i] = __builtin_nontemporal_load(src + (wb + pc / C < nblk ? pc : 0));
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int pc = 64 * i + lane;
      st[row_slot<BF16>(pc / C, pc % C)] = raw[i];
    }
    // only this wave reads its area: a wave-scope release/acquire orders the accesses (the
    // lanes of a wave run in lockstep and the wave's LDS operations complete in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < C; ++i) raw[i] = st[row_slot<BF16>(lane, i)];
    if (b >= nblk) return;
  } else {
    if (b >= nblk) return;
    const int64_t r = b / bpr;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(x) + (r * ld + 32 * (b - r * bpr)) * (BF16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < C; ++i) raw[i] = __builtin_nontemporal_load(src + i);
  }
  float w[32];
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) widen_signed8<HAD>(raw[i], sign_mask, 8 * i, w + 8 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[4 * i] = __uint_as_float(raw[i].x); w[4 * i + 1] = __uint_as_float(raw[i].y);
      w[4 * i + 2] = __uint_as_float(raw[i].z); w[4 * i + 3] = __uint_as_float(raw[i].w);
    }
    if (HAD) {
#pragma unroll
      for (int j = 0; j < 32; ++j)
        w[j] = __uint_as_float(__float_as_uint(w[j]) ^ (((sign_mask >> j) & 1u) << 31));
    }
  }
  // 32-point transform [P1 paragraph 2], then the block's scale and codes
  if (HAD) hadamard32_inlane(w);
  uint32_t sb;
  const u32x4 out = quant_block32<SR, CEIL, BF16>(w, seed, (uint64_t)(4 * b), sb);
  __builtin_nontemporal_store(out, codes + b);
  scales[b] = (uint8_t)sb;
}

// ---------------------------------------------------------------------------------------------
// 8x8 patch loader shared by the column and 2-D kernels: rows r0..r0+7, columns c0..c0+7.
// p[j][k] = x[r0 + j][c0 + k].
// ---------------------------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load_patch(const void* __restrict__ x, int64_t ld, int64_t r0,
                                           int64_t c0, float (&p)[8][8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) load8<BF16>(x, (r0 + j) * ld + c0, p[j]);
}

// Patch loader with the random signs of the column transform applied: position 8q + j of the
// 32-block is patch row j of quad lane q, negated when bit 8q + j of sign_mask is set. For bf16
// the sign goes in with the widening (adding 2^31 toggles bit 31 as a XOR does).
template <bool BF16>
__device__ __forceinline__ void load_patch_signed(const void* __restrict__ x, int64_t ld,
                                                  int64_t r0, int64_t c0, uint32_t sign_mask,
                                                  int q, float (&p)[8][8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t s = ((sign_mask >> (8 * q + j)) & 1u) << 31;
    if (BF16) {
      const u32x4 raw = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + (r0 + j) * ld + c0));
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[j][2 * i] = __uint_as_float((w[i] << 16) + s);
        p[j][2 * i + 1] = __uint_as_float((w[i] & 0xFFFF0000u) ^ s);
      }
    } else {
      load8<false>(x, (r0 + j) * ld + c0, p[j]);
#pragma unroll
      for (int k = 0; k < 8; ++k) p[j][k] = __uint_as_float(__float_as_uint(p[j][k]) ^ s);
    }
  }
}

// Column transform of a patch stack (signs already applied): the five butterfly stages per
// column, spans 1, 2, 4 down the lane's patch rows and 8, 16 across the quad.
__device__ __forceinline__ void fwht_columns(float (&p)[8][8], int q) {
  const uint32_t up8 = (q & 1) ? 0x80000000u : 0u;
  const uint32_t up16 = (q & 2) ? 0x80000000u : 0u;
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = p[j][k], b = p[j + h][k];
        p[j][k] = a + b;
        p[j + h][k] = a - b;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) p[j][k] = butterfly_xlane<kQuadXor1>(p[j][k], up8);
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) p[j][k] = butterfly_xlane<kQuadXor2>(p[j][k], up16);
}

// ---------------------------------------------------------------------------------------------
// Workgroup tiles of 256 rows x 128 columns for the column-blocked and 32x32 outputs. The 8 row
// tiles that share one 64-byte segment of a transposed scale row are given to the same XCD
// (workgroup id modulo 8) at consecutive positions, so their partial scale writes meet in one
// L2 instead of reaching memory as partial lines. Returns false for padding workgroups.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bool col_tile_of(int64_t n_rt, int64_t n_ct, int64_t& rt, int64_t& ct) {
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid & 7, slot = bid >> 3;
  const int64_t n_rg = (n_rt + 7) >> 3;           // groups of 8 row tiles
  const int64_t unit = (slot >> 3) * 8 + xcd;     // (column tile, row group) pair
  ct = unit / n_rg;
  rt = (unit - ct * n_rg) * 8 + (slot & 7);
  return ct < n_ct && rt < n_rt;
}

constexpr int kColTileRows = 256, kColTileCols = 128;
constexpr int kColHalves = kColTileCols / 128;
constexpr int kCodeStride = 144;  // LDS bytes per column of the code tile (128 + 16 padding)

// Store phase of a column tile (after a workgroup barrier): the codes of a column leave as one
// 128-byte piece (8 lanes per column, 16 bytes = one row block each, so that one store
// instruction writes the whole pieces of 8 columns); thread t writes the scale bytes of column t.
template <int TC = kColTileCols, int NT = kThreads>
__device__ __forceinline__ void col_tile_store(int tid, int64_t rows, int64_t cols, int64_t rb0,
                                               int nrb, int64_t ctile0, const uint8_t* ctile,
                                               const uint8_t* stile, uint8_t* __restrict__ codes_t,
                                               uint8_t* __restrict__ scales_t) {
  const int64_t rows2 = rows / 2;
#pragma unroll
  for (int round = 0; round < TC * 8 / NT; ++round) {
    const int c = round * (NT / 8) + (tid >> 3), rbl = tid & 7;
    if (ctile0 + c < cols && rbl < nrb)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(ctile + c * kCodeStride + rbl * 16),
          reinterpret_cast<u32x4*>(codes_t + (ctile0 + c) * rows2 + rb0 * 16 + rbl * 16));
  }
  for (int cs = tid; cs < TC; cs += NT) {
    if (ctile0 + cs >= cols) break;
    uint8_t* dst = scales_t + (ctile0 + cs) * (rows / 32) + rb0;
    const uint8_t* src = stile + cs * 8;
    if (nrb == 8 && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else {
      for (int i = 0; i < nrb; ++i) dst[i] = src[i];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 1x32 blocks down the columns (blocks along rows), output in the layout of the transpose:
// codes_t [cols][rows/2], scales_t [cols][rows/32]; the fp32-input path (bf16 input takes the
// whole-column kernel further down). A workgroup owns 256 rows x 128 columns;
// wave w handles row blocks w and w + 4 of the tile, lane = 4 * column-group + q. Each lane's
// 8 codes of a column (one dword) go to an LDS tile first, so the global writes are whole
// 128-byte column pieces.
// ---------------------------------------------------------------------------------------------
template <bool BF16, bool HAD, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint64_t seed, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, int64_t n_rt,
    int64_t n_ct) {
  static_assert(!BF16, "bf16 input takes quant_cols_bf16_kernel");
  __shared__ __attribute__((aligned(16))) uint8_t ctile[kColTileCols * kCodeStride];
  __shared__ __attribute__((aligned(16))) uint8_t stile[kColTileCols * 8];
  int64_t rt, ct;
  if (!col_tile_of(n_rt, n_ct, rt, ct)) return;  // uniform per workgroup

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane & 3, cg = lane >> 2;
  const int64_t rb0 = rt * 8;
  const int nrb = (int)min((int64_t)8, rows / 32 - rb0);
  const int64_t ctile0 = ct * kColTileCols;

#pragma unroll
  for (int pass = 0; pass < 2 * kColHalves; ++pass) {
    const int rbl = (pass & 1) * 4 + wave;
    const int ch = pass >> 1;                 // which 128-column slice of the tile
    const int64_t c0 = ctile0 + ch * 128 + cg * 8;
    if (rbl >= nrb || c0 >= cols) continue;  // whole quads leave together
    const int64_t rb = rb0 + rbl;
    const int64_t r0 = rb * 32 + 8 * q;
    float p[8][8];
    if (HAD) {
      load_patch_signed<BF16>(x, ld, r0, c0, sign_mask, q, p);
      fwht_columns(p, q);
    } else {
      load_patch<BF16>(x, ld, r0, c0, p);
    }

    uint32_t sb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, abs_bits(p[j][k]));
      m = max(m, dpp_u32<kQuadXor1>(m));
      m = max(m, dpp_u32<kQuadXor2>(m));
      sb[k] = scale_byte<CEIL>(m);
    }
    uint32_t r[8][8];  // r[j][k]: converter random word of patch element (j, k)
    if (SR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sr_rand8((uint64_t)((r0 + j) * cols + c0) >> 3, seed, r[j]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t word = 0;
      if (sb[k] != 0xFFu) {
        const float inv = inv_scale_from_byte(sb[k]);
        float col[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) col[j] = p[j][k] * inv;
        if (SR) {
          uint32_t rc[8];  // column k: element (j, k) of the patch for code j
#pragma unroll
          for (int j = 0; j < 8; ++j) rc[j] = r[j][k];
          word = sr_pack8(col, rc);
        } else {
          word = cvt_rne_pack8(col);
        }
      }
      const int cl = ch * 128 + cg * 8 + k;  // column within the tile
      *reinterpret_cast<uint32_t*>(ctile + cl * kCodeStride + rbl * 16 + 4 * q) = word;
      if (q == 0) stile[cl * 8 + rbl] = (uint8_t)sb[k];
    }
  }
  __syncthreads();
  col_tile_store(threadIdx.x, rows, cols, rb0, nrb, ctile0, ctile, stile, codes_t, scales_t);
}

// ---------------------------------------------------------------------------------------------
// 1x32 blocks down the columns of a bf16 tensor, whole 32-row columns per lane, as the row kernel
// quantizes them (no lane exchanges in the transform, one scale per lane). A workgroup owns 256
// rows x 64 CWV columns, with 4 CWV waves: pass p of wave w takes row block 4p + w % 4 of the
// 64 columns 64 (w / 4).., and lane l column l of those. Lane (q, cg) = (l / 8, l % 8) loads
// the 8 columns 8cg.. of rows 4q..4q+3 (8 lanes: one 128-byte row) and, for stochastic
// rounding, computes the Philox words of the same chunk of rows q, q + 8, q + 16, q + 24.
// The wave's own 4 KiB of LDS holds 32 rows of 128 bytes: first the values, which each lane
// reads back as the 16-bit entries of its column, then the random fields, stored with the
// layout of the values they round and read back the same way. Every access of the area covers
// whole 128-byte rows (no bank conflicts). A lane keeps the codes and scales of its two passes
// in registers; once all waves are done with their areas, the same 16 CWV KiB hold the code
// tile for the store phase. With at most 64 registers and 16 KiB of LDS per four waves, eight
// waves share a SIMD (stochastic rounding without the transform needs 75 registers: six waves,
// 2-11% faster than seven with 3 spilled). Measured on a 16384x28672 tensor (Hadamard, ceil, SR, CWV = 1): 128-column
// tiles with two columns per lane (128 registers, four waves per SIMD) 286-291 us; this kernel
// with the code tile beside the exchange areas (26 KiB, six waves) 264-266 us; as it stands
// 259-266 us (247 us with the scale fold). Code bytes stored straight from the lanes (16 bytes
// per line per store) were 20-30% slower. With nearest-even rounding the 8192x14336 Hadamard
// case took 58.6 us with the 8x8-patch kernel below and 54.8-55.4 us here.
// ---------------------------------------------------------------------------------------------
constexpr int kColLaneTileCols = 64;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool HAD, bool SR, bool CEIL, int CWV>
__global__ __launch_bounds__(kThreads * CWV) __attribute__((amdgpu_waves_per_eu(HAD || !SR ? 8 : 6, 8)))
void quant_cols_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint64_t seed, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, int64_t n_rt,
    int64_t n_ct) {
  constexpr int TC = kColLaneTileCols * CWV;
  static_assert(TC * (kCodeStride + 8) <= 4 * CWV * 4096, "the code tile fits in the areas");
  __shared__ __attribute__((aligned(16))) uint8_t xarea[4 * CWV * 4096];
  uint8_t* const ctile = xarea;                   // after both passes
  uint8_t* const stile = xarea + TC * kCodeStride;  // after both passes
  u32x4 codes[2];
  uint32_t sbv[2];
  int64_t rt, ct;
  if (!col_tile_of(n_rt, n_ct, rt, ct)) return;  // uniform per workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  const int q = lane >> 3, cg = lane & 7, wr = wave & 3, wc = wave >> 2;
  const int64_t rb0 = rt * 8;
  const int nrb = (int)min((int64_t)8, rows / 32 - rb0);
  const int64_t ctile0 = ct * TC;
  // the wave's 64 columns; a half past the last column loads the tile's first half instead
  const int64_t cw0 = ctile0 + 64 * wc, cl0 = cw0 < cols ? cw0 : ctile0;
  uint8_t* const xa = xarea + wave * 4096;
  // Lane parts of the addresses, fixed over the passes: the element offset of row 4q, chunk cg
  // from the row block's first row (a piece past the last column reads the tile's first piece
  // instead; its values are never stored), and the counter offset of row q, chunk cg.
  const int64_t xo = 4 * q * ld + (cl0 + 8 * cg < cols ? 8 * cg : 0);
  const int64_t go = q * (cols >> 3) + cg;

  // nearest-even: both passes' loads go out first (the rounding is short, so a wave's second
  // load would otherwise wait in the open; 10-15% on the 8B operands, within 1.5% on larger
  // ones); with SR the registers are not there, and the rounding hides the load
  constexpr bool kAhead = !SR;
  u32x4 raw2[2][4];
  if (kAhead) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int rbl = pass * 4 + wr;
      if (rbl < nrb) {
        const uint16_t* xb = x + (rb0 + rbl) * 32 * ld + cl0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          raw2[pass][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xb + j * ld + xo));
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rbl = pass * 4 + wr;
    if (rbl >= nrb) break;  // uniform per wave (rbl grows with the pass)
    const int64_t rb = rb0 + rbl;
    const uint16_t* xb = x + rb * 32 * ld + cl0;
    u32x4 raw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j] = kAhead ? raw2[pass][j]
                      : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xb + j * ld + xo));
    const uint64_t gb = (uint64_t)rb * 4 * (uint64_t)cols + (uint64_t)(cw0 >> 3);
    u32x4 wd[4];  // complemented Philox words of chunk cg of rows q + 8m
    if (SR) {
#pragma unroll
      for (int m = 0; m < 4; ++m) wd[m] = sr_words(gb + (uint64_t)m * cols + go, seed);
    }
    // values: area row r = 128 bytes, the 64 columns in order
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(xa + (4 * q + j) * 128 + 16 * cg) = raw[j];
    wave_sync();
    uint32_t val[32];  // row r of column `lane`
#pragma unroll
    for (int r = 0; r < 32; ++r) val[r] = *reinterpret_cast<const uint16_t*>(xa + r * 128 + 2 * lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read before the area is written again
    wave_sync();
    if (SR) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<u32x4*>(xa + (q + 8 * m) * 128 + 16 * cg) = wd[m];
      wave_sync();
    }
    uint32_t sm = sign_mask;
    asm volatile("" : "+s"(sm));  // sign bits made per pass, not held across the loop
    float w[32];
#pragma unroll
    for (int r = 0; r < 32; ++r)  // widen and apply the sign in one shift-and-add
      w[r] = __uint_as_float((val[r] << 16) + (HAD ? ((sm >> r) & 1u) << 31 : 0u));
    if (HAD) hadamard32_inlane(w);
    uint32_t sb;
    const u32x4 code = quant_block32_with<SR, CEIL, true>(
        w,
        [&](int d, uint32_t (&rw)[8]) {
#pragma unroll
          for (int k = 0; k < 8; ++k)  // the field of row 8d + k in the high half
            rw[k] = sr_word_lo(*reinterpret_cast<const uint16_t*>(xa + (8 * d + k) * 128 + 2 * lane));
        },
        sb);
    codes[pass] = code;
    sbv[pass] = sb;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // fields read before the next pass writes the area
    wave_sync();
  }
  __syncthreads();  // every wave is done with its area
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rbl = pass * 4 + wr, cl = 64 * wc + lane;
    if (rbl < nrb) {
      *reinterpret_cast<u32x4*>(ctile + cl * kCodeStride + rbl * 16) = codes[pass];
      stile[cl * 8 + rbl] = (uint8_t)sbv[pass];
    }
  }
  __syncthreads();
  col_tile_store<TC, kThreads * CWV>(threadIdx.x, rows, cols, rb0, nrb, ctile0, ctile, stile,
                                      codes_t, scales_t);
}

// ---------------------------------------------------------------------------------------------
// 32x32 tiles: one scale per tile from the tile maximum; every element is rounded once and
// written to the row-major codes and (optionally) to the K-major codes of the transpose.
// A workgroup owns 256 rows x 256 columns (8 x 8 tiles). Pass p of wave w covers row block
// (p & 1) * 4 + w and the 128-column half p >> 1; there lane = 16 * tile + 4 * column-group + q
// holds the 8x8 patch at rows 8q.., columns 8 (4 tile + column-group).., so the 16 lanes of a
// tile are one DPP row. Both code layouts are assembled in LDS and leave as whole 128-byte rows.
// ---------------------------------------------------------------------------------------------
constexpr int k2dTile = 256;
constexpr int k2dStride = 144;  // LDS bytes per row (row-major) or column (transposed) + padding

template <bool BF16, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_2d_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, int64_t n_ct) {
  // one code tile, used for the row-major codes and then for the transposed ones (half the LDS
  // of two tiles, so twice the workgroups per CU); each lane keeps its 4 patches' codes
  __shared__ __attribute__((aligned(16))) uint8_t ctile[k2dTile * k2dStride];  // [row or col][../2]
  __shared__ uint8_t stile[64];                                                 // [rb][cb]
  uint32_t Rk[4][8];  // codes of pass p: patch row j (nibble k = column k)
  const int64_t rt = blockIdx.x / n_ct, ct = blockIdx.x - rt * n_ct;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane & 3, cgl = lane >> 2;  // cgl = 4 * tile + column-group, 0..15
  const int64_t rtile0 = rt * k2dTile, ctile0 = ct * k2dTile;
  const int nrb = (int)min((int64_t)8, rows / 32 - rt * 8);
  const int ncb = (int)min((int64_t)8, cols / 32 - ct * 8);

#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int rbl = (pass & 1) * 4 + wave, ch = pass >> 1;
    const int cl0 = ch * 128 + cgl * 8;  // first column of the patch within the tile
    if (rbl >= nrb || cl0 >= ncb * 32) continue;  // whole 32x32 tiles leave together
    const int64_t r0 = rtile0 + rbl * 32 + 8 * q, c0 = ctile0 + cl0;
    float p[8][8];
    load_patch<BF16>(x, ld, r0, c0, p);

    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) m = max(m, abs_bits(p[j][k]));
    m = max(m, dpp_u32<kQuadXor1>(m));
    m = max(m, dpp_u32<kQuadXor2>(m));
    m = max(m, dpp_u32<kRowRor4>(m));
    m = max(m, dpp_u32<kRowRor8>(m));
    const uint32_t sb = scale_byte<CEIL>(m);

    uint32_t R[8];  // R[j] = codes of patch row j (nibble k = column k)
    if (sb == 0xFFu) {
#pragma unroll
      for (int j = 0; j < 8; ++j) R[j] = 0;
    } else {
      const float inv = inv_scale_from_byte(sb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int k = 0; k < 8; ++k) p[j][k] = p[j][k] * inv;
        if (SR) {
          uint32_t rw[8];
          sr_rand8((uint64_t)((r0 + j) * cols + c0) >> 3, seed, rw);
          R[j] = sr_pack8(p[j], rw);
        } else {
          R[j] = cvt_rne_pack8(p[j]);
        }
      }
    }
    const int rl0 = rbl * 32 + 8 * q;  // first row of the patch within the tile
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<uint32_t*>(ctile + (rl0 + j) * k2dStride + cl0 / 2) = R[j];
      Rk[pass][j] = R[j];
    }
    if ((lane & 15) == 0) stile[rbl * 8 + cl0 / 32] = (uint8_t)sb;
  }
  __syncthreads();

  // codes: 8 lanes per row (column) of the tile, 16 bytes each: every store instruction writes
  // the whole 128-byte pieces of 8 rows; first the row-major codes, then (the tile refilled
  // with the transposed patches) the codes of the transpose
  const int64_t cols2 = cols / 2, rows2 = rows / 2;
  const int seg = threadIdx.x & 7;
#pragma unroll
  for (int round = 0; round < k2dTile * 8 / kThreads; ++round) {
    const int i = round * (kThreads / 8) + (threadIdx.x >> 3);
    if (i < nrb * 32 && seg < ncb)  // a 32-column block is one 16-byte segment
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(ctile + i * k2dStride + 16 * seg),
          reinterpret_cast<u32x4*>(codes + (rtile0 + i) * cols2 + ctile0 / 2 + 16 * seg));
  }
  if (codes_t) {
    __syncthreads();  // every row-major piece has been read from the tile
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rbl = (pass & 1) * 4 + wave, ch = pass >> 1;
      const int cl0 = ch * 128 + cgl * 8;
      if (rbl >= nrb || cl0 >= ncb * 32) continue;
      transpose_nibbles8x8(Rk[pass]);  // Rk[pass][k] = codes of patch column k (nibble j = row j)
      const int rl0 = rbl * 32 + 8 * q;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint32_t*>(ctile + (cl0 + k) * k2dStride + rl0 / 2) = Rk[pass][k];
    }
    __syncthreads();
#pragma unroll
    for (int round = 0; round < k2dTile * 8 / kThreads; ++round) {
      const int i = round * (kThreads / 8) + (threadIdx.x >> 3);
      if (i < ncb * 32 && seg < nrb)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(ctile + i * k2dStride + 16 * seg),
            reinterpret_cast<u32x4*>(codes_t + (ctile0 + i) * rows2 + rtile0 / 2 + 16 * seg));
    }
  }
  // scales: thread t < 64 writes tile (t / 8, t % 8) to both layouts
  if (threadIdx.x < 64) {
    const int rbl = threadIdx.x >> 3, cbl = threadIdx.x & 7;
    if (rbl < nrb && cbl < ncb) {
      const uint8_t sb = stile[rbl * 8 + cbl];
      scales[(rt * 8 + rbl) * (cols / 32) + ct * 8 + cbl] = sb;
      if (scales_t) scales_t[(ct * 8 + cbl) * (rows / 32) + rt * 8 + rbl] = sb;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// B x B tiles, B = 8 or 64 [P3 "The fix ...", Table 4: the 32x32 rule with smaller and larger
// tiles]. A workgroup owns 256 rows x 256 columns, as the 32x32 kernel; pass p of wave w covers
// the 64x64 sub-tile t = 4p + w (sub-row t / 4, sub-column t % 4), where lane l holds the 8x8
// patch at rows 8 (l / 8), columns 8 (l % 8). With B = 8 a patch is a tile (its maximum stays in
// the lane); with B = 64 the sub-tile is a tile, its maximum reduced over the wave. Codes are
// assembled in LDS in both layouts and leave as whole 128-byte rows. Scales: B = 8, [rows/8]
// [cols/8] and [cols/8][rows/8]; B = 64, the GEMM layout [rows/64][cols/32] and
// [cols/64][rows/32], each tile's byte stored for both of its 32-wide halves. rows and cols
// are multiples of max(B, 32).
// ---------------------------------------------------------------------------------------------
template <int B, bool BF16, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_2d_var_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, int64_t n_ct) {
  static_assert(B == 8 || B == 64, "8x8 or 64x64 tiles");
  constexpr int NS = k2dTile / B;  // tiles per edge of the workgroup tile
  // one code tile for the row-major codes, then the transposed ones (as in the 32x32 kernel)
  __shared__ __attribute__((aligned(16))) uint8_t ctile[k2dTile * k2dStride];  // [row or col][../2]
  __shared__ __attribute__((aligned(16))) uint8_t stile[NS * NS];               // [tr][tc]
  uint32_t Rk[4][8];  // codes of pass p: patch row j (nibble k = column k)
  const int64_t rt = blockIdx.x / n_ct, ct = blockIdx.x - rt * n_ct;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pr = lane >> 3, pc = lane & 7;
  const int64_t rtile0 = rt * k2dTile, ctile0 = ct * k2dTile;
  const int nr = (int)min((int64_t)k2dTile, rows - rtile0);  // multiple of 32 (of 64 for B = 64)
  const int nc = (int)min((int64_t)k2dTile, cols - ctile0);

#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int t = 4 * pass + wave, sr = t >> 2, sc = t & 3;
    const int rl0 = 64 * sr + 8 * pr, cl0 = 64 * sc + 8 * pc;  // patch origin in the tile
    if (B == 64) {
      if (64 * sr >= nr || 64 * sc >= nc) continue;  // whole 64x64 tiles, uniform per wave
    } else if (rl0 >= nr || cl0 >= nc) {
      continue;                                       // whole 8x8 tiles
    }
    const int64_t r0 = rtile0 + rl0, c0 = ctile0 + cl0;
    float p[8][8];
    load_patch<BF16>(x, ld, r0, c0, p);

    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) m = max(m, abs_bits(p[j][k]));
    if (B == 64) {
      m = max(m, dpp_u32<kQuadXor1>(m));
      m = max(m, dpp_u32<kQuadXor2>(m));
      m = max(m, dpp_u32<kRowRor4>(m));
      m = max(m, dpp_u32<kRowRor8>(m));
      m = max(m, (uint32_t)__shfl_xor((int)m, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    }
    const uint32_t sb = scale_byte<CEIL>(m);

    uint32_t R[8];  // R[j] = codes of patch row j (nibble k = column k)
    if (sb == 0xFFu) {
#pragma unroll
      for (int j = 0; j < 8; ++j) R[j] = 0;
    } else {
      const float inv = inv_scale_from_byte(sb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int k = 0; k < 8; ++k) p[j][k] = p[j][k] * inv;
        if (SR) {
          uint32_t rw[8];
          sr_rand8((uint64_t)((r0 + j) * cols + c0) >> 3, seed, rw);
          R[j] = sr_pack8(p[j], rw);
        } else {
          R[j] = cvt_rne_pack8(p[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<uint32_t*>(ctile + (rl0 + j) * k2dStride + cl0 / 2) = R[j];
      Rk[pass][j] = R[j];
    }
    if (B == 8) stile[(rl0 / 8) * NS + cl0 / 8] = (uint8_t)sb;
    else if (lane == 0) stile[sr * NS + sc] = (uint8_t)sb;
  }
  __syncthreads();

  // codes: 8 lanes per row (column) of the tile, 16 bytes (32 codes) each; the row-major codes
  // first, then the tile refilled with the transposed patches
  const int64_t cols2 = cols / 2, rows2 = rows / 2;
  const int seg = threadIdx.x & 7;
#pragma unroll
  for (int round = 0; round < k2dTile * 8 / kThreads; ++round) {
    const int i = round * (kThreads / 8) + (threadIdx.x >> 3);
    if (i < nr && 32 * seg < nc)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(ctile + i * k2dStride + 16 * seg),
          reinterpret_cast<u32x4*>(codes + (rtile0 + i) * cols2 + ctile0 / 2 + 16 * seg));
  }
  if (codes_t) {
    __syncthreads();  // every row-major piece has been read from the tile
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int t = 4 * pass + wave, sr = t >> 2, sc = t & 3;
      const int rl0 = 64 * sr + 8 * pr, cl0 = 64 * sc + 8 * pc;
      if (B == 64) {
        if (64 * sr >= nr || 64 * sc >= nc) continue;
      } else if (rl0 >= nr || cl0 >= nc) {
        continue;
      }
      transpose_nibbles8x8(Rk[pass]);  // Rk[pass][k] = codes of patch column k (nibble j = row j)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint32_t*>(ctile + (cl0 + k) * k2dStride + rl0 / 2) = Rk[pass][k];
    }
    __syncthreads();
#pragma unroll
    for (int round = 0; round < k2dTile * 8 / kThreads; ++round) {
      const int i = round * (kThreads / 8) + (threadIdx.x >> 3);
      if (i < nc && 32 * seg < nr)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(ctile + i * k2dStride + 16 * seg),
            reinterpret_cast<u32x4*>(codes_t + (ctile0 + i) * rows2 + rtile0 / 2 + 16 * seg));
    }
  }
  if (B == 8) {
    // thread t: scale row (column) t / 8 of the tile, 4 bytes (32 source columns) at t % 8
    const int a = threadIdx.x >> 3, b4 = 4 * (threadIdx.x & 7);
    if (8 * a < nr && 8 * b4 < nc)
      *reinterpret_cast<uint32_t*>(scales + (rtile0 / 8 + a) * (cols / 8) + ctile0 / 8 + b4) =
          *reinterpret_cast<const uint32_t*>(stile + a * NS + b4);
    if (scales_t && 8 * a < nc && 8 * b4 < nr) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= (uint32_t)stile[(b4 + i) * NS + a] << (8 * i);
      *reinterpret_cast<uint32_t*>(scales_t + (ctile0 / 8 + a) * (rows / 8) + rtile0 / 8 + b4) = w;
    }
  } else if (threadIdx.x < NS * NS) {
    const int i = threadIdx.x / NS, j = threadIdx.x % NS;
    if (64 * i < nr && 64 * j < nc) {
      const uint16_t v = (uint16_t)(stile[i * NS + j] * 0x0101u);
      *reinterpret_cast<uint16_t*>(scales + (rtile0 / 64 + i) * (cols / 32) + ctile0 / 32 + 2 * j) = v;
      if (scales_t)
        *reinterpret_cast<uint16_t*>(scales_t + (ctile0 / 64 + j) * (rows / 32) + rtile0 / 32 + 2 * i) = v;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 1D scale-difference map [P3 "The aha: transposition scrambles the blocks", Figure 1]: for
// every element, the scale exponent of its 1x32 block along the row minus that of its 1x32
// block down the column, saturated to [-127, 127] (-128 where a block maximum is not finite).
// Wave unit u = 4 blockIdx + wave covers row block u / ncg (32 rows) and 128-column group
// u % ncg, laid out as in the 32x32 kernel: lane = 16 tile + 4 cg + q holds the 8x8 patch at
// rows 8q, columns 8 (4 tile + cg). Column maxima reduce over the quad (q), row maxima over the
// four column groups of the tile (DPP row rotations by 4 and 8).
// ---------------------------------------------------------------------------------------------
template <bool BF16, bool CEIL>
__global__ __launch_bounds__(kThreads) void mismatch_map_kernel(
    const void* __restrict__ x, int64_t cols, int64_t ld, u32x2* __restrict__ map,
    int64_t nunits, int64_t ncg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t u = (int64_t)blockIdx.x * 4 + wave;
  if (u >= nunits) return;  // uniform per wave
  const int q = lane & 3, cgl = lane >> 2;
  const int64_t rb = u / ncg, g = u - rb * ncg;
  const int64_t r0 = rb * 32 + 8 * q, c0 = g * 128 + 8 * cgl;
  if (c0 >= cols) return;  // whole 32-column tiles (cols % 32 == 0), i.e. whole DPP rows
  float p[8][8];
  load_patch<BF16>(x, ld, r0, c0, p);
  uint32_t sc[8], sr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, abs_bits(p[j][k]));
    m = max(m, dpp_u32<kQuadXor1>(m));
    m = max(m, dpp_u32<kQuadXor2>(m));
    sc[k] = scale_byte<CEIL>(m);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, abs_bits(p[j][k]));
    m = max(m, dpp_u32<kRowRor4>(m));
    m = max(m, dpp_u32<kRowRor8>(m));
    sr[j] = scale_byte<CEIL>(m);
  }
  const int64_t cpr = cols / 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int d = (int)sr[j] - (int)sc[k];
      d = min(max(d, -127), 127);
      if (sr[j] == 0xFFu || sc[k] == 0xFFu) d = -128;
      w[k >> 2] |= ((uint32_t)d & 0xFFu) << (8 * (k & 3));
    }
    __builtin_nontemporal_store(u32x2{w[0], w[1]}, map + (r0 + j) * cpr + c0 / 8);
  }
}

// ---------------------------------------------------------------------------------------------
// MXFP8 [P3 "The fix, and its supporting cast": queries and keys in MXFP8]: the same block
// structure with one code byte per element (E4M3 or E5M2). Along rows a lane's 8 codes are 8
// consecutive output bytes; down the columns a lane's 8 codes of one column go to an LDS tile
// of 256 bytes per column (the tile's 256 rows), which leaves as whole 256-byte pieces.
// ---------------------------------------------------------------------------------------------
template <int FMT, bool BF16, bool HAD, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_rows_fp8_kernel(
    const void* __restrict__ x, int64_t nchunks, int64_t cpr, int64_t ld, int contiguous,
    uint32_t sign_mask, uint64_t seed, u32x2* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int q = threadIdx.x & 3;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kRowChunksPerThread) + threadIdx.x;
  float v[kRowChunksPerThread][8];
#pragma unroll
  for (int u = 0; u < kRowChunksPerThread; ++u) {
    const int64_t g = base + (int64_t)u * kThreads;
    if (g < nchunks) {
      int64_t off = 8 * g;
      if (!contiguous) {
        const int64_t r = g / cpr;
        off = r * ld + 8 * (g - r * cpr);
      }
      load8<BF16>(x, off, v[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kRowChunksPerThread; ++u) {
    const int64_t g = base + (int64_t)u * kThreads;
    if (g >= nchunks) continue;  // quads are all in or all out (cols % 32 == 0)
    uint32_t sb;
    const uint2 w = quant_chunk8_fp8<FMT, HAD, SR, CEIL>(v[u], q, sign_mask, seed, (uint64_t)g, sb);
    __builtin_nontemporal_store(u32x2{w.x, w.y}, codes + g);
    if (q == 0) scales[g >> 2] = (uint8_t)sb;
  }
}

constexpr int kCodeStride8 = 272;  // LDS bytes per column of the FP8 code tile (256 + 16)

template <int FMT, bool BF16, bool HAD, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) void quant_cols_fp8_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint64_t seed, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, int64_t n_rt,
    int64_t n_ct) {
  static_assert(!BF16, "bf16 input takes quant_cols_fp8_bf16_kernel");
  __shared__ __attribute__((aligned(16))) uint8_t ctile[kColTileCols * kCodeStride8];
  __shared__ __attribute__((aligned(16))) uint8_t stile[kColTileCols * 8];
  int64_t rt, ct;
  if (!col_tile_of(n_rt, n_ct, rt, ct)) return;  // uniform per workgroup

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane & 3, cg = lane >> 2;
  const int64_t rb0 = rt * 8;
  const int nrb = (int)min((int64_t)8, rows / 32 - rb0);
  const int64_t ctile0 = ct * kColTileCols;

#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rbl = pass * 4 + wave;
    const int64_t c0 = ctile0 + cg * 8;
    if (rbl >= nrb || c0 >= cols) continue;  // whole quads leave together
    const int64_t r0 = (rb0 + rbl) * 32 + 8 * q;
    float p[8][8];
    if (HAD) {
      load_patch_signed<BF16>(x, ld, r0, c0, sign_mask, q, p);
      fwht_columns(p, q);
    } else {
      load_patch<BF16>(x, ld, r0, c0, p);
    }

    uint32_t sb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, abs_bits(p[j][k]));
      m = max(m, dpp_u32<kQuadXor1>(m));
      m = max(m, dpp_u32<kQuadXor2>(m));
      sb[k] = scale_byte_fp8<CEIL, FMT>(m);
    }
    uint32_t r[8][8];  // r[j][k]: random field of patch element (j, k)
    if (SR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sr_fields8((uint64_t)((r0 + j) * cols + c0) >> 3, seed, r[j]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint2 w = make_uint2(0u, 0u);
      if (sb[k] != 0xFFu) {
        const float inv = inv_scale_from_byte(sb[k]);
        float col[8];
        uint32_t rc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          col[j] = p[j][k] * inv;
          rc[j] = SR ? r[j][k] : 0u;
        }
        w = fp8_pack8<FMT, SR>(col, rc);
      }
      const int cl = cg * 8 + k;  // column within the tile
      *reinterpret_cast<u32x2*>(ctile + cl * kCodeStride8 + rbl * 32 + 8 * q) = u32x2{w.x, w.y};
      if (q == 0) stile[cl * 8 + rbl] = (uint8_t)sb[k];
    }
  }
  __syncthreads();

  // codes: 16 lanes per column, 16 bytes each, so one store instruction writes the 256-byte
  // pieces of 4 columns
#pragma unroll
  for (int round = 0; round < kColTileCols * 16 / kThreads; ++round) {
    const int c = round * (kThreads / 16) + (threadIdx.x >> 4), piece = threadIdx.x & 15;
    if (ctile0 + c < cols && piece < 2 * nrb)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(ctile + c * kCodeStride8 + 16 * piece),
          reinterpret_cast<u32x4*>(codes_t + (ctile0 + c) * rows + rb0 * 32 + 16 * piece));
  }
  for (int cs = threadIdx.x; cs < kColTileCols; cs += kThreads) {
    if (ctile0 + cs >= cols) break;
    uint8_t* dst = scales_t + (ctile0 + cs) * (rows / 32) + rb0;
    const uint8_t* src = stile + cs * 8;
    if (nrb == 8 && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else {
      for (int i = 0; i < nrb; ++i) dst[i] = src[i];
    }
  }
}

// MXFP8 down the columns of a bf16 tensor with the whole-column kernel's layout: a workgroup
// owns 256 rows x 64 columns, lane l the 32-row column l of a row block, whose 32 code bytes
// (two 16-byte pieces) stay in registers over the two passes; after them the same LDS holds the
// code tile (256 bytes per column, 272-byte stride) for 256-byte stores. Stochastic rounding
// without the transform needs 75 registers and runs at six waves per SIMD: at eight, the 15
// registers spilled to scratch made it 18% slower on a 16384x8192 tensor.
template <int FMT, bool HAD, bool SR, bool CEIL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HAD || !SR ? 8 : 6, 8)))
void quant_cols_fp8_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint64_t seed, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, int64_t n_rt,
    int64_t n_ct) {
  constexpr int kCodeBytes = kColLaneTileCols * kCodeStride8;  // 17 KiB
  static_assert(kCodeBytes + kColLaneTileCols * 8 >= 4 * 4096, "the exchange areas fit");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kCodeBytes + kColLaneTileCols * 8];
  uint8_t* const ctile = lds;               // after both passes
  uint8_t* const stile = lds + kCodeBytes;  // after both passes
  u32x4 codes[2][2];
  uint32_t sbv[2];
  int64_t rt, ct;
  if (!col_tile_of(n_rt, n_ct, rt, ct)) return;  // uniform per workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  const int q = lane >> 3, cg = lane & 7;
  const int64_t rb0 = rt * 8;
  const int nrb = (int)min((int64_t)8, rows / 32 - rb0);
  const int64_t ctile0 = ct * kColLaneTileCols;
  uint8_t* const xa = lds + wave * 4096;
  const int64_t xo = 4 * q * ld + (ctile0 + 8 * cg < cols ? 8 * cg : 0);
  const int64_t go = q * (cols >> 3) + cg;

#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rbl = pass * 4 + wave;
    if (rbl >= nrb) break;  // uniform per wave (rbl grows with the pass)
    const int64_t rb = rb0 + rbl;
    const uint16_t* xb = x + rb * 32 * ld + ctile0;
    u32x4 raw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xb + j * ld + xo));
    const uint64_t gb = (uint64_t)rb * 4 * (uint64_t)cols + (uint64_t)(ctile0 >> 3);
    u32x4 wd[4];  // complemented Philox words of chunk cg of rows q + 8m
    if (SR) {
#pragma unroll
      for (int m = 0; m < 4; ++m) wd[m] = sr_words(gb + (uint64_t)m * cols + go, seed);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(xa + (4 * q + j) * 128 + 16 * cg) = raw[j];
    wave_sync();
    uint32_t val[32];  // row r of column `lane`
#pragma unroll
    for (int r = 0; r < 32; ++r) val[r] = *reinterpret_cast<const uint16_t*>(xa + r * 128 + 2 * lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read before the area is written again
    wave_sync();
    if (SR) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<u32x4*>(xa + (q + 8 * m) * 128 + 16 * cg) = wd[m];
      wave_sync();
    }
    uint32_t sm = sign_mask;
    asm volatile("" : "+s"(sm));  // sign bits made per pass, not held across the loop
    float w[32];
#pragma unroll
    for (int r = 0; r < 32; ++r)
      w[r] = __uint_as_float((val[r] << 16) + (HAD ? ((sm >> r) & 1u) << 31 : 0u));
    if (HAD) hadamard32_inlane(w);
    const uint32_t sb = scale_byte_fp8<CEIL, FMT>(block32_amax_bits(w));
    uint32_t o[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (sb != 0xFFu) {
      const float inv = inv_scale_from_byte(sb);
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // rows 8d .. 8d + 7
        float v8[8];
        uint32_t r8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v8[k] = w[8 * d + k] * inv;
          // the raw field of row 8d + k (the area holds it complemented)
          r8[k] = SR ? ~(uint32_t)*reinterpret_cast<const uint16_t*>(xa + (8 * d + k) * 128 + 2 * lane)
                     : 0u;
        }
        const uint2 pr = fp8_pack8<FMT, SR>(v8, r8);
        o[2 * d] = pr.x;
        o[2 * d + 1] = pr.y;
      }
    }
    codes[pass][0] = u32x4{o[0], o[1], o[2], o[3]};
    codes[pass][1] = u32x4{o[4], o[5], o[6], o[7]};
    sbv[pass] = sb;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // fields read before the next pass writes the area
    wave_sync();
  }
  __syncthreads();  // every wave is done with its area
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rbl = pass * 4 + wave;
    if (rbl < nrb) {
      *reinterpret_cast<u32x4*>(ctile + lane * kCodeStride8 + rbl * 32) = codes[pass][0];
      *reinterpret_cast<u32x4*>(ctile + lane * kCodeStride8 + rbl * 32 + 16) = codes[pass][1];
      stile[lane * 8 + rbl] = (uint8_t)sbv[pass];
    }
  }
  __syncthreads();
  // codes: 16 lanes per column, 16 bytes each (one store instruction writes the 256-byte pieces
  // of 4 columns); then thread t the scale bytes of column t
#pragma unroll
  for (int round = 0; round < kColLaneTileCols * 16 / kThreads; ++round) {
    const int c = round * (kThreads / 16) + (threadIdx.x >> 4), piece = threadIdx.x & 15;
    if (ctile0 + c < cols && piece < 2 * nrb)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(ctile + c * kCodeStride8 + 16 * piece),
          reinterpret_cast<u32x4*>(codes_t + (ctile0 + c) * rows + rb0 * 32 + 16 * piece));
  }
  if ((int)threadIdx.x < kColLaneTileCols && ctile0 + threadIdx.x < cols) {
    uint8_t* dst = scales_t + (ctile0 + threadIdx.x) * (rows / 32) + rb0;
    const uint8_t* src = stile + threadIdx.x * 8;
    if (nrb == 8 && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else {
      for (int i = 0; i < nrb; ++i) dst[i] = src[i];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Dequantize: out = E2M1(code) * 2^(byte-127) in fp32; optional inverse rotation (1/32) D H
// per 32-block along the row. One lane per 8 elements, flat over the tensor.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t E = (code >> 1) & 3u, M = code & 1u;
  const uint32_t mag = E ? (((E + 126u) << 23) | (M << 22)) : (M ? 0x3F000000u : 0u);
  return __uint_as_float(mag | ((code & 8u) << 28));
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
    int64_t cols, int block_rows, int inv_had, uint32_t sign_mask, float* __restrict__ out) {
  const int64_t cpr = cols / 8;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= rows * cpr) return;  // quads stay whole (cols % 32 == 0)
  const int64_t row = g / cpr;
  const int64_t cc = g - row * cpr;
  const uint32_t word = codes[g];
  const uint32_t s = scales[(row / block_rows) * (cols / 32) + (cc >> 2)];
  float v[8];
  if (s == 0xFFu) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(0x7FC00000u);
  } else {
    const float p = __uint_as_float(s ? (s << 23) : 0x00400000u);  // 2^(s-127)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = e2m1_value((word >> (4 * k)) & 0xFu) * p;
  }
  if (inv_had) {
    const int q = threadIdx.x & 3;
    fwht8_inlane(v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = butterfly_xlane<kQuadXor1>(v[k], (q & 1) ? 0x80000000u : 0u);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = butterfly_xlane<kQuadXor2>(v[k], (q & 2) ? 0x80000000u : 0u);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = v[k] * 0.03125f;
      v[k] = __uint_as_float(__float_as_uint(v[k]) ^ (((sign_mask >> (8 * q + k)) & 1u) << 31));
    }
  }
  float4* o = reinterpret_cast<float4*>(out + 8 * g);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------------------------
// host-side dispatch over the compile-time variants
// ---------------------------------------------------------------------------------------------
template <bool BF16, bool HAD, bool SR, bool CEIL>
hipError_t launch_rows(const QuantArgs& a) {
  const int64_t bpr = a.cols / 32;
  const int64_t nblk = a.rows * bpr;
  const int64_t nblocks = (nblk + kThreads - 1) / kThreads;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_rows_kernel<BF16, HAD, SR, CEIL>), dim3((unsigned)nblocks), dim3(kThreads),
                     0, (hipStream_t)a.stream, a.x, nblk, bpr, a.ld, a.ld == a.cols ? 1 : 0,
                     a.sign_mask, a.seed, reinterpret_cast<u32x4*>(a.codes), a.scales);
  return hipGetLastError();
}

// Grid of the 256x128 column tiles: 64 workgroup ids per 8 (column tile, row group) units.
inline int64_t col_tile_grid(int64_t rows, int64_t cols, int64_t& n_rt, int64_t& n_ct,
                             int64_t tile_cols = kColTileCols) {
  n_rt = (rows + kColTileRows - 1) / kColTileRows;
  n_ct = (cols + tile_cols - 1) / tile_cols;
  const int64_t units = n_ct * ((n_rt + 7) / 8);
  return ((units + 7) / 8) * 64;
}

template <bool BF16, bool HAD, bool SR, bool CEIL>
hipError_t launch_cols(const QuantArgs& a) {
  int64_t n_rt, n_ct;
  if constexpr (BF16) {
    // nearest-even: 128-column tiles (two waves per row block) ran up to 6% faster than 64;
    // stochastic rounding: 0.5-1% slower
    constexpr int CWV = SR ? 1 : 2;
    const int64_t nblocks = col_tile_grid(a.rows, a.cols, n_rt, n_ct, kColLaneTileCols * CWV);
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_cols_bf16_kernel<HAD, SR, CEIL, CWV>), dim3((unsigned)nblocks),
                       dim3(kThreads * CWV), 0, (hipStream_t)a.stream,
                       reinterpret_cast<const uint16_t*>(a.x), a.rows, a.cols, a.ld, a.sign_mask,
                       a.seed, a.codes, a.scales, n_rt, n_ct);
  } else {
    const int64_t nblocks = col_tile_grid(a.rows, a.cols, n_rt, n_ct);
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_cols_kernel<false, HAD, SR, CEIL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, (hipStream_t)a.stream, a.x, a.rows, a.cols, a.ld,
                       a.sign_mask, a.seed, a.codes, a.scales, n_rt, n_ct);
  }
  return hipGetLastError();
}

template <bool BF16, bool SR, bool CEIL>
hipError_t launch_2d(const QuantArgs& a) {
  const int64_t n_rt = (a.rows + k2dTile - 1) / k2dTile, n_ct = (a.cols + k2dTile - 1) / k2dTile;
  if (n_rt * n_ct > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_2d_kernel<BF16, SR, CEIL>), dim3((unsigned)(n_rt * n_ct)), dim3(kThreads),
                     0, (hipStream_t)a.stream, a.x, a.rows, a.cols, a.ld, a.seed, a.codes, a.scales,
                     a.codes_t, a.scales_t, n_ct);
  return hipGetLastError();
}

template <bool BF16, bool HAD, bool SR>
hipError_t pick_rule_1d(const QuantArgs& a) {
  if (a.axis == 1)
    return a.ceil ? launch_rows<BF16, HAD, SR, true>(a) : launch_rows<BF16, HAD, SR, false>(a);
  return a.ceil ? launch_cols<BF16, HAD, SR, true>(a) : launch_cols<BF16, HAD, SR, false>(a);
}

template <bool BF16>
hipError_t pick_1d(const QuantArgs& a) {
  if (a.hadamard)
    return a.sr ? pick_rule_1d<BF16, true, true>(a) : pick_rule_1d<BF16, true, false>(a);
  return a.sr ? pick_rule_1d<BF16, false, true>(a) : pick_rule_1d<BF16, false, false>(a);
}

template <bool BF16>
hipError_t pick_2d(const QuantArgs& a) {
  if (a.sr) return a.ceil ? launch_2d<BF16, true, true>(a) : launch_2d<BF16, true, false>(a);
  return a.ceil ? launch_2d<BF16, false, true>(a) : launch_2d<BF16, false, false>(a);
}

template <int B, bool BF16, bool SR, bool CEIL>
hipError_t launch_2d_var(const QuantArgs& a) {
  const int64_t n_rt = (a.rows + k2dTile - 1) / k2dTile, n_ct = (a.cols + k2dTile - 1) / k2dTile;
  if (n_rt * n_ct > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_2d_var_kernel<B, BF16, SR, CEIL>), dim3((unsigned)(n_rt * n_ct)),
                     dim3(kThreads), 0, (hipStream_t)a.stream, a.x, a.rows, a.cols, a.ld, a.seed,
                     a.codes, a.scales, a.codes_t, a.scales_t, n_ct);
  return hipGetLastError();
}

template <int B, bool BF16>
hipError_t pick_2d_var(const QuantArgs& a) {
  if (a.sr) return a.ceil ? launch_2d_var<B, BF16, true, true>(a) : launch_2d_var<B, BF16, true, false>(a);
  return a.ceil ? launch_2d_var<B, BF16, false, true>(a) : launch_2d_var<B, BF16, false, false>(a);
}

template <bool BF16, bool CEIL>
hipError_t launch_mismatch(const void* x, int64_t rows, int64_t cols, int64_t ld, int8_t* map,
                           void* stream) {
  const int64_t ncg = (cols + 127) / 128, nunits = (rows / 32) * ncg;
  const int64_t nblocks = (nunits + 3) / 4;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mismatch_map_kernel<BF16, CEIL>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                     (hipStream_t)stream, x, cols, ld, reinterpret_cast<u32x2*>(map), nunits, ncg);
  return hipGetLastError();
}

template <int FMT, bool BF16, bool HAD, bool SR, bool CEIL>
hipError_t launch_fp8(const QuantArgs& a) {
  if (a.axis == 1) {
    const int64_t cpr = a.cols / 8;
    const int64_t nchunks = a.rows * cpr;
    const int64_t per_block = kThreads * kRowChunksPerThread;
    const int64_t nblocks = (nchunks + per_block - 1) / per_block;
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_rows_fp8_kernel<FMT, BF16, HAD, SR, CEIL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, (hipStream_t)a.stream, a.x, nchunks, cpr, a.ld,
                       a.ld == a.cols ? 1 : 0, a.sign_mask, a.seed,
                       reinterpret_cast<u32x2*>(a.codes), a.scales);
  } else if constexpr (BF16) {
    int64_t n_rt, n_ct;
    const int64_t nblocks = col_tile_grid(a.rows, a.cols, n_rt, n_ct, kColLaneTileCols);
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_cols_fp8_bf16_kernel<FMT, HAD, SR, CEIL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, (hipStream_t)a.stream,
                       reinterpret_cast<const uint16_t*>(a.x), a.rows, a.cols, a.ld, a.sign_mask,
                       a.seed, a.codes, a.scales, n_rt, n_ct);
  } else {
    int64_t n_rt, n_ct;
    const int64_t nblocks = col_tile_grid(a.rows, a.cols, n_rt, n_ct);
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_cols_fp8_kernel<FMT, false, HAD, SR, CEIL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, (hipStream_t)a.stream, a.x, a.rows, a.cols, a.ld,
                       a.sign_mask, a.seed, a.codes, a.scales, n_rt, n_ct);
  }
  return hipGetLastError();
}

template <int FMT, bool BF16, bool HAD>
hipError_t pick_fp8_rule(const QuantArgs& a) {
  if (a.sr) return a.ceil ? launch_fp8<FMT, BF16, HAD, true, true>(a)
                          : launch_fp8<FMT, BF16, HAD, true, false>(a);
  return a.ceil ? launch_fp8<FMT, BF16, HAD, false, true>(a)
                : launch_fp8<FMT, BF16, HAD, false, false>(a);
}

template <int FMT>
hipError_t pick_fp8(const QuantArgs& a) {
  if (a.bf16) return a.hadamard ? pick_fp8_rule<FMT, true, true>(a) : pick_fp8_rule<FMT, true, false>(a);
  return a.hadamard ? pick_fp8_rule<FMT, false, true>(a) : pick_fp8_rule<FMT, false, false>(a);
}

}  // namespace

hipError_t mx_launch_quantize(const QuantArgs& a) {
  return a.bf16 ? pick_1d<true>(a) : pick_1d<false>(a);
}

hipError_t mx_launch_quantize_2d(const QuantArgs& a) {
  return a.bf16 ? pick_2d<true>(a) : pick_2d<false>(a);
}

hipError_t mx_launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, int block_rows, int inv_had, uint32_t sign_mask,
                                float* out, void* stream) {
  const int64_t nblocks = (rows * (cols / 8) + kThreads - 1) / kThreads;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)nblocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint32_t*>(codes), scales, rows, cols, block_rows,
                     inv_had, sign_mask, out);
  return hipGetLastError();
}

hipError_t mx_launch_quantize_fp8(const QuantArgs& a, int fmt) {
  return fmt == 0 ? pick_fp8<0>(a) : pick_fp8<1>(a);
}

hipError_t mx_launch_quantize_2d_blocks(const QuantArgs& a, int block) {
  if (block == 32) return mx_launch_quantize_2d(a);
  if (block == 8) return a.bf16 ? pick_2d_var<8, true>(a) : pick_2d_var<8, false>(a);
  return a.bf16 ? pick_2d_var<64, true>(a) : pick_2d_var<64, false>(a);
}

hipError_t mx_launch_scale_mismatch(const void* x, bool bf16, int64_t rows, int64_t cols,
                                    int64_t ld, bool ceil, int8_t* map, void* stream) {
  if (bf16) return ceil ? launch_mismatch<true, true>(x, rows, cols, ld, map, stream)
                        : launch_mismatch<true, false>(x, rows, cols, ld, map, stream);
  return ceil ? launch_mismatch<false, true>(x, rows, cols, ld, map, stream)
              : launch_mismatch<false, false>(x, rows, cols, ld, map, stream);
}
