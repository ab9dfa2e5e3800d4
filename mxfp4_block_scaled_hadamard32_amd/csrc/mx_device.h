// mx_device.h — device-side building blocks of the gfx950 MXFP4 path (quantize and GEMM
// kernels include it; it is not part of the C ABI).
//
// Pages, cited by title and section:
//  [P1] "Block-Scaled MXFP4 With Stochastic Hadamard Rounding Matches BF16 Convergence on 70B
//       Pre-Training", paragraphs 1-2 (E8M0 per 32 E2M1 values; 32-point Walsh-Hadamard in
//       registers before packing to 4 bits).
//  [P3] "Stable FP4 Training via Transposition-Invariant Block Quantization", sections "Why FP4
//       training is the current frontier" (E2M1; scale from the block maximum) and "The fix,
//       and its supporting cast" (power-of-two scale rounded up; stochastic rounding).
//  [P4] "Training LLMs with MXFP4", abstract (stochastic rounding, random Hadamard signs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// lane exchange inside a quad (4 consecutive lanes) through DPP quad_perm
// ---------------------------------------------------------------------------------------------
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;  // rotate right by 4 within a row of 16 lanes
constexpr int kRowRor8 = 0x128;  // rotate right by 8 within a row of 16 lanes

// Every caller exchanges inside whole quads or whole 16-lane rows of active lanes, so no source
// lane is inactive; bound_ctrl lets the compiler fold the move into the consuming add or max.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// ---------------------------------------------------------------------------------------------
// widening: bf16 -> fp32 is exact (the bf16 bits are the high half of the fp32 bits)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void widen_bf16x8(const u32x4 raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------------------------------------
// 32-point Walsh-Hadamard transform [P1 paragraph 2], unnormalised, natural order: butterfly
// stages of span 1, 2, 4 inside a lane's 8 values, then span 8 and 16 across the lanes of a
// quad (lane bit 0 carries span 8, lane bit 1 carries span 16). Each output of a stage is one
// fp32 add or subtract of the two stage inputs, so the result does not depend on which lane
// computes it.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void fwht8_inlane(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// Cross-lane stage: the lane whose quad bit is clear computes own + partner, the other
// partner - own (its own value is the stage's second operand). upper_sign is 0x80000000 on the
// lanes with the bit set, 0 otherwise.
template <int CTRL>
__device__ __forceinline__ float butterfly_xlane(float own, uint32_t upper_sign) {
  const float partner = dpp_f32<CTRL>(own);
  return partner + __uint_as_float(__float_as_uint(own) ^ upper_sign);
}

// ---------------------------------------------------------------------------------------------
// E8M0 scale byte from the block maximum's bits [P1 paragraph 1; P3 "The fix ..."].
// amax_bits: bits of a non-negative float. With exponent field F (amax = m * 2^(F-127)):
//   floor: e = F - 127 - 2;  ceil: e += 1 when the mantissa exceeds 1.5.
// byte = e + 127 clamped to [0, 254] (F = 0, i.e. zero or subnormal amax, gives byte 0);
// a non-finite amax gives 0xFF.
// ---------------------------------------------------------------------------------------------
template <bool CEIL>
__device__ __forceinline__ uint32_t scale_byte(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;
  int32_t b = (int32_t)(amax_bits >> 23) - 2;
  if (CEIL) b += (amax_bits & 0x7FFFFFu) > 0x400000u ? 1 : 0;
  b = b < 0 ? 0 : b;
  return (uint32_t)b;  // F <= 254 -> b <= 253
}

// 2^-e for a finite scale byte: (254 - byte) << 23 is a normal float for byte <= 253.
__device__ __forceinline__ float inv_scale_from_byte(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// ---------------------------------------------------------------------------------------------
// E2M1 rounding of v = x * 2^-e (already computed in fp32); both saturate at 6 and copy the sign.
// RNE: gfx950's v_cvt_scalef32_pk_fp4_f32 with unit scale rounds to nearest with ties to the
//      even code, as the definition requires.
// SR : round up iff r < f * 2^16 (r the element's 16-bit random field, f the position of |v|
//      between its two grid neighbours). gfx950's stochastic converter
//      (v_cvt_scalef32_sr_pk_fp4_f32) rounds the first value of its pair up iff
//      floor(f * 2^22) + (R >> 10) >= 2^22 for its random word R. With R = (~r << 16) | 0xFFFF
//      that is floor(f * 2^22) > 64 r, while the rule wants f * 2^22 > 64 r, i.e.
//      ceil(f * 2^22) > 64 r. The two agree once f * 2^22 is an integer: the value is first
//      rounded up (in magnitude) to a multiple of 2^-23, ceil(|v| * 2^23) * 2^-23, which is the
//      identity for |v| >= 1 (there the 22 bits below E2M1's mantissa bit are all of f) and
//      turns f * 2^22 into ceil(f * 2^22) below 1 (grid step 1/2); a value just under a grid
//      point that rounds up onto it is then rounded up by the converter for every r, as the
//      rule does. |v| * 2^23 and the products are exact fp32 operations. The converter divides
//      its input by its scale operand, so ceil(|v| * 2^23) goes in with scale 2^23 (checked
//      equal to the unit-scale conversion of the rounded value on 1M random value/word pairs).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t cvt_rne_pack8(const float (&v)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// One stochastic conversion into byte BYTE of acc: the converter writes the codes of its pair
// (value, 0) to that byte, the value's code in the low nibble and the zero's code (0) in the high
// one, and keeps the other three bytes. The compiler's builtin for this instruction does not
// model the kept bytes, so the instruction is written out with acc tied to its destination
// (byte 0 starts a word: whatever the other bytes held is overwritten by the later bytes). A
// VALU read of a register written with a byte select needs one wait state on gfx950, hence the
// s_nop. rw = (~r << 16) | 0xFFFF; the input is the value rounded up to a multiple of 2^-23,
// times 2^23, so the scale operand is 2^23.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <int BYTE>
__device__ __forceinline__ void cvt_sr_fp4_byte(uint32_t& acc, float up, uint32_t rw) {
  const f32x2_t pair = {up, 0.0f};
  const float scale = 8388608.0f;
  if constexpr (BYTE == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3\n\ts_nop 0"
        : "=v"(acc) : "v"(pair), "v"(rw), "s"(scale));
  else if constexpr (BYTE == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]\n\ts_nop 0"
        : "+v"(acc) : "v"(pair), "v"(rw), "s"(scale));
  else if constexpr (BYTE == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]\n\ts_nop 0"
        : "+v"(acc) : "v"(pair), "v"(rw), "s"(scale));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]\n\ts_nop 0"
        : "+v"(acc) : "v"(pair), "v"(rw), "s"(scale));
}

// |v| rounded up to a multiple of 2^-23, times 2^23, with the sign of v
__device__ __forceinline__ float sr_round_up23(float v) {
  return __builtin_copysignf(__builtin_ceilf(fabsf(v) * 8388608.0f), v);
}

// 8 values already rounded up by sr_round_up23 -> 8 codes (value k in nibble k). Even values go
// to bytes 0-3 of one word and odd values to bytes 0-3 of another, each code in the low nibble
// of its byte; the odd word is then shifted into the high nibbles. rw[k] = (~r_k << 16) | 0xFFFF.
__device__ __forceinline__ uint32_t sr_pack8_up(const float (&up)[8], const uint32_t (&rw)[8]) {
  uint32_t ev, od;
  cvt_sr_fp4_byte<0>(ev, up[0], rw[0]);
  cvt_sr_fp4_byte<0>(od, up[1], rw[1]);
  cvt_sr_fp4_byte<1>(ev, up[2], rw[2]);
  cvt_sr_fp4_byte<1>(od, up[3], rw[3]);
  cvt_sr_fp4_byte<2>(ev, up[4], rw[4]);
  cvt_sr_fp4_byte<2>(od, up[5], rw[5]);
  cvt_sr_fp4_byte<3>(ev, up[6], rw[6]);
  cvt_sr_fp4_byte<3>(od, up[7], rw[7]);
  return ev | (od << 4);
}

// 8 scaled values -> 8 codes
__device__ __forceinline__ uint32_t sr_pack8(const float (&v)[8], const uint32_t (&rw)[8]) {
  float up[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) up[k] = sr_round_up23(v[k]);
  return sr_pack8_up(up, rw);
}

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of two 32x32->64 products of
// counter words 0 and 2 with the Philox multipliers, mixed with words 1, 3 and the key; the key
// advances by the Weyl constants between rounds. Returns the 128-bit output.
// ---------------------------------------------------------------------------------------------
// One round: two 32x32->64 products, their high words mixed with words 1, 3 and the key by a
// three-input bit operation (TT = 0x96 is a ^ b ^ c, 0x69 its complement).
template <int TT>
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, TT);
  const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, TT);
  c1 = (uint32_t)p1;
  c3 = (uint32_t)p0;
  c0 = n0;
  c2 = n2;
}

// INV02: return words 0 and 2 complemented (the last round's XOR becomes an XNOR for free).
template <bool INV02 = false>
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 9; ++round) {
    philox_round<0x96>(c0, c1, c2, c3, k0, k1);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  philox_round<INV02 ? 0x69 : 0x96>(c0, c1, c2, c3, k0, k1);
  return make_uint4(c0, c1, c2, c3);
}

// Converter random words of source elements 8g .. 8g+7: rw[k] = (~r_k << 16) | 0xFFFF with r_k
// field k (16 bits) of the Philox output at counter g (the low half of output word k / 2 for
// even k, the high half for odd k).
// The complemented Philox words of chunk g: field k (value k of the chunk) is the half k % 2 of
// word k / 2, complemented.
__device__ __forceinline__ u32x4 sr_words(uint64_t g, uint64_t seed) {
  const uint4 w = philox4x32_10<true>((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, (uint32_t)seed,
                                      (uint32_t)(seed >> 32));
  return u32x4{w.x, ~w.y, w.z, ~w.w};  // words 0 and 2 come complemented
}

// converter word of the field in the low / high half of a complemented word
__device__ __forceinline__ uint32_t sr_word_lo(uint32_t nw) { return (nw << 16) | 0xFFFFu; }
__device__ __forceinline__ uint32_t sr_word_hi(uint32_t nw) { return nw | 0xFFFFu; }

__device__ __forceinline__ void sr_rand8(uint64_t g, uint64_t seed, uint32_t (&rw)[8]) {
  const u32x4 v = sr_words(g, seed);
  const uint32_t nw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rw[2 * i] = sr_word_lo(nw[i]);
    rw[2 * i + 1] = sr_word_hi(nw[i]);
  }
}

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------------------------
// One lane's 8 values of a 1x32 block, the block held by the 4 lanes of a DPP quad (lane q
// holds positions 8q .. 8q+7), in the order the pages give [P1 paragraph 2; P3 "Why FP4 ..."]:
// random signs and the Hadamard transform (HAD), block maximum, scale byte, v = x * 2^-e,
// rounding, packing. g is the chunk's index for the random fields (source element index of
// value 0, divided by 8). Returns the 8 codes (value k in nibble k); sb gets the block's scale
// byte, equal on the 4 lanes. All 4 lanes of the quad must be active.
// ---------------------------------------------------------------------------------------------
template <bool HAD, bool SR, bool CEIL>
__device__ __forceinline__ uint32_t quant_chunk8(float (&w)[8], int q, uint32_t sign_mask,
                                                 uint64_t seed, uint64_t g, uint32_t& sb) {
  if (HAD) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = __uint_as_float(__float_as_uint(w[k]) ^ (((sign_mask >> (8 * q + k)) & 1u) << 31));
    fwht8_inlane(w);
    const uint32_t up8 = (q & 1) ? 0x80000000u : 0u;
    const uint32_t up16 = (q & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = butterfly_xlane<kQuadXor1>(w[k], up8);
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = butterfly_xlane<kQuadXor2>(w[k], up16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, abs_bits(w[k]));
  m = max(m, dpp_u32<kQuadXor1>(m));
  m = max(m, dpp_u32<kQuadXor2>(m));
  sb = scale_byte<CEIL>(m);
  if (sb == 0xFFu) return 0u;
  const float inv = inv_scale_from_byte(sb);
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = w[k] * inv;
  if (SR) {
    uint32_t rw[8];
    sr_rand8(g, seed, rw);
    return sr_pack8(w, rw);
  }
  return cvt_rne_pack8(w);
}

// ---------------------------------------------------------------------------------------------
// A whole 1x32 block in one lane [P1 paragraphs 1-2; P3 "Why FP4 ..."].
// hadamard32_inlane: the 32-point transform, spans 1, 2, 4, 8, 16, each output one IEEE add or
// subtract of the stage's two inputs (the random signs are applied before, by the caller).
// quant_block32: block maximum, scale byte, v = x * 2^-e, rounding, packing (value j in nibble
// j % 8 of word j / 8). g0 is the block's first chunk index for the random fields (source
// element index of value 0, divided by 8). sb gets the scale byte; a block with a non-finite
// maximum gets 0xFF and zero codes.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void hadamard32_inlane(float (&w)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      const float a = w[i], c = w[i + h];
      w[i] = a + c;
      w[i + h] = a - c;
    }
  }
}

// Block maximum of |x| as bits: the unsigned maximum of the raw bits is the largest negative
// value (if any), the signed maximum the largest positive one (if any); with the sign bits
// cleared the larger of the two is the largest magnitude, NaN and infinity included.
__device__ __forceinline__ uint32_t block32_amax_bits(const float (&w)[32]) {
  uint32_t mu = __float_as_uint(w[0]);
  int32_t mi = (int32_t)mu;
#pragma unroll
  for (int j = 1; j < 31; j += 2) {  // one three-input maximum per two values
    mu = max(max(mu, __float_as_uint(w[j])), __float_as_uint(w[j + 1]));
    mi = max(max(mi, (int32_t)__float_as_uint(w[j])), (int32_t)__float_as_uint(w[j + 1]));
  }
  mu = max(mu, __float_as_uint(w[31]));
  mi = max(mi, (int32_t)__float_as_uint(w[31]));
  return max(mu & 0x7FFFFFFFu, (uint32_t)mi & 0x7FFFFFFFu);
}

// quant_block32_with takes the stochastic-rounding words from rw_of(d, rw), which fills the
// converter words of values 8d .. 8d+7.
// FOLD (stochastic rounding of values derived from bf16 input): |x| 2^-e 2^23 is one multiply.
// It equals |v| 2^23 for v = fl32(x 2^-e) except where that product underflows to zero
// (|x 2^-e| <= 2^-150), which the fold would round up on a zero field. A nonzero value derived
// from bf16 by the transform's adds and subtracts is a multiple of 2^-133 (the smallest bf16),
// so with e <= 16 the product is at least 2^-149; e > 16, and e < -104 (where 2^(23 - e)
// overflows), take the two multiplies.
template <bool SR, bool CEIL, bool FOLD = false, class RW>
__device__ __forceinline__ u32x4 quant_block32_with(float (&w)[32], RW&& rw_of, uint32_t& sb) {
  sb = scale_byte<CEIL>(block32_amax_bits(w));
  u32x4 out = {0u, 0u, 0u, 0u};
  if (SR && FOLD && sb - 23u <= 143u - 23u) {  // e = sb - 127 in [-104, 16]
    const float inv23 = __uint_as_float((277u - sb) << 23);  // 2^(23 - e)
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float up[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        up[k] = __builtin_copysignf(__builtin_ceilf(fabsf(w[8 * d + k]) * inv23), w[8 * d + k]);
      uint32_t rw[8];
      rw_of(d, rw);
      o[d] = sr_pack8_up(up, rw);
    }
    out = u32x4{o[0], o[1], o[2], o[3]};
  } else if (sb != 0xFFu) {
    const float inv = inv_scale_from_byte(sb);
#pragma unroll
    for (int j = 0; j < 32; ++j) w[j] = w[j] * inv;
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float (&v8)[8] = *reinterpret_cast<const float(*)[8]>(w + 8 * d);
      if (SR) {
        uint32_t rw[8];
        rw_of(d, rw);
        o[d] = sr_pack8(v8, rw);
      } else {
        o[d] = cvt_rne_pack8(v8);
      }
    }
    out = u32x4{o[0], o[1], o[2], o[3]};
  }
  return out;
}

template <bool SR, bool CEIL, bool FOLD = false>
__device__ __forceinline__ u32x4 quant_block32(float (&w)[32], uint64_t seed, uint64_t g0,
                                               uint32_t& sb) {
  return quant_block32_with<SR, CEIL, FOLD>(
      w, [&](int d, uint32_t (&rw)[8]) { sr_rand8(g0 + d, seed, rw); }, sb);
}

// ---------------------------------------------------------------------------------------------
// in-lane transpose of an 8x8 matrix of nibbles: R[j] nibble k -> R[k] nibble j
// (swap 4x4 quadrants, then 2x2 sub-blocks, then single nibbles)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void transpose_nibbles8x8(uint32_t (&R)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // quadrants: bytes {a0,a1,b0,b1} and {a2,a3,b2,b3}
    const uint32_t a = R[j], b = R[j + 4];
    R[j] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    R[j + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int base = 0; base < 8; base += 4) {  // 2x2 blocks: bytes {a0,b0,a2,b2} and {a1,b1,a3,b3}
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t a = R[base + j], b = R[base + j + 2];
      R[base + j] = __builtin_amdgcn_perm(b, a, 0x06020400u);
      R[base + j + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {  // single nibbles
    const uint32_t a = R[j], b = R[j + 1];
    R[j] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    R[j + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// ---------------------------------------------------------------------------------------------
// MXFP8 [P3 "The fix, and its supporting cast": queries and keys in MXFP8]: the E8M0 scale of
// the FP4 path with 8-bit elements, E4M3 (FMT 0: bias 7, 3 mantissa bits, largest 448, no
// infinity) or E5M2 (FMT 1: bias 15, 2 mantissa bits, largest 57344), the OCP MX encodings.
// ---------------------------------------------------------------------------------------------
template <int FMT>
struct Fp8 {
  static constexpr int kMant = FMT == 0 ? 3 : 2;
  static constexpr int kBias = FMT == 0 ? 7 : 15;
  static constexpr int kEmax = FMT == 0 ? 8 : 15;            // exponent of the largest value
  static constexpr uint32_t kLargest = FMT == 0 ? 0x43E00000u : 0x47600000u;  // 448, 57344
  static constexpr uint32_t kTop = FMT == 0 ? 0x7Eu : 0x7Bu;  // its code
  static constexpr int kMinNormal = 1 - kBias;                 // exponent of the least normal
};

// scale byte from the block maximum's bits: floor e = F - 127 - emax; ceil adds one when the
// mantissa exceeds 1.75 (the largest value is 1.75 * 2^emax); clamped at 0; non-finite -> 0xFF
template <bool CEIL, int FMT>
__device__ __forceinline__ uint32_t scale_byte_fp8(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;
  int32_t b = (int32_t)(amax_bits >> 23) - Fp8<FMT>::kEmax;
  if (CEIL) b += (amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0;
  return (uint32_t)(b < 0 ? 0 : b);
}

// Rounding to the element format, on gfx950's converters (unit scale). Values are first
// clamped to +-largest (saturation; the converters themselves are not used beyond it).
// Nearest-even: v_cvt_scalef32_pk_fp8_f32 / _bf8_f32, two values per instruction (the first in
// the low byte). Stochastic: v_cvt_scalef32_sr_fp8_f32 / _bf8_f32 rounds the magnitude up iff
// floor(f * 2^d) + (R >> (32 - d)) >= 2^d, where f is the position of |v| between its two
// neighbours and d = 23 - mantissa bits; with R = (~r << 16) | 0xFFFF that is floor(f * 2^d) >
// 2^(d - 16) r, the rule r < f * 2^16 once f * 2^d is an integer. In the normal range it is
// (the d dropped significand bits). Below the least normal the step stays 2^(min - mant), so
// |v| is first rounded up to a multiple of 2^(min - mant - d) (2^-29 for E4M3, 2^-37 grid
// refined to 2^-36 for E5M2); the thresholds lo + r 2^(min - mant - 16) lie on that grid, so
// the rounding up moves no value across one. Both were checked bit for bit against the
// integer definition over every bf16 value at five scales, random fp32 values, and random and
// extreme fields.
typedef short v2s_fp8 __attribute__((ext_vector_type(2)));

template <int FMT>
__device__ __forceinline__ float fp8_clamp(float v) {
  const float lim = __uint_as_float(Fp8<FMT>::kLargest);
  return __builtin_amdgcn_fmed3f(v, -lim, lim);
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_rne_pair(float a, float b) {
  v2s_fp8 o = {0, 0};
  if (FMT == 0) o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, fp8_clamp<FMT>(a), fp8_clamp<FMT>(b), 1.0f, false);
  else o = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, fp8_clamp<FMT>(a), fp8_clamp<FMT>(b), 1.0f, false);
  return (uint32_t)(uint16_t)o.x;
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_sr_byte(float v, uint32_t r) {
  v = fp8_clamp<FMT>(v);
  const float a = fabsf(v);
  constexpr float kMinNormal = FMT == 0 ? 0x1p-6f : 0x1p-14f;
  constexpr float kUp = FMT == 0 ? 0x1p29f : 0x1p36f;
  constexpr float kDown = FMT == 0 ? 0x1p-29f : 0x1p-36f;
  const float up = a < kMinNormal ? __builtin_ceilf(a * kUp) * kDown : a;
  const float vv = __builtin_copysignf(up, v);
  const uint32_t R = (~r << 16) | 0xFFFFu;
  const uint32_t w = FMT == 0 ? __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0u, vv, R, 1.0f, 0)
                              : __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(0u, vv, R, 1.0f, 0);
  return w & 0xFFu;
}

// raw 16-bit random fields of source elements 8g .. 8g+7 (field k: the low half of Philox
// output word k / 2 for even k, the high half for odd k)
__device__ __forceinline__ void sr_fields8(uint64_t g, uint64_t seed, uint32_t (&r)[8]) {
  const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, (uint32_t)seed,
                                (uint32_t)(seed >> 32));
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = wd[i] & 0xFFFFu;
    r[2 * i + 1] = wd[i] >> 16;
  }
}

// 8 scaled values -> 8 code bytes (value k in byte k of the pair of words)
template <int FMT, bool SR>
__device__ __forceinline__ uint2 fp8_pack8(const float (&v)[8], const uint32_t (&r)[8]) {
  uint32_t w[2] = {0u, 0u};
  if (SR) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k >> 2] |= fp8_sr_byte<FMT>(v[k], r[k]) << (8 * (k & 3));
  } else {
#pragma unroll
    for (int k = 0; k < 8; k += 2) w[k >> 2] |= fp8_rne_pair<FMT>(v[k], v[k + 1]) << (8 * (k & 3));
  }
  return make_uint2(w[0], w[1]);
}

// The MXFP8 counterpart of quant_chunk8: one lane's 8 values of a 1x32 block held by a quad;
// returns the 8 code bytes, sb gets the block's scale byte.
template <int FMT, bool HAD, bool SR, bool CEIL>
__device__ __forceinline__ uint2 quant_chunk8_fp8(float (&w)[8], int q, uint32_t sign_mask,
                                                  uint64_t seed, uint64_t g, uint32_t& sb) {
  if (HAD) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = __uint_as_float(__float_as_uint(w[k]) ^ (((sign_mask >> (8 * q + k)) & 1u) << 31));
    fwht8_inlane(w);
    const uint32_t up8 = (q & 1) ? 0x80000000u : 0u;
    const uint32_t up16 = (q & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = butterfly_xlane<kQuadXor1>(w[k], up8);
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = butterfly_xlane<kQuadXor2>(w[k], up16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, abs_bits(w[k]));
  m = max(m, dpp_u32<kQuadXor1>(m));
  m = max(m, dpp_u32<kQuadXor2>(m));
  sb = scale_byte_fp8<CEIL, FMT>(m);
  if (sb == 0xFFu) return make_uint2(0u, 0u);
  const float inv = inv_scale_from_byte(sb);
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = w[k] * inv;
  uint32_t r[8];
  if (SR) sr_fields8(g, seed, r);
  return fp8_pack8<FMT, SR>(w, r);
}

}  // namespace mxd
