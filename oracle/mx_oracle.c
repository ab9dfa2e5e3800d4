/*
 * mx_oracle.c — TEST INFRASTRUCTURE ONLY. A plain, slow, scalar CPU reference of the MXFP4
 * block-scaled Hadamard-32 quantizer. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 *
 * It shares no code, header or table with the GPU library. Build (see build_oracle.py):
 *     gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
 * fp32 arithmetic is IEEE single with round-to-nearest-even and gradual underflow (SSE).
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Block-Scaled MXFP4 With Stochastic Hadamard Rounding Matches BF16 Convergence on 70B
 *       Pre-Training", paragraphs 1-2.
 *  [P2] "Pretraining large language models with MXFP4", abstract.
 *  [P3] "Stable FP4 Training via Transposition-Invariant Block Quantization", sections
 *       "Why FP4 training is the current frontier", "The fix, and its supporting cast".
 *  [P4] "Training LLMs with MXFP4", abstract.
 *
 * Readings where the pages are silent (each one is a stated choice, not a page fact):
 *  - E2M1 magnitudes follow from 1 sign, 2 exponent (bias 1) and 1 mantissa bit with a
 *    subnormal at exponent 0 and no inf/nan: {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *  - Floor scale: e = floor(log2 amax) - 2; ceil scale: least e with amax <= 6 * 2^e.
 *    amax = 0 -> e = -127; e clamped to [-127, 127]; byte = e + 127; non-finite amax ->
 *    byte 0xFF and all codes 0.
 *  - Hadamard: unnormalised, natural (Sylvester) order, butterflies of span 1,2,4,8,16 in fp32.
 *  - RNE ties go to the even code; |v| >= 6 saturates.
 *  - SR: round up iff r16 < frac * 65536, r16 from Philox4x32-10 field (i & 7) of counter i >> 3.
 *  - MXFP8 (E4M3 / E5M2 elements): OCP MX FP8 element encodings; floor scale e =
 *    floor(log2 amax) - emax (8 or 15), ceil scale the least e with amax <= largest * 2^e;
 *    |v| >= largest saturates; rounding and the random fields as for E2M1.
 *
 * Parity pins: see the tests under tests/ (exhaustive grid/scale checks, SR enumeration,
 * dense Hadamard matrix, transposition invariance). Philox4x32-10 is pinned against rocRAND's
 * header-only engine, built for the host CPU from the ROCm headers; on a host without those
 * headers that one pin is skipped.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* Options: the oracle's own copy of the quantizer knobs (not shared with the library).       */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t scale_rule; /* 0 = floor (OCP), 1 = ceil (truncation-free) */
  int32_t round;      /* 0 = nearest-even, 1 = stochastic */
  int32_t hadamard;   /* 0/1 */
  uint32_t sign_mask; /* bit j negates block position j before the transform */
  uint64_t seed;      /* Philox key */
} orc_opts;

/* ------------------------------------------------------------------------------------------ */
/* E2M1 element format [P3 "Why FP4 ...": 1 sign, 2 exponent, 1 mantissa bit].               */
/* The magnitude of code m (0..7) is derived from its bit fields rather than tabulated:       */
/*   exponent field E = m >> 1, mantissa bit M = m & 1, bias 1:                               */
/*   E == 0 -> subnormal M * 0.5 ; else (1 + M/2) * 2^(E-1).                                  */
/* ------------------------------------------------------------------------------------------ */
float orc_e2m1_magnitude(int m) {
  int E = (m >> 1) & 3, M = m & 1;
  if (E == 0) return 0.5f * (float)M;
  return (1.0f + 0.5f * (float)M) * ldexpf(1.0f, E - 1);
}

float orc_e2m1_decode(int code) {
  float mag = orc_e2m1_magnitude(code & 7);
  return (code & 8) ? -mag : mag;
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy as 1, 2, 3",  */
/* SC'11). A round multiplies counter words 0 and 2 by the two Philox constants into 64-bit   */
/* products and mixes the halves with the other counter words and the key; the key is bumped  */
/* by the two Weyl constants between rounds.                                                  */
/* ------------------------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t MUL0 = 0xD2511F53u, MUL1 = 0xCD9E8D57u;
  const uint32_t WEYL0 = 0x9E3779B9u, WEYL1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += WEYL0;
      k1 += WEYL1;
    }
    uint64_t p0 = (uint64_t)MUL0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)MUL1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16-bit random field of source element i: counter = i / 8, field i % 8 of the 128-bit
 * output (word (i % 8) / 2, low half for even i). */
uint32_t orc_sr_field(uint64_t seed, uint64_t i) {
  uint64_t group = i >> 3;
  uint32_t ctr[4] = {(uint32_t)group, (uint32_t)(group >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  uint32_t word = out[(i & 7) >> 1];
  return (i & 1) ? (word >> 16) : (word & 0xFFFFu);
}

/* ------------------------------------------------------------------------------------------ */
/* 32-point Walsh-Hadamard transform, unnormalised, natural order [P1 paragraph 2: block-     */
/* diagonal, O(d log d)]. Stage with span h pairs positions i and i + h (bit h of i clear).   */
/* ------------------------------------------------------------------------------------------ */
void orc_fwht32(float x[32]) {
  for (int h = 1; h < 32; h <<= 1) {
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* E8M0 scale exponent from the block maximum [P1 paragraph 1; P3 "Why FP4 ..." and          */
/* "The fix ..."]. Returns the unclamped-then-clamped e in [-127, 127]; amax must be finite.  */
/* ------------------------------------------------------------------------------------------ */
int orc_scale_exponent(float amax, int scale_rule) {
  if (amax == 0.0f) return -127;
  int E2;
  float frac = frexpf(amax, &E2); /* amax = frac * 2^E2, frac in [0.5, 1): exact */
  float m = 2.0f * frac;          /* amax = m * 2^(E2-1), m in [1, 2) */
  int E = E2 - 1;
  int e;
  if (scale_rule == 0) {
    e = E - 2; /* floor(log2 amax) - emax(E2M1) */
  } else {
    /* least e with amax <= 6 * 2^e = 1.5 * 2^(e+2) */
    e = (m > 1.5f) ? (E - 1) : (E - 2);
  }
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* ------------------------------------------------------------------------------------------ */
/* E2M1 rounding of a scaled value v [P3 "The fix ...": nearest or stochastic].               */
/* ------------------------------------------------------------------------------------------ */
int orc_e2m1_encode(float v, int round_mode, uint32_t r16) {
  int sign = signbit(v) ? 1 : 0;
  float a = fabsf(v);
  int idx;
  if (a >= 6.0f) {
    idx = 7; /* saturate: the largest magnitude */
  } else {
    int k = 0; /* largest grid index with magnitude <= a */
    while (k < 7 && orc_e2m1_magnitude(k + 1) <= a) ++k;
    float lo = orc_e2m1_magnitude(k);
    float hi = orc_e2m1_magnitude(k + 1);
    float frac = (a - lo) / (hi - lo); /* exact: Sterbenz, power-of-two step */
    if (round_mode == 0) {
      if (frac > 0.5f) idx = k + 1;
      else if (frac < 0.5f) idx = k;
      else idx = (k % 2 == 0) ? k : k + 1; /* tie: the even code */
    } else {
      idx = ((float)r16 < frac * 65536.0f) ? k + 1 : k;
    }
  }
  return (sign << 3) | idx;
}

static float widen(const void* x, int dtype, int64_t offset) {
  if (dtype == 1) {
    uint32_t bits = (uint32_t)((const uint16_t*)x)[offset] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
  }
  return ((const float*)x)[offset];
}

static void put_nibble(uint8_t* bytes, int64_t elem, int code) {
  uint8_t* p = bytes + (elem >> 1);
  if (elem & 1) *p = (uint8_t)((*p & 0x0F) | (code << 4));
  else *p = (uint8_t)((*p & 0xF0) | code);
}

/* Quantize one block of n values (n = 32 or 1024). vals is modified in place (signs and
 * transform). idx[j] is the source row-major index of value j (for the SR field). Writes
 * the scale byte and codes[j]. */
static uint8_t quantize_block(float* vals, const uint64_t* idx, int n, const orc_opts* o,
                              int* codes) {
  if (o->hadamard) { /* n == 32 */
    for (int j = 0; j < 32; ++j)
      if ((o->sign_mask >> j) & 1u) vals[j] = -vals[j];
    orc_fwht32(vals);
  }
  float amax = 0.0f;
  int finite = 1;
  for (int j = 0; j < n; ++j) {
    float a = fabsf(vals[j]);
    if (!isfinite(a)) finite = 0;
    if (a > amax) amax = a;
  }
  if (!finite) {
    for (int j = 0; j < n; ++j) codes[j] = 0;
    return 0xFF;
  }
  int e = orc_scale_exponent(amax, o->scale_rule);
  float inv_scale = ldexpf(1.0f, -e); /* 2^-e, exact (2^-127 is an fp32 subnormal) */
  for (int j = 0; j < n; ++j) {
    float v = vals[j] * inv_scale;
    uint32_t r16 = o->round ? orc_sr_field(o->seed, idx[j]) : 0u;
    codes[j] = orc_e2m1_encode(v, o->round, r16);
  }
  return (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------------------------------ */
/* 1x32 quantize [P1 paragraph 1; P3 "Why FP4 ..."]. Processes rows [row_begin, row_end)     */
/* (for axis 0 both must be multiples of 32) into full-size outputs.                          */
/*   axis 1: codes[rows][cols/2], scales[rows][cols/32]                                       */
/*   axis 0: codes[cols][rows/2], scales[cols][rows/32]  (layout of the transpose)            */
/* ------------------------------------------------------------------------------------------ */
int orc_quantize_1d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                    const orc_opts* o, uint8_t* codes, uint8_t* scales, int64_t row_begin,
                    int64_t row_end) {
  float vals[32];
  uint64_t idx[32];
  int cds[32];
  if (axis == 1) {
    for (int64_t r = row_begin; r < row_end; ++r) {
      for (int64_t b = 0; b < cols / 32; ++b) {
        for (int j = 0; j < 32; ++j) {
          int64_t c = b * 32 + j;
          vals[j] = widen(x, dtype, r * ld + c);
          idx[j] = (uint64_t)(r * cols + c);
        }
        scales[r * (cols / 32) + b] = quantize_block(vals, idx, 32, o, cds);
        for (int j = 0; j < 32; ++j) put_nibble(codes, r * cols + b * 32 + j, cds[j]);
      }
    }
  } else {
    for (int64_t b = row_begin / 32; b < row_end / 32; ++b) {
      for (int64_t c = 0; c < cols; ++c) {
        for (int j = 0; j < 32; ++j) {
          int64_t r = b * 32 + j;
          vals[j] = widen(x, dtype, r * ld + c);
          idx[j] = (uint64_t)(r * cols + c);
        }
        scales[c * (rows / 32) + b] = quantize_block(vals, idx, 32, o, cds);
        for (int j = 0; j < 32; ++j) put_nibble(codes, c * rows + b * 32 + j, cds[j]);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* 32x32 quantize [P3 "The fix ...": block (i,j) of X is block (j,i) of X^T]. One scale per  */
/* tile from the tile's maximum; each element is rounded once and written to both layouts.   */
/* Rows [row_begin, row_end), multiples of 32.                                                */
/* ------------------------------------------------------------------------------------------ */
int orc_quantize_2d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                    const orc_opts* o, uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                    uint8_t* scales_t, int64_t row_begin, int64_t row_end) {
  float* vals = (float*)malloc(1024 * sizeof(float));
  uint64_t* idx = (uint64_t*)malloc(1024 * sizeof(uint64_t));
  int* cds = (int*)malloc(1024 * sizeof(int));
  orc_opts plain = *o;
  plain.hadamard = 0;
  for (int64_t br = row_begin / 32; br < row_end / 32; ++br) {
    for (int64_t bc = 0; bc < cols / 32; ++bc) {
      for (int i = 0; i < 32; ++i)
        for (int j = 0; j < 32; ++j) {
          int64_t r = br * 32 + i, c = bc * 32 + j;
          vals[i * 32 + j] = widen(x, dtype, r * ld + c);
          idx[i * 32 + j] = (uint64_t)(r * cols + c);
        }
      uint8_t s = quantize_block(vals, idx, 1024, &plain, cds);
      scales[br * (cols / 32) + bc] = s;
      if (scales_t) scales_t[bc * (rows / 32) + br] = s;
      for (int i = 0; i < 32; ++i)
        for (int j = 0; j < 32; ++j) {
          int64_t r = br * 32 + i, c = bc * 32 + j;
          put_nibble(codes, r * cols + c, cds[i * 32 + j]);
          if (codes_t) put_nibble(codes_t, c * rows + r, cds[i * 32 + j]);
        }
    }
  }
  free(vals);
  free(idx);
  free(cds);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* BxB tiles, B in {8, 32, 64} [P3 "The fix ...": Table 4 compares 8x8, 32x32 and 64x64       */
/* blocks]: the 32x32 rule with another tile edge. One scale per tile from the tile maximum;   */
/* codes[rows][cols/2], scales[rows/B][cols/B], and the transposed copies codes_t[cols][rows/2],*/
/* scales_t[cols/B][rows/B] (nullable). Rows [row_begin, row_end), multiples of B.             */
/* ------------------------------------------------------------------------------------------ */
int orc_quantize_2d_block(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                          int B, const orc_opts* o, uint8_t* codes, uint8_t* scales,
                          uint8_t* codes_t, uint8_t* scales_t, int64_t row_begin,
                          int64_t row_end) {
  const int n = B * B;
  float* vals = (float*)malloc((size_t)n * sizeof(float));
  uint64_t* idx = (uint64_t*)malloc((size_t)n * sizeof(uint64_t));
  int* cds = (int*)malloc((size_t)n * sizeof(int));
  orc_opts plain = *o;
  plain.hadamard = 0;
  for (int64_t br = row_begin / B; br < row_end / B; ++br) {
    for (int64_t bc = 0; bc < cols / B; ++bc) {
      for (int i = 0; i < B; ++i)
        for (int j = 0; j < B; ++j) {
          int64_t r = br * B + i, c = bc * B + j;
          vals[i * B + j] = widen(x, dtype, r * ld + c);
          idx[i * B + j] = (uint64_t)(r * cols + c);
        }
      uint8_t s = quantize_block(vals, idx, n, &plain, cds);
      scales[br * (cols / B) + bc] = s;
      if (scales_t) scales_t[bc * (rows / B) + br] = s;
      for (int i = 0; i < B; ++i)
        for (int j = 0; j < B; ++j) {
          int64_t r = br * B + i, c = bc * B + j;
          put_nibble(codes, r * cols + c, cds[i * B + j]);
          if (codes_t) put_nibble(codes_t, c * rows + r, cds[i * B + j]);
        }
    }
  }
  free(vals);
  free(idx);
  free(cds);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Dequantize: value = E2M1(code) * 2^(byte - 127) in fp32 [P3 "Why FP4 ...": P * S].        */
/* Optional inverse rotation per 32-block along a row: (1/32) * D * H.                        */
/* ------------------------------------------------------------------------------------------ */
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                   int block_rows, int inv_hadamard, uint32_t sign_mask, float* out) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      int64_t e = r * cols + c;
      int code = (codes[e >> 1] >> ((e & 1) * 4)) & 0xF;
      uint8_t s = scales[(r / block_rows) * (cols / 32) + c / 32];
      float v;
      if (s == 0xFF) v = NAN;
      else v = orc_e2m1_decode(code) * ldexpf(1.0f, (int)s - 127);
      out[e] = v;
    }
    if (inv_hadamard) {
      for (int64_t b = 0; b < cols / 32; ++b) {
        float* y = out + r * cols + b * 32;
        orc_fwht32(y);
        for (int j = 0; j < 32; ++j) {
          y[j] = y[j] * 0.03125f;
          if ((sign_mask >> j) & 1u) y[j] = -y[j];
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* MXFP8 [P3 "The fix, and its supporting cast": queries and keys are quantized in MXFP8]:    */
/* the same E8M0 scale per 32 consecutive values, with 8-bit E4M3 (fmt 0) or E5M2 (fmt 1)     */
/* elements. The pages fix neither encoding; both are the OCP MX FP8 element types (reading): */
/*   E4M3: 4 exponent bits (bias 7), 3 mantissa bits; exponent 15 with mantissa 7 is NaN, no  */
/*         infinity, so the largest magnitude is 1.75 * 2^8 = 448.                            */
/*   E5M2: 5 exponent bits (bias 15), 2 mantissa bits; exponent 31 is inf / NaN, so the        */
/*         largest magnitude is 1.75 * 2^15 = 57344.                                          */
/* Exponent field 0 is subnormal: M * 2^(1 - bias - mbits). Codes 0..max_code of the 7-bit   */
/* magnitude are finite and increase with the code.                                          */
/* ------------------------------------------------------------------------------------------ */
static void fp8_fields(int fmt, int* ebits, int* mbits, int* bias, int* max_code) {
  if (fmt == 0) {
    *ebits = 4; *mbits = 3; *bias = 7; *max_code = 0x7E;
  } else {
    *ebits = 5; *mbits = 2; *bias = 15; *max_code = 0x7B;
  }
}

/* magnitude of 7-bit code m; inf or NaN for the non-finite codes */
double orc_fp8_magnitude(int m, int fmt) {
  int ebits, mbits, bias, max_code;
  fp8_fields(fmt, &ebits, &mbits, &bias, &max_code);
  m &= 0x7F;
  int E = m >> mbits, M = m & ((1 << mbits) - 1);
  if (m > max_code) {
    if (fmt == 1 && M == 0) return INFINITY;
    return NAN;
  }
  if (E == 0) return ldexp((double)M, 1 - bias - mbits);
  return ldexp(1.0 + ldexp((double)M, -mbits), E - bias);
}

double orc_fp8_decode(int code, int fmt) {
  double mag = orc_fp8_magnitude(code & 0x7F, fmt);
  return (code & 0x80) ? -mag : mag;
}

/* Scale exponent: floor (OCP) e = floor(log2 amax) - emax with emax the exponent of the      */
/* largest magnitude (8 or 15); ceil: the least e with amax <= largest * 2^e, found by        */
/* stepping up from the floor value (exact in double). Clamped to [-127, 127]; amax = 0 ->    */
/* -127. amax must be finite.                                                                 */
int orc_fp8_scale_exponent(float amax, int scale_rule, int fmt) {
  int ebits, mbits, bias, max_code;
  fp8_fields(fmt, &ebits, &mbits, &bias, &max_code);
  if (amax == 0.0f) return -127;
  const double largest = orc_fp8_magnitude(max_code, fmt);
  const int emax = (max_code >> mbits) - bias;
  int E2;
  frexpf(amax, &E2); /* amax in [2^(E2-1), 2^E2) */
  int e = (E2 - 1) - emax;
  if (scale_rule == 1)
    while (ldexp(largest, e) < (double)amax) ++e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* Rounding of a scaled value v to the format: |v| >= largest saturates; otherwise lo <= |v| < */
/* hi are the neighbouring magnitudes, frac = (|v| - lo) / (hi - lo) is exact in fp32 (lo >=   */
/* |v|/2 or a multiple of the subnormal step; hi - lo is a power of two). Nearest with ties to */
/* the even code, or stochastic: up iff r16 < frac * 65536. The sign is copied (bit 7).       */
int orc_fp8_encode(float v, int fmt, int round_mode, uint32_t r16) {
  int ebits, mbits, bias, max_code;
  fp8_fields(fmt, &ebits, &mbits, &bias, &max_code);
  int sign = signbit(v) ? 1 : 0;
  float a = fabsf(v);
  int idx;
  if ((double)a >= orc_fp8_magnitude(max_code, fmt)) {
    idx = max_code;
  } else {
    /* largest code k with magnitude(k) <= a, by bisection over the increasing magnitudes */
    int k = 0, top = max_code; /* invariant: magnitude(k) <= a < magnitude(top) */
    while (top - k > 1) {
      int mid = (k + top) / 2;
      if (orc_fp8_magnitude(mid, fmt) <= (double)a) k = mid;
      else top = mid;
    }
    float lo = (float)orc_fp8_magnitude(k, fmt);
    float hi = (float)orc_fp8_magnitude(k + 1, fmt);
    float frac = (a - lo) / (hi - lo);
    if (round_mode == 0) {
      if (frac > 0.5f) idx = k + 1;
      else if (frac < 0.5f) idx = k;
      else idx = (k % 2 == 0) ? k : k + 1;
    } else {
      idx = ((float)r16 < frac * 65536.0f) ? k + 1 : k;
    }
  }
  return (sign << 7) | idx;
}

/* One 32-value block in the order of the FP4 path: signs and transform (optional), block     */
/* maximum, scale, v = x * 2^-e, rounding. Non-finite block: byte 0xFF, codes 0.              */
static uint8_t quantize_block_fp8(float* vals, const uint64_t* idx, int fmt, const orc_opts* o,
                                  int* codes) {
  if (o->hadamard) {
    for (int j = 0; j < 32; ++j)
      if ((o->sign_mask >> j) & 1u) vals[j] = -vals[j];
    orc_fwht32(vals);
  }
  float amax = 0.0f;
  int finite = 1;
  for (int j = 0; j < 32; ++j) {
    float a = fabsf(vals[j]);
    if (!isfinite(a)) finite = 0;
    if (a > amax) amax = a;
  }
  if (!finite) {
    for (int j = 0; j < 32; ++j) codes[j] = 0;
    return 0xFF;
  }
  int e = orc_fp8_scale_exponent(amax, o->scale_rule, fmt);
  float inv_scale = ldexpf(1.0f, -e);
  for (int j = 0; j < 32; ++j) {
    float v = vals[j] * inv_scale;
    uint32_t r16 = o->round ? orc_sr_field(o->seed, idx[j]) : 0u;
    codes[j] = orc_fp8_encode(v, fmt, o->round, r16);
  }
  return (uint8_t)(e + 127);
}

/* 1x32 MXFP8 quantize, one code byte per element, rows [row_begin, row_end):                */
/*   axis 1: codes[rows][cols], scales[rows][cols/32]                                         */
/*   axis 0: codes[cols][rows], scales[cols][rows/32]  (layout of the transpose)              */
int orc_quantize_fp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                     int fmt, const orc_opts* o, uint8_t* codes, uint8_t* scales,
                     int64_t row_begin, int64_t row_end) {
  float vals[32];
  uint64_t idx[32];
  int cds[32];
  if (axis == 1) {
    for (int64_t r = row_begin; r < row_end; ++r)
      for (int64_t b = 0; b < cols / 32; ++b) {
        for (int j = 0; j < 32; ++j) {
          int64_t c = b * 32 + j;
          vals[j] = widen(x, dtype, r * ld + c);
          idx[j] = (uint64_t)(r * cols + c);
        }
        scales[r * (cols / 32) + b] = quantize_block_fp8(vals, idx, fmt, o, cds);
        for (int j = 0; j < 32; ++j) codes[r * cols + b * 32 + j] = (uint8_t)cds[j];
      }
  } else {
    for (int64_t b = row_begin / 32; b < row_end / 32; ++b)
      for (int64_t c = 0; c < cols; ++c) {
        for (int j = 0; j < 32; ++j) {
          int64_t r = b * 32 + j;
          vals[j] = widen(x, dtype, r * ld + c);
          idx[j] = (uint64_t)(r * cols + c);
        }
        scales[c * (rows / 32) + b] = quantize_block_fp8(vals, idx, fmt, o, cds);
        for (int j = 0; j < 32; ++j) codes[c * rows + b * 32 + j] = (uint8_t)cds[j];
      }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Threaded driver for timing the oracle on many cores: splits the row range of a 1x32 or     */
/* 32x32 quantize into nthreads contiguous pieces (multiples of 32 rows). Each piece runs     */
/* the same scalar code above; outputs do not overlap.                                        */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
  const void* x; int dtype; int64_t rows, cols, ld; int axis; int two_d; const orc_opts* o;
  uint8_t *codes, *scales, *codes_t, *scales_t; int64_t r0, r1;
} orc_job;

static void* run_job(void* arg) {
  orc_job* j = (orc_job*)arg;
  if (j->two_d)
    orc_quantize_2d(j->x, j->dtype, j->rows, j->cols, j->ld, j->o, j->codes, j->scales,
                    j->codes_t, j->scales_t, j->r0, j->r1);
  else
    orc_quantize_1d(j->x, j->dtype, j->rows, j->cols, j->ld, j->axis, j->o, j->codes,
                    j->scales, j->r0, j->r1);
  return NULL;
}

int orc_quantize_threaded(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                          int axis, int two_d, const orc_opts* o, uint8_t* codes,
                          uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                          int64_t row_begin, int64_t row_end, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  int64_t nblk = (row_end - row_begin) / 32; /* row ranges are split in 32-row units */
  if (nblk < 1 || nthreads == 1) {
    orc_job j = {x, dtype, rows, cols, ld, axis, two_d, o, codes, scales, codes_t, scales_t,
                 row_begin, row_end};
    run_job(&j);
    return 0;
  }
  if (nthreads > nblk) nthreads = (int)nblk;
  orc_job jobs[256];
  pthread_t th[256];
  int64_t start = row_begin;
  for (int t = 0; t < nthreads; ++t) {
    int64_t count = nblk / nthreads + (t < nblk % nthreads ? 1 : 0);
    int64_t stop = start + count * 32;
    if (t == nthreads - 1) stop = row_end;
    orc_job j = {x, dtype, rows, cols, ld, axis, two_d, o, codes, scales, codes_t, scales_t,
                 start, stop};
    jobs[t] = j;
    start = stop;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}
