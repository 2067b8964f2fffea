/*
 * mxq_oracle.c -- plain, slow, scalar CPU oracle for block-scaled microscaling
 * quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the bench may build, load or call this file.  The GPU
 * library shares no code, header, table or helper with it.
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (x86-64 SSE arithmetic: binary32 ops are IEEE round-to-nearest-even with
 * subnormals kept).  Every "RN" below is one such binary32 operation.
 *
 * Sources, cited by page title and section:
 *  [mxfp4 page]  "nemo_automodel.components.quantization.mxfp4":
 *                quantize_mxfp4, dequantize_mxfp4, Data (_FP4_E2M1_TABLE,
 *                _FP4_E2M1_MIDPOINTS, _FP4_BYTE_TABLE, MXFP4_BLOCK_SIZE).
 *  [nvfp4 page]  "nemo_automodel.components.quantization.nvfp4":
 *                module introduction, quantize_nvfp4, quantize_nvfp4_modelopt,
 *                dequantize_nvfp4, _check_last_dim, Data (E2M1_MAX, E4M3_MAX,
 *                E4M3_MIN_SUBNORMAL, NVFP4_BLOCK_SIZE).
 *  [cache page]  "nemo_automodel.components.models.deepseek_v41.quantization":
 *                quantize_cache, _power_of_two_ceiling, _CacheQuantization.
 *  [modelopt]    Model-Optimizer tensor_quantizer.py: TensorQuantizer.forward
 *                (inputs upcast to float before quantizing; blocks padded with
 *                zeros), _FP8_E4M3_MIN_POSITIVE (scale clamp),
 *                TensorQuantizer._real_quantize (the MX branch and its MXFP8
 *                case), _clamp_scale, _amax_to_scale,
 *                StaticBlockScaleQuantizer._block_scale_from_amax and
 *                StaticBlockScaleQuantizer._fake_quantize.
 *  [longlive]    LongLive utils/quant.py: dequantize_kv_cache, k_smooth,
 *                quantize_kv.
 *
 * Readings where the pages are silent, ambiguous or cut off:
 *  R1 midpoint ties go to the smaller magnitude (a count of midpoints strictly
 *     below |q|, i.e. the lower bucket of the midpoint table);
 *  R2 the sign nibble is the sign bit of the input, also when |q| rounds to 0;
 *  R3 floor(log2(amax)) is exact (taken from the binary exponent);
 *  R4 an MXFP4 scale below 2^-127 is stored as byte 0 and the block is
 *     quantized with that stored scale; amax = 0 gives byte 0;
 *  R5 NVFP4 arithmetic is binary32, evaluated left to right as the formula is
 *     written: g = A / 2688, u = (a / 6) / g, den = sigma * g, q = x / den;
 *  R6 NVFP4 block scales are clamped to [2^-9, 448] before the e4m3 cast
 *     (maxNum: a NaN ratio takes the lower bound);
 *  R7 an NVFP4 "row" is one index of the flattened leading dims of a
 *     contiguous [..., K] tensor (one row scale per row of the packed output);
 *  R8 a given global scale is either one value per row or one value for all
 *     rows;
 *  R9 cache scales: fp8 and mxfp4 use the power-of-two ceiling of
 *     amax / elem_max (elem_max 448 or 6), floored at the smallest normal
 *     binary32; nvfp4 uses a single e4m3 scale e4m3(clamp(amax / 6));
 *  R10 a partial last cache group behaves as if zero-padded;
 *  R11 the fp8 cache keeps the sign of zero; e2m1 codes decode through the
 *     table, whose index 8 holds +0.0;
 *  R12 NaN and infinite input elements are outside the contract: the pages
 *     define nothing for them, and what the formulas below give for them is
 *     neither specified nor tested (NaN quotients that finite inputs produce,
 *     such as 0 / 0 under a zero row scale, are covered by R1);
 *  R13 float16 inputs and outputs use the same binary32 arithmetic, with one
 *     final round-to-nearest-even into float16;
 *  R14 e4m3 encodes saturate at 448.
 *  R15 MXFP8 ([modelopt] _real_quantize, MX branch with e4m3 elements and
 *     block 32): the pages print the dispatch but not the MXFP8 arithmetic.
 *     The block scale follows the one fp8 rule with a power-of-two scale that
 *     the pages do print ([cache page] quantize_cache, fp8): s = pow2ceil(
 *     max(amax / 448, 2^-126)), stored as the e8m0 byte 127 + log2(s); the
 *     codes are e4m3(x / s) (R11, R14); decoding multiplies the e4m3 value by
 *     2^(b - 127) in binary32 and rounds once to the output dtype;
 *  R16 static two-level FP4 ([modelopt] _block_scale_from_amax with FP8 block
 *     scales, then _fake_quantize): binary32 throughout, left to right,
 *       P  = G / 6, replaced by 1e-8 when <= 1e-8     (per-tensor scale)
 *       m  = c * P with c = binary32(2^-9 / 448)      (smallest block scale)
 *       s  = a / 6, replaced by m when <= m           (block scale)
 *       t  = 448 / P; b = e4m3(s * t); s' = e4m3value(b) / t
 *       y  = RN_dtype(e2m1(x / s') * s')
 *     The e4m3 fake-quant under the amax P (scaled_e4m3 is named, not
 *     printed) is taken as multiply by 448 / P, cast, divide by 448 / P.  The
 *     printed division / cast / multiply with one amax for both the pre and
 *     the post scale is taken as the static branch's arithmetic (its callee
 *     is named, not printed); the fp4 cast rounds as R1 and R2;
 *  R17 static FP4 amax inputs: one float32 block amax per B consecutive
 *     columns of a row ([rows, K / B]) and one float32 global amax, all
 *     finite and >= 0 (the quantizer's own amax validation rejects others);
 *  R18 paged KV cache ([longlive] dequantize_kv_cache): block b holds the
 *     rows t * H + h (token t < block_tokens, head h) of D columns, in
 *     NVFP4 with row-major e4m3 scale bytes [block_tokens * H, D / 16] (the
 *     swizzled layout of the page's third-party tensor class is out of
 *     scope) and one float32 amax; its global scale is amax / (6 * 448) in
 *     binary32 (the e2m1 and e4m3 maxima of the default scale rule); rows
 *     decode as R5's NVFP4 and land at token b * block_tokens + t;
 *  R19 k_smooth ([longlive] k_smooth): the mean over the last dim is the
 *     binary32 pairwise sum (halves summed recursively, D a power of two)
 *     times 1 / D, rounded to the tensor dtype; k - mean is evaluated in
 *     binary32 and rounded to the dtype (reduced-precision tensors compute
 *     in binary32 and round the result);
 *  R20 quantize_kv ([longlive] quantize_kv): each head's [S, D] slice, after
 *     k_smooth when it holds keys, is quantized to NVFP4 with the amax of the
 *     whole slice (the quantize_nvfp4_modelopt rule: one global scale per
 *     head, written to each of the head's rows); the page's MSE scale rule
 *     belongs to a third-party library and is out of scope.
 */
#include "mxq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------
 * Threads.  The row loops below are OpenMP loops with a static schedule:
 * rows are independent and each row's arithmetic runs on one thread in the
 * order written, so the results do not depend on the thread count.  The
 * count is the oracle's own (set by orc_set_threads, else the runtime's
 * default) and is passed to every loop, so that other users of the same
 * OpenMP runtime in the process cannot change it.
 * ---------------------------------------------------------------------- */
static int g_threads = 0;

static int team(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_threads(int n) { g_threads = n > 0 ? n : 0; }

int orc_max_threads(void) { return team(); }

/* ------------------------------------------------------------------------
 * Number formats
 * ---------------------------------------------------------------------- */

/* The e2m1 value table, [mxfp4 page] Data, _FP4_E2M1_TABLE: 16 entries, the
 * first eight are the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; entry 8 is +0.0
 * and entries 9..15 are the negatives of entries 1..7 (the printed list is
 * cut off after -2; the rest follows by sign symmetry and E2M1_MAX = 6 on the
 * [nvfp4 page] Data section). */
static const double E2M1_TABLE[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0};

/* The rounding midpoints, [mxfp4 page] Data, _FP4_E2M1_MIDPOINTS (float32). */
static const float E2M1_MIDPOINTS[7] = {0.25f, 0.75f, 1.25f, 1.75f,
                                        2.5f,  3.5f,  5.0f};

double orc_e2m1_decode(uint32_t code) { return E2M1_TABLE[code & 15u]; }

/* Round a scaled value to an e2m1 magnitude index: the number of midpoints
 * that lie strictly below |q| (reading R1: a value on a midpoint takes the
 * lower bucket).  NaN compares false everywhere and gives 0; values beyond
 * the last midpoint give 7, i.e. saturate at 6. */
uint32_t orc_e2m1_round_mag(float q) {
  float a = fabsf(q);
  uint32_t n = 0;
  for (int j = 0; j < 7; ++j)
    if (a > E2M1_MIDPOINTS[j]) ++n;
  return n;
}

/* e2m1 code of element x whose scaled value is q (reading R2). */
static uint32_t e2m1_code(float x, float q) {
  return (signbit(x) ? 8u : 0u) | orc_e2m1_round_mag(q);
}

/* Round v to the nearest number with a p-bit significand (implicit bit
 * included) and exponent >= emin (smaller magnitudes use the subnormal
 * quantum 2^(emin-p+1)); no upper exponent bound; ties to even.
 * This is the textbook definition of round-to-nearest-even into a binary
 * floating-point format; callers apply their own overflow rule. */
double orc_round_binary(double v, int p, int emin) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  double a = fabs(v);
  int ex;
  (void)frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex-1 */
  int e = ex - 1;
  if (e < emin) e = emin;
  double quantum = ldexp(1.0, e - (p - 1));
  double n = a / quantum;       /* exact: scaling by a power of two */
  double r = nearbyint(n) * quantum; /* default rounding: to nearest even */
  return v < 0 ? -r : r;
}

/* float8 e4m3fn decoding (bias 7, 3 mantissa bits, subnormal quantum 2^-9,
 * no infinities, 0x7F/0xFF are NaN).  The [nvfp4 page] names the dtype and
 * its constants E4M3_MAX = 448 and E4M3_MIN_SUBNORMAL = 2^-9. */
double orc_e4m3_decode(uint32_t byte) {
  byte &= 0xFFu;
  int s = (byte >> 7) & 1, E = (byte >> 3) & 15, m = byte & 7;
  if (E == 15 && m == 7) return NAN;
  double v = (E == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
  return s ? -v : v;
}

/* float8 e4m3fn encoding of v: round to nearest even on the e4m3 grid
 * (4-bit significand, minimum exponent -6), saturating at 448 (reading R14),
 * then write the byte whose decoding is that value.  The sign bit is kept. */
uint32_t orc_e4m3_encode(float v) {
  double r = orc_round_binary(fabs((double)v), 4, -6);
  if (r > 448.0) r = 448.0;
  uint32_t byte;
  if (r < ldexp(1.0, -6)) {
    byte = (uint32_t)(r / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
  } else {
    int ex;
    double m = frexp(r, &ex); /* r = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;           /* r = (1 + f/8) * 2^E */
    uint32_t f = (uint32_t)((m * 2.0 - 1.0) * 8.0);
    byte = ((uint32_t)(E + 7) << 3) | f;
  }
  return (signbit(v) ? 0x80u : 0u) | byte;
}

/* float8 e8m0fnu decoding: 2^(b-127); 0xFF is NaN ([mxfp4 page] names the
 * dtype float8_e8m0fnu for the block scales). */
double orc_e8m0_decode(uint32_t byte) {
  byte &= 0xFFu;
  if (byte == 0xFFu) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* floor(log2(a)) for a > 0, exact (reading R3). */
int orc_floor_log2(float a) {
  int ex;
  (void)frexpf(a, &ex);
  return ex - 1;
}

/* [cache page] _power_of_two_ceiling: the smallest power of two that is >= v,
 * for a positive normal binary32 v. */
float orc_pow2_ceil(float v) {
  int ex;
  float m = frexpf(v, &ex); /* v = m * 2^ex, m in [0.5, 1) */
  if (m == 0.5f) return v;  /* already a power of two */
  return ldexpf(1.0f, ex);
}

/* ---- element load / store for the three floating dtypes ---- */

static float f16_bits_to_float(uint16_t h) {
  int s = (h >> 15) & 1, E = (h >> 10) & 31, m = h & 1023;
  double v;
  if (E == 31) v = m ? NAN : INFINITY;
  else if (E == 0) v = ldexp((double)m, -24);
  else v = ldexp(1.0 + m / 1024.0, E - 15);
  return (float)(s ? -v : v);
}

float orc_load(const void* x, int dtype, int64_t i) {
  if (dtype == 0) return ((const float*)x)[i];
  uint16_t h = ((const uint16_t*)x)[i];
  if (dtype == 1) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  return f16_bits_to_float(h);
}

/* Round a binary32 value to the output dtype: round-to-nearest-even, IEEE
 * overflow to infinity. */
void orc_store(void* y, int dtype, int64_t i, float v) {
  if (dtype == 0) { ((float*)y)[i] = v; return; }
  uint16_t out;
  if (isnan(v)) {
    out = (dtype == 1) ? 0x7FC0u : 0x7E00u;
  } else if (dtype == 1) {
    /* bfloat16: 8-bit significand, same exponent range as binary32 */
    double r = orc_round_binary((double)v, 8, -126);
    double maxv = ldexp(2.0 - ldexp(1.0, -7), 127);
    if (fabs(r) > maxv) r = signbit(v) ? -INFINITY : INFINITY;
    float rf = (float)r; /* exact: r is a bfloat16 value */
    uint32_t u;
    memcpy(&u, &rf, 4);
    out = (uint16_t)(u >> 16);
  } else {
    /* float16: 11-bit significand, exponents -14..15 */
    double r = orc_round_binary((double)v, 11, -14);
    uint16_t s = signbit(v) ? 0x8000u : 0u;
    double a = fabs(r);
    if (a > 65504.0) out = s | 0x7C00u;
    else if (a == 0.0) out = s;
    else if (a < ldexp(1.0, -14)) out = s | (uint16_t)(a / ldexp(1.0, -24));
    else {
      int ex;
      double m = frexp(a, &ex); /* a = m * 2^ex, m in [0.5,1) */
      int E = ex - 1;
      uint16_t man = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
      out = s | (uint16_t)((E + 15) << 10) | man;
    }
  }
  ((uint16_t*)y)[i] = out;
}

/* ------------------------------------------------------------------------
 * MXFP4  ([mxfp4 page] quantize_mxfp4, dequantize_mxfp4)
 * ---------------------------------------------------------------------- */

#define MXFP4_BLOCK 32 /* [mxfp4 page] Data, MXFP4_BLOCK_SIZE */

/* Quantize along the last dim: one e8m0 scale per 32 columns, the scale being
 * 2^(floor(log2(amax)) - 2) ([mxfp4 page] quantize_mxfp4), two e2m1 codes per
 * byte with the even column in the low nibble ([mxfp4 page] introduction). */
void orc_quantize_mxfp4(const void* x, int dtype, int64_t rows, int64_t K,
                        uint8_t* packed, uint8_t* scales) {
  int64_t nblk = K / MXFP4_BLOCK;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nblk; ++b) {
      int64_t base = r * K + b * MXFP4_BLOCK;
      /* step 1: block amax */
      float amax = 0.0f;
      for (int j = 0; j < MXFP4_BLOCK; ++j) {
        float v = fabsf(orc_load(x, dtype, base + j));
        if (v > amax) amax = v;
      }
      /* step 2: scale exponent floor(log2 amax) - 2, stored as e8m0 (R4) */
      int e = (amax > 0.0f) ? orc_floor_log2(amax) - 2 : -127;
      if (e < -127) e = -127;
      uint8_t sbyte = (uint8_t)(e + 127);
      scales[r * nblk + b] = sbyte;
      float scale = (float)orc_e8m0_decode(sbyte);
      /* step 3: divide by the scale, round to e2m1, pack pairs */
      uint32_t code[MXFP4_BLOCK];
      for (int j = 0; j < MXFP4_BLOCK; ++j) {
        float v = orc_load(x, dtype, base + j);
        code[j] = e2m1_code(v, v / scale);
      }
      for (int j = 0; j < MXFP4_BLOCK; j += 2)
        packed[(base + j) / 2] = (uint8_t)(code[j] | (code[j + 1] << 4));
    }
  }
}

/* Decode: unpack the two nibbles (low nibble = even column), look up the e2m1
 * table, multiply by the e8m0 scale 2^(b-127) in binary32, round to dtype
 * ([mxfp4 page] dequantize_mxfp4 and _FP4_BYTE_TABLE). */
void orc_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scales,
                          int64_t rows, int64_t K, void* y, int dtype) {
  int64_t nblk = K / MXFP4_BLOCK;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      int64_t i = r * K + k;
      uint8_t byte = packed[i / 2];
      uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
      float scale = (float)orc_e8m0_decode(scales[r * nblk + k / MXFP4_BLOCK]);
      float v = (float)orc_e2m1_decode(code) * scale;
      orc_store(y, dtype, i, v);
    }
  }
}

/* ------------------------------------------------------------------------
 * NVFP4  ([nvfp4 page] quantize_nvfp4, quantize_nvfp4_modelopt,
 *         dequantize_nvfp4, Data)
 * ---------------------------------------------------------------------- */

#define NVFP4_BLOCK 16           /* NVFP4_BLOCK_SIZE */
static const float E2M1_MAX = 6.0f;   /* E2M1_MAX */
static const float E4M3_MAX = 448.0f; /* E4M3_MAX */
#define E4M3_MIN_SUBNORMAL 0.001953125f /* 2^-9, E4M3_MIN_SUBNORMAL */

/* Block-scale clamp (reading R6): maxNum with the smallest e4m3 subnormal
 * (fmaxf returns the non-NaN operand), then min with E4M3_MAX. */
static float clamp_block_scale(float u) {
  return fminf(fmaxf(u, E4M3_MIN_SUBNORMAL), E4M3_MAX);
}

/* Quantize along the last dim ([nvfp4 page] quantize_nvfp4):
 *   global      = amax / (6 * 448)                (per row, or given)
 *   block_scale = e4m3(amax(block) / 6 / global)
 *   code        = round_to_e2m1(w / (block_scale * global))
 * mode 2 uses one amax for the whole tensor ([nvfp4 page]
 * quantize_nvfp4_modelopt) and writes that one scale to every row. */
void orc_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t K,
                        int mode, const float* given, int64_t given_stride,
                        uint8_t* packed, uint8_t* scales, float* row_scale) {
  int64_t nblk = K / NVFP4_BLOCK;
  float tensor_amax = 0.0f;
  if (mode == 2) {
#pragma omp parallel for schedule(static) num_threads(team()) reduction(max : tensor_amax)
    for (int64_t i = 0; i < rows * K; ++i) {
      float v = fabsf(orc_load(x, dtype, i));
      if (v > tensor_amax) tensor_amax = v;
    }
  }
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    /* step 1: the row's global scale */
    float g;
    if (mode == 1) {
      g = given[r * given_stride];
    } else {
      float amax = tensor_amax;
      if (mode == 0) {
        amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
          float v = fabsf(orc_load(x, dtype, r * K + k));
          if (v > amax) amax = v;
        }
      }
      g = amax / (E2M1_MAX * E4M3_MAX); /* 6 * 448 = 2688, exact */
    }
    row_scale[r] = g;
    for (int64_t b = 0; b < nblk; ++b) {
      int64_t base = r * K + b * NVFP4_BLOCK;
      /* step 2: block amax and the e4m3 block scale */
      float a = 0.0f;
      for (int j = 0; j < NVFP4_BLOCK; ++j) {
        float v = fabsf(orc_load(x, dtype, base + j));
        if (v > a) a = v;
      }
      float u = a / E2M1_MAX;
      u = u / g;
      uint32_t sbyte = orc_e4m3_encode(clamp_block_scale(u));
      scales[r * nblk + b] = (uint8_t)sbyte;
      float sigma = (float)orc_e4m3_decode(sbyte);
      /* step 3: divide by block_scale * global, round to e2m1, pack */
      float den = sigma * g;
      uint32_t code[NVFP4_BLOCK];
      for (int j = 0; j < NVFP4_BLOCK; ++j) {
        float v = orc_load(x, dtype, base + j);
        code[j] = e2m1_code(v, v / den);
      }
      for (int j = 0; j < NVFP4_BLOCK; j += 2)
        packed[(base + j) / 2] = (uint8_t)(code[j] | (code[j + 1] << 4));
    }
  }
}

/* Decode ([nvfp4 page] dequantize_nvfp4): e2m1 * float(e4m3 block scale) *
 * row scale, binary32 intermediates evaluated left to right, one final
 * rounding to dtype. */
void orc_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales,
                          const float* row_scale, int64_t rows, int64_t K,
                          void* y, int dtype) {
  int64_t nblk = K / NVFP4_BLOCK;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    float g = row_scale[r];
    for (int64_t k = 0; k < K; ++k) {
      int64_t i = r * K + k;
      uint8_t byte = packed[i / 2];
      uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
      float sigma = (float)orc_e4m3_decode(scales[r * nblk + k / NVFP4_BLOCK]);
      float t = (float)orc_e2m1_decode(code) * sigma;
      float z = t * g;
      orc_store(y, dtype, i, z);
    }
  }
}

/* ------------------------------------------------------------------------
 * Cache quantize/dequantize round trip ([cache page] quantize_cache,
 * _CacheQuantization.forward, _power_of_two_ceiling)
 * ---------------------------------------------------------------------- */

/* One group of n <= block_size consecutive channels (n < block_size only for
 * the last group of a row, which then behaves as if zero-padded: the padding
 * never raises the amax and is never written, reading R10). */
static void cache_group(const void* x, void* y, int dtype, int64_t base,
                        int64_t n, int fmt) {
  float a = 0.0f;
  for (int64_t j = 0; j < n; ++j) {
    float v = fabsf(orc_load(x, dtype, base + j));
    if (v > a) a = v;
  }
  if (fmt == 0) {
    /* fp8: power-of-two scale >= amax / 448, values stored as e4m3 */
    float v = fmaxf(a / E4M3_MAX, FLT_MIN);
    float s = orc_pow2_ceil(v);
    for (int64_t j = 0; j < n; ++j) {
      float xv = orc_load(x, dtype, base + j);
      uint32_t qb = orc_e4m3_encode(xv / s); /* sign kept (R11) */
      float out = (float)orc_e4m3_decode(qb) * s;
      orc_store(y, dtype, base + j, out);
    }
  } else if (fmt == 1) {
    /* mxfp4: power-of-two (e8m0) scale >= amax / 6, values e2m1 */
    float v = fmaxf(a / E2M1_MAX, FLT_MIN);
    float s = orc_pow2_ceil(v);
    for (int64_t j = 0; j < n; ++j) {
      float xv = orc_load(x, dtype, base + j);
      uint32_t c = e2m1_code(xv, xv / s);
      float out = (float)orc_e2m1_decode(c) * s;
      orc_store(y, dtype, base + j, out);
    }
  } else {
    /* nvfp4: one e4m3 scale per group, values e2m1 */
    float sigma =
        (float)orc_e4m3_decode(orc_e4m3_encode(clamp_block_scale(a / E2M1_MAX)));
    for (int64_t j = 0; j < n; ++j) {
      float xv = orc_load(x, dtype, base + j);
      uint32_t c = e2m1_code(xv, xv / sigma);
      float out = (float)orc_e2m1_decode(c) * sigma;
      orc_store(y, dtype, base + j, out);
    }
  }
}

void orc_quantize_cache(const void* x, void* y, int dtype, int64_t rows,
                        int64_t C, int fmt, int64_t block_size) {
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c0 = 0; c0 < C; c0 += block_size) {
      int64_t n = (C - c0 < block_size) ? C - c0 : block_size;
      cache_group(x, y, dtype, r * C + c0, n, fmt);
    }
}

/* ------------------------------------------------------------------------
 * Grouped GEMM ([mxfp4 page] MXFP4GroupedMM.forward / backward, [nvfp4 page]
 * NVFP4GroupedMM.forward / backward): the activations of expert e are rows
 * offs[e-1] .. offs[e]-1 of x (offs[-1] = 0); the forward multiplies them by
 * the transposed dequantized weights W_e^T ([N, K] stored, [K, N] used), the
 * backward multiplies the output gradient by W_e.  The weights enter as the
 * dequantized values in the activation dtype, as the pages' dequantize-then-
 * grouped-matmul does.  Written as the plain sum of products, per output.
 * ---------------------------------------------------------------------- */
void orc_grouped_mm(const void* x, int xdt, int64_t T, const void* w, int wdt,
                    int64_t E, int64_t N, int64_t K, const int32_t* offs,
                    int trans, const int64_t* rows, int64_t nrows,
                    double* out, double* absout) {
  int64_t din = trans ? N : K, dout = trans ? K : N;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = rows[i];
    int64_t e = -1, lo = 0;
    for (int64_t j = 0; j < E; ++j) {
      int64_t hi = offs[j];
      if (r >= lo && r < hi) { e = j; break; }
      if (hi > lo) lo = hi;
    }
    for (int64_t o = 0; o < dout; ++o) {
      double acc = 0.0, aacc = 0.0;
      if (e >= 0 && r < T) {
        for (int64_t d = 0; d < din; ++d) {
          double xv = orc_load(x, xdt, r * din + d);
          int64_t wi = trans ? (e * N + d) * K + o : (e * N + o) * K + d;
          double wv = orc_load(w, wdt, wi);
          acc += xv * wv;
          aacc += fabs(xv * wv);
        }
      }
      out[i * dout + o] = acc;
      absout[i * dout + o] = aacc;
    }
  }
}


/* ------------------------------------------------------------------------
 * MXFP8 real quantization ([modelopt] _real_quantize, MX branch, e4m3
 * elements; reading R15)
 * ---------------------------------------------------------------------- */

#define MXFP8_BLOCK 32 /* the branch asserts MXFP8's block size of 32 */

void orc_quantize_mxfp8(const void* x, int dtype, int64_t rows, int64_t K,
                        uint8_t* codes, uint8_t* scales) {
  int64_t nblk = K / MXFP8_BLOCK;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nblk; ++b) {
      int64_t base = r * K + b * MXFP8_BLOCK;
      /* step 1: block amax */
      float amax = 0.0f;
      for (int j = 0; j < MXFP8_BLOCK; ++j) {
        float v = fabsf(orc_load(x, dtype, base + j));
        if (v > amax) amax = v;
      }
      /* step 2: power-of-two scale >= amax / 448, floored at 2^-126 */
      float s = orc_pow2_ceil(fmaxf(amax / E4M3_MAX, FLT_MIN));
      int ex;
      (void)frexpf(s, &ex);             /* s = 2^(ex - 1) */
      scales[r * nblk + b] = (uint8_t)(ex - 1 + 127);
      /* step 3: e4m3 of x / s, sign kept */
      for (int j = 0; j < MXFP8_BLOCK; ++j) {
        float v = orc_load(x, dtype, base + j);
        codes[base + j] = (uint8_t)orc_e4m3_encode(v / s);
      }
    }
  }
}

void orc_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales,
                          int64_t rows, int64_t K, void* y, int dtype) {
  int64_t nblk = K / MXFP8_BLOCK;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      int64_t i = r * K + k;
      float scale = (float)orc_e8m0_decode(scales[r * nblk + k / MXFP8_BLOCK]);
      float v = (float)orc_e4m3_decode(codes[i]) * scale;
      orc_store(y, dtype, i, v);
    }
  }
}

/* ------------------------------------------------------------------------
 * Static two-level FP4 fake quantization ([modelopt]
 * StaticBlockScaleQuantizer._block_scale_from_amax, _fake_quantize,
 * _amax_to_scale, _clamp_scale, _FP8_E4M3_MIN_POSITIVE; readings R16, R17)
 * ---------------------------------------------------------------------- */

/* _clamp_scale: values at or below the floor are replaced by the floor. */
static float clamp_scale_floor(float v, float floor_value) {
  return (v <= floor_value) ? floor_value : v;
}

/* The dequantization-side block scale s' of a block with amax a under the
 * global amax G (reading R16). */
float orc_static_block_scale(float a, float G) {
  /* _amax_to_scale(global_amax, 6) with the default floor 1e-8 */
  float P = clamp_scale_floor(G / E2M1_MAX, 1e-8f);
  /* smallest encodable block scale in physical units: (2^-9 / 448) * P */
  float c = (float)(0x1p-9 / 448.0);
  float m = c * P;
  /* _amax_to_scale(amax, 6, min_value = m) */
  float s = clamp_scale_floor(a / E2M1_MAX, m);
  /* e4m3 fake quantization of s with P mapped to 448 */
  float t = E4M3_MAX / P;
  uint32_t byte = orc_e4m3_encode(s * t);
  return (float)orc_e4m3_decode(byte) / t;
}

void orc_fake_quantize_fp4_static(const void* x, int dtype, int64_t rows,
                                  int64_t K, int64_t block,
                                  const float* block_amax, float G, void* y) {
  int64_t nblk = K / block;
#pragma omp parallel for schedule(static) num_threads(team())
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nblk; ++b) {
      float sp = orc_static_block_scale(block_amax[r * nblk + b], G);
      for (int64_t j = 0; j < block; ++j) {
        int64_t i = r * K + b * block + j;
        float v = orc_load(x, dtype, i);
        float q = v / sp;                          /* quant_input */
        uint32_t c = e2m1_code(v, q);              /* fp4 cast */
        float w = (float)orc_e2m1_decode(c);
        orc_store(y, dtype, i, w * sp);            /* times the post scale */
      }
    }
  }
}

/* ------------------------------------------------------------------------
 * Paged NVFP4 KV cache and k_smooth ([longlive] dequantize_kv_cache,
 * k_smooth, quantize_kv; readings R18 - R20)
 * ---------------------------------------------------------------------- */

/* Block b of the cache: values[b] (uint8 [block_tokens * H, D / 2]),
 * scales[b] (e4m3 bytes [block_tokens * H, D / 16]), amax[b] (one float).
 * Output y: [nblocks * block_tokens, H, D] in dtype. */
void orc_dequantize_kv_pages(const uint8_t* const* values,
                             const uint8_t* const* scales, const float* amax,
                             int64_t nblocks, int64_t block_tokens, int64_t H,
                             int64_t D, void* y, int dtype) {
  int64_t rows = block_tokens * H;
  for (int64_t b = 0; b < nblocks; ++b) {
    float g = amax[b] / (E2M1_MAX * E4M3_MAX);
#pragma omp parallel for schedule(static) num_threads(team())
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t d = 0; d < D; ++d) {
        uint8_t byte = values[b][(r * D + d) / 2];
        uint32_t code = (d & 1) ? (byte >> 4) : (byte & 15u);
        float sigma = (float)orc_e4m3_decode(scales[b][r * (D / NVFP4_BLOCK) + d / NVFP4_BLOCK]);
        float t = (float)orc_e2m1_decode(code) * sigma;
        /* token b * block_tokens + t_in, head h: row b * rows + r of y */
        orc_store(y, dtype, (b * rows + r) * D + d, t * g);
      }
    }
  }
}

/* Pairwise binary32 sum of n values (n a power of two). */
static float pairwise_sum(const float* v, int64_t n) {
  if (n == 1) return v[0];
  return pairwise_sum(v, n / 2) + pairwise_sum(v + n / 2, n / 2);
}

/* k_smooth of one row of D values in dtype, in place in `row` (R19). */
void orc_k_smooth_row(float* row, int64_t D, int dtype) {
  float mean = pairwise_sum(row, D) * (1.0f / (float)D);  /* exact scaling */
  float m = mean;
  if (dtype != 0) {            /* round the mean to the tensor dtype */
    uint16_t h;
    orc_store(&h, dtype, 0, mean);
    m = orc_load(&h, dtype, 0);
  }
  for (int64_t d = 0; d < D; ++d) {
    float diff = row[d] - m;
    uint16_t h;
    if (dtype != 0) {
      orc_store(&h, dtype, 0, diff);
      diff = orc_load(&h, dtype, 0);
    }
    row[d] = diff;
  }
}

/* quantize_kv for one tensor k [S, H, D] (R20): per head, optional k_smooth
 * of every row, then NVFP4 with the head slice's amax.  Outputs in the
 * layout of k: packed [S, H, D / 2], scales [S, H, D / 16], row_scale [S, H]
 * (the head's global scale on each of its rows). */
void orc_quantize_kv_nvfp4(const void* k, int dtype, int64_t S, int64_t H,
                           int64_t D, int smooth, uint8_t* packed,
                           uint8_t* scales, float* row_scale) {
  float* slice = (float*)malloc(sizeof(float) * (size_t)(S * D));
  uint8_t* p = (uint8_t*)malloc((size_t)(S * D / 2));
  uint8_t* sc = (uint8_t*)malloc((size_t)(S * D / NVFP4_BLOCK));
  float* g = (float*)malloc(sizeof(float) * (size_t)S);
  for (int64_t h = 0; h < H; ++h) {
    /* the head's slice k[:, h, :], smoothed row by row */
#pragma omp parallel for schedule(static) num_threads(team())
    for (int64_t s = 0; s < S; ++s) {
      for (int64_t d = 0; d < D; ++d)
        slice[s * D + d] = orc_load(k, dtype, (s * H + h) * D + d);
      if (smooth) orc_k_smooth_row(slice + s * D, D, dtype);
    }
    /* NVFP4 of the slice with its whole-slice amax (mode 2); the smoothed
     * values are dtype values, so quantizing their float32 copies is the
     * same as quantizing the dtype tensor */
    orc_quantize_nvfp4(slice, 0, S, D, 2, NULL, 0, p, sc, g);
    for (int64_t s = 0; s < S; ++s) {
      memcpy(packed + (s * H + h) * (D / 2), p + s * (D / 2), (size_t)(D / 2));
      memcpy(scales + (s * H + h) * (D / NVFP4_BLOCK), sc + s * (D / NVFP4_BLOCK),
             (size_t)(D / NVFP4_BLOCK));
      row_scale[s * H + h] = g[s];
    }
  }
  free(slice);
  free(p);
  free(sc);
  free(g);
}
