// mxq_device.h -- per-element arithmetic and wave primitives for the gfx950
// kernels of libmxq.
//
// The element math (MXQ_HD functions) is written so that it also compiles for
// the host: the test-suite builds it into a small host library and checks it
// exhaustively against the CPU oracle without a GPU.  Everything here is plain
// binary32/binary64 IEEE arithmetic plus integer bit manipulation; no fast-math
// and no contraction (the library is compiled with -ffp-contract=off, and the
// only fused multiply-adds are the explicit fmaf/fma calls below).
//
// Formats (sources cited by page title and section):
//  e2m1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6, rounding midpoints .25 .. 5
//        ("nemo_automodel.components.quantization.mxfp4", Data section);
//        a value on a midpoint rounds to the smaller magnitude.
//  e8m0: 2^(b - 127) (same page, scales of quantize_mxfp4).
//  e4m3fn: bias 7, 3 mantissa bits, max 448, subnormal quantum 2^-9
//        ("nemo_automodel.components.quantization.nvfp4", Data section).
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MXQ_HD __host__ __device__ __forceinline__
#else
#include <math.h>
#define MXQ_HD static inline
#endif

namespace mxq {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum : int { FMT_FP8 = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2 };

MXQ_HD uint32_t fbits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
MXQ_HD float bitsf(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
MXQ_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
MXQ_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------- e2m1

// Rounding constants for the bit-level e2m1 rounding.  For q in [1, 8) the
// float32 pattern of q, plus (2^21 - 1), shifted right by 22, is 252 + code:
// the kept mantissa bit is bit 22 and the +(2^21 - 1) rounds a remainder that
// is strictly above one half up and a remainder of exactly one half down,
// which is "ties to the smaller magnitude" because the e2m1 midpoints above 1
// (1.25, 1.75, 2.5, 3.5, 5) are exactly the half-way points of that grid.
constexpr int32_t kHiBias = 0x1FFFFF - (252 << 22);
// For q in [0, 1) the e2m1 grid is 0, 0.5, 1 with midpoints 0.25 and 0.75;
// 1 + q lies in [1, 2) whose 1-bit-mantissa grid is 1, 1.5, 2 with the same
// relative midpoints, so the same rounding applied to 1 + q gives 254 + code.
constexpr int32_t kLoBias = 0x1FFFFF - (254 << 22);
constexpr int32_t kCodeMax = 7 << 22;

// Magnitude code (0..7) of q = a * s, where a = |x| has at most 12
// significant bits (a bfloat16 or float16 input) and s is a power of two.
// Exactness: a * s is exact; 1 + q is exact whenever q >= 2^-13 (its lowest
// set bit is then >= 2^-23), and for smaller q both 1 + q and the result are
// below 1.25 so the code is 0 either way.
MXQ_HD uint32_t e2m1_mag_short(float a, float s) {
  float q = a * s;
  float q1 = fmaf(a, s, 1.0f);
  int32_t hi = (int32_t)fbits(q) + kHiBias;
  int32_t lo = (int32_t)fbits(q1) + kLoBias;
  return (uint32_t)imin(imax(lo, hi), kCodeMax) >> 22;
}

// Magnitude code of an arbitrary non-negative float32 q (24-bit significand,
// any size, +inf included).  Below 1 the two midpoints are compared directly;
// NaN must be handled by the caller.
MXQ_HD uint32_t e2m1_mag_f32(float q) {
  int32_t hi = (int32_t)fbits(q) + kHiBias;
  int32_t lo = ((int32_t)(q > 0.25f) + (int32_t)(q > 0.75f)) << 22;
  return (uint32_t)imin(imax(lo, hi), kCodeMax) >> 22;
}

// Round a float32 magnitude up to at most 22 significant bits, keeping the
// sign.  Every e2m1 midpoint (and every e2m1 value) has at most 3 significant
// bits, so it lies on the 22-bit grid and q <= m holds exactly when
// ceil22(q) <= m: the e2m1 rounding decisions of q and ceil22(q) are the same.
// (The gfx950 stochastic-rounding fp4 converter is exact for operands with at
// most 22 significant bits; it can drop the lowest two bits of a 24-bit
// operand that it aligns into the e2m1 subnormal range.)
MXQ_HD float ceil22(float q) { return bitsf((fbits(q) + 3u) & ~3u); }

// Operand for a round-to-nearest-even e2m1 conversion (scale 1, or a power of
// two that keeps the midpoints normal) that is to round half down instead,
// for any float32 q.  Ties to even already go down at the midpoints 0.25,
// 1.25, 2.5 and 5 (their lower neighbour has the even code) and go up at
// 0.75, 1.75 and 3.5 -- exactly the midpoints whose significand has bit 22
// set (0.25 has none of its fraction bits set, the other three bit 21 only).
// Taking one unit in the last place off every operand with that bit set
// moves an operand that sits on one of those three just below it, and the
// operand one unit above lands on the midpoint, which still rounds up.  A
// one-unit step can carry an operand across a midpoint only from the
// midpoint itself, so no other decision changes.  Zeros (bit 22 clear),
// infinities (likewise) and subnormals (far below 0.25) keep their codes, and
// the sign is untouched.
MXQ_HD float half_down_for_rne(float q) {
  const uint32_t u = fbits(q);
  return bitsf(u - ((u >> 22) & 1u));
}

// 2 * e2m1 magnitude for code 0..7: 0 1 2 3 4 6 8 12 (an integer).
MXQ_HD uint32_t e2m1_twice_mag(uint32_t c) {
  return (uint32_t)((0x0C08060403020100ull >> (8 * (c & 7))) & 0xFF);
}

// float32 value of a 4-bit e2m1 code; code 8 (negative zero) gives +0.0.
MXQ_HD float e2m1_decode(uint32_t c) {
  int32_t m = (int32_t)e2m1_twice_mag(c);
  if (c & 8) m = -m;
  return (float)m * 0.5f;
}

// ---------------------------------------------------------------- e4m3

// e4m3fn byte of u in [2^-9, 448]: round to nearest, ties to even.  Both
// ranges are evaluated and one is selected (no branches).  *value receives
// the float32 value of the byte.
MXQ_HD uint32_t e4m3_encode_pos_v(float u, float* value) {
  // below 2^-6 the quantum is 2^-9: adding and removing 2^14 (ulp 2^-9)
  // rounds to nearest even
  const float r = (u + 16384.0f) - 16384.0f;
  const uint32_t sub = (uint32_t)(r * 512.0f);                 // 1..8
  // normal range: keep 3 mantissa bits, round to nearest even
  const uint32_t b = fbits(u);
  const uint32_t rb = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  const uint32_t nrm = (rb >> 20) - (120u << 3);                // rebias 127 -> 7
  const bool small = u < 0.015625f;
  *value = small ? r : bitsf(rb);
  return small ? sub : nrm;
}

MXQ_HD uint32_t e4m3_encode_pos(float u) {
  float v;
  return e4m3_encode_pos_v(u, &v);
}

// e4m3fn byte and value of u in [2^-9, 448]: on the GPU the hardware fp8
// converters, which round to nearest even and agree with e4m3_encode_pos_v
// on every float32 of that range; on the host e4m3_encode_pos_v itself.
MXQ_HD uint32_t e4m3_encode_clamped(float u, float* value) {
#if defined(__HIP_DEVICE_COMPILE__)
  // Both bytes of the low half take the code and the high half keeps the old
  // operand (u's own bits, which saves zeroing a register); the decode reads
  // byte 0 only.
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(u, u, (int)fbits(u), false);
  *value = __builtin_amdgcn_cvt_f32_fp8(w, 0);
  return (uint32_t)w & 0xFFu;
#else
  return e4m3_encode_pos_v(u, value);
#endif
}

// float32 value of a positive e4m3fn byte (0x00..0x7E).
MXQ_HD float e4m3_decode_pos(uint32_t b) {
  return b >= 8 ? bitsf((b << 20) + (120u << 23)) : (float)b * 0.001953125f;
}

// e4m3 round-to-nearest-even of r in [0, 448 * (1 + 2^-23)], returned as a
// float32 value (saturates at 448): add and remove a power of two whose ulp is
// the e4m3 quantum of r's binade (2^-9 below 2^-6).
MXQ_HD float e4m3_round_value(float r) {
  uint32_t e = fbits(r) >> 23;
  e = e < 121u ? 121u : e;                   // binades below 2^-6 share 2^-9
  float c = bitsf((e + 20u) << 23);          // 2^(E + 20): ulp = 2^(E - 3)
  float v = (r + c) - c;
  return v > 448.0f ? 448.0f : v;
}

// ---------------------------------------------------------------- e8m0

// e8m0 byte of the MXFP4 block scale 2^(floor(log2 amax) - 2), clamped below
// at 2^-127: floor(log2 amax) is the unbiased exponent field, and every amax
// below 2^-125 (subnormal or zero included) gives byte 0.
MXQ_HD uint32_t mxfp4_scale_byte(float amax) {
  uint32_t ex = fbits(amax) >> 23;           // amax >= 0
  return ex < 2u ? 0u : ex - 2u;
}

// 2^-(b - 127) as float32 for an e8m0 byte b in [0, 252] (always normal).
MXQ_HD float e8m0_inverse(uint32_t b) { return bitsf((254u - b) << 23); }

// 2^(b - 128) as float32 (half the e8m0 value, so that twice-magnitude
// integers times it give e2m1 * 2^(b - 127) exactly); NaN for b = 255.
MXQ_HD float e8m0_half(uint32_t b) {
  if (b == 255u) return bitsf(0x7FC00000u);
  if (b >= 2u) return bitsf((b - 1u) << 23);
  return bitsf(0x200000u << b);              // 2^-128, 2^-127: subnormal
}

// ---------------------------------------------------------------- pow2 ceiling

// Smallest power of two >= v for a positive normal float32 v (the cache
// page's _power_of_two_ceiling): adding 2^23 - 1 to the pattern carries into
// the exponent exactly when the mantissa is non-zero.
MXQ_HD float pow2_ceil(float v) { return bitsf((fbits(v) + 0x7FFFFFu) & 0xFF800000u); }

// ---------------------------------------------------------------- rounding to dtype

MXQ_HD uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = fbits(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float32 -> float16, round to nearest even, IEEE overflow to infinity, in
// integer arithmetic.  (A float conversion of a float32 product may be fused
// by the compiler into a single mixed-precision multiply-add, which rounds
// once instead of twice and turns -0 into +0; the integer form keeps the
// binary32 intermediate that the decode definitions require.)
MXQ_HD uint32_t f32_to_f16_rne(float f) {
  const uint32_t u = fbits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7E00u;            // NaN
  if (a >= 0x477FF000u) return sign | 0x7C00u;           // >= 65520: inf
  if (a >= 0x38800000u) {                                // normal float16
    const uint32_t r = a + 0xFFFu + ((a >> 13) & 1u);    // RNE at bit 13
    return sign | ((r >> 13) - (112u << 10));
  }
  const uint32_t e = a >> 23;                            // subnormal or 0
  if (e < 102u) return sign;                             // < 2^-25 (ties -> 0)
  const uint32_t m = (a & 0x7FFFFFu) | 0x800000u;
  const uint32_t shift = 126u - e;                       // 14..24
  uint32_t r = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (r & 1u))) ++r;
  return sign | r;
}

MXQ_HD float f16_to_f32(uint32_t h) {
  uint16_t u = (uint16_t)h;
  _Float16 v;
  memcpy(&v, &u, 2);
  return (float)v;
}

// ---------------------------------------------------------------- exact NVFP4 helpers

// float32 round-to-nearest of a / 6 (a >= 0 finite), as a binary64 product
// with a correctly rounded 1/6, rounded once to float32.  This equals the
// correctly rounded float32 quotient, subnormal results included: a / 6 =
// (a / 2) / 3 is either exact (when 3 divides a's significand) or not dyadic,
// so it is never a float32 rounding boundary.  For a normal quotient its
// relative distance to the nearest boundary is at least 2^-27; for a
// subnormal one (a below 6 * 2^-126) a and every boundary are multiples of
// 2^-150, so the distance is at least 2^-150 / 6.  The binary64 product is
// within 2^-52 (relative) of a / 6: far closer than either margin.
MXQ_HD float div6_rn(float a) { return (float)((double)a * (1.0 / 6.0)); }

// ---------------------------------------------------------------- per-chunk steps
// The kernels hand 8 consecutive elements (one "chunk", already widened to
// float32) and the block-level quantities to these functions; the reductions
// across lanes stay in the kernels.

// MXFP4: packed word of 8 codes (element i in nibble i) given the block's
// e8m0 byte.  `wide` selects the float32-input rounding (24-bit q).
MXQ_HD uint32_t mxfp4_quant8(const float f[8], uint32_t sbyte, bool wide) {
  const float s = e8m0_inverse(sbyte);         // 1 / stored scale, exact
  uint32_t word = 0;
  for (int i = 0; i < 8; ++i) {
    const float m = fabsf(f[i]);
    const uint32_t mag = wide ? e2m1_mag_f32(m * s) : e2m1_mag_short(m, s);
    word |= (mag | ((fbits(f[i]) >> 28) & 8u)) << (4 * i);
  }
  return word;
}

// MXFP4 decode of a packed word into 8 float32 values e2m1 * 2^(b - 127).
MXQ_HD void mxfp4_dequant8(uint32_t w, uint32_t sbyte, float out[8]) {
  const float s = e8m0_half(sbyte);            // 2^(b - 128)
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = (w >> (4 * i)) & 15u;
    int32_t m = (int32_t)e2m1_twice_mag(code);
    m = (code & 8u) ? -m : m;                  // -0 -> +0
    out[i] = (float)m * s;                     // exact
  }
}

// NVFP4 block scale from the block amax a and the row scale g:
// e4m3(clamp((a / 6) / g, 2^-9, 448)), a NaN ratio taking 2^-9; returns the
// byte and the divisor block_scale * g.  `rg` is the binary64 value 1 / g
// (correctly rounded), computed once per row.
//
// Both divisions are evaluated as binary64 products rounded once to float32
// (div6_rn above for a / 6).  For (a / 6) / g: the quotient of two 24-bit
// significands is never a float32 half-way point (the odd significand of a
// half-way point has 25 bits, more than a product of the two operands' odd
// parts can cancel), and when it is not, its relative distance to the nearest
// half-way point is above 2^-49, while the binary64 product is within 2^-52
// of it; so rounding the product gives the correctly rounded quotient.  Below
// the float32 normal range the clamp to 2^-9 hides any difference.
MXQ_HD uint32_t nvfp4_block_scale(float a, float g, double rg, float* den) {
  float u = div6_rn(a);
  u = (float)((double)u * rg);
  u = fminf(fmaxf(u, 0.001953125f), 448.0f);
  float sigma;
  const uint32_t sb = e4m3_encode_clamped(u, &sigma);
  *den = sigma * g;
  return sb;
}

// 1 / d in binary64 to within about 2^-52 relative error, for d a float32
// value that is finite and non-zero.  On the GPU: the hardware reciprocal
// refined by two Newton steps (the refinement the compiler's own binary64
// division builds on; each step squares the relative error), on the host the
// correctly rounded quotient.
MXQ_HD double recip64(double d) {
#if defined(__HIP_DEVICE_COMPILE__)
  double r = __builtin_amdgcn_rcp(d);
  double e = fma(-d, r, 1.0);
  r = fma(r, e, r);
  e = fma(-d, r, 1.0);
  return fma(r, e, r);
#else
  return 1.0 / d;
#endif
}

// NVFP4: packed word of 8 codes for elements divided by den; `rden` is the
// correctly rounded binary64 1 / den.  The code of x is decided by the
// float32 quotient q = RN(|x| / den) only through the comparisons
// q > m for the e2m1 midpoints m, i.e. |x| / den > m + ulp(m) / 2.  Those
// boundaries have 25-bit odd significands; |x| (bf16, f16 or f32) over den
// (24 bits) is never equal to one and, when not equal, differs by a relative
// 2^-49 or more, while the binary64 product |x| * rden is within 2^-51 of
// |x| / den.  So its float32 rounding lies on the same side of every boundary
// and gives the same code (a 0 / 0 NaN gives code 0, x / 0 code 7).
MXQ_HD uint32_t nvfp4_quant8(const float f[8], double rden) {
  uint32_t word = 0;
  for (int i = 0; i < 8; ++i) {
    float q = (float)((double)fabsf(f[i]) * rden);
    q = (q == q) ? q : 0.0f;
    word |= (e2m1_mag_f32(q) | ((fbits(f[i]) >> 28) & 8u)) << (4 * i);
  }
  return word;
}

// Any e4m3fn byte: sign, NaN for 0x7F / 0xFF.
MXQ_HD float e4m3_decode_any(uint32_t b) {
  const uint32_t m = b & 0x7Fu;
  const float v = (m == 0x7Fu) ? bitsf(0x7FC00000u) : e4m3_decode_pos(m);
  return (b & 0x80u) ? -v : v;
}

// NVFP4 decode: (e2m1 * e4m3) * g in float32, left to right.
MXQ_HD void nvfp4_dequant8(uint32_t w, uint32_t sbyte, float g, float out[8]) {
  const float sigma = e4m3_decode_any(sbyte);
  for (int i = 0; i < 8; ++i) {
    const float t = e2m1_decode((w >> (4 * i)) & 15u) * sigma;   // exact
    out[i] = t * g;
  }
}

// Cache round trip: the per-group scale and the per-element image.
struct CacheGroupScale {
  float inv;     // multiplier into the quantized domain (fp8, mxfp4)
  float s;       // the group scale (power of two, or the e4m3 value)
  float half_s;  // s / 2: twice-magnitude integers times this are e2m1 * s
};

// float32 round-to-nearest of a / 448 (a >= 0 finite) for quotients of at
// least 2^-126, as a binary64 product with a correctly rounded 1/448 rounded
// once to float32.  With a = M 2^E (M < 2^24), a / 448 = M 2^E / (7 2^6) is an
// exact float32 value of at most 21 significant bits when 7 divides M, and
// otherwise differs from every float32 rounding boundary (a 25-bit odd
// multiple, B) by |M 2^E - 448 B| / 448 >= 2^(f-19) / 448 for a quotient in
// [2^f, 2^(f+1)) (E > f - 16): at least 2^-27.8 relative, against the
// product's 2^-52.  Below 2^-126 the results may differ, which the clamp to
// 2^-126 in cache_scale hides (both sides then give 2^-126).
MXQ_HD float div448_rn_normal(float a) { return (float)((double)a * (1.0 / 448.0)); }

MXQ_HD CacheGroupScale cache_scale(int fmt, float a) {
  CacheGroupScale r;
  if (fmt == FMT_FP8 || fmt == FMT_MXFP4) {
    // a / 448 and a / 6 rounded to nearest, as binary64 products (3 VALU
    // operations instead of a correctly rounded float32 division)
    const float v = fmaxf(fmt == FMT_FP8 ? div448_rn_normal(a) : div6_rn(a), 1.17549435e-38f);
    r.s = pow2_ceil(v);
    r.inv = bitsf((254u - (fbits(r.s) >> 23)) << 23);   // 2^-k, exact
  } else {
    const float u = fminf(fmaxf(div6_rn(a), 0.001953125f), 448.0f);
    e4m3_encode_clamped(u, &r.s);
    r.inv = 0.0f;                                      // nvfp4 divides by s
  }
  r.half_s = r.s * 0.5f;
  return r;
}

// `wide`: float32 input (24-bit significands) for the mxfp4 rounding.
MXQ_HD float cache_qdq1(int fmt, bool wide, float x, const CacheGroupScale& g) {
  const float m = fabsf(x);
  if (fmt == FMT_FP8) {
    const float v = e4m3_round_value(m * g.inv) * g.s;  // exact product
    return copysignf(v, x);                             // sign of zero kept
  }
  uint32_t mag;
  if (fmt == FMT_MXFP4)
    mag = wide ? e2m1_mag_f32(m * g.inv) : e2m1_mag_short(m, g.inv);
  else
    mag = e2m1_mag_f32(m / g.s);                        // correctly rounded
  int32_t t = (int32_t)e2m1_twice_mag(mag);
  t = (fbits(x) >> 31) ? -t : t;                        // -0 -> +0
  return (float)t * g.half_s;                           // exact
}

} // namespace mxq
