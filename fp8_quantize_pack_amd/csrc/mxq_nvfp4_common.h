// mxq_nvfp4_common.h -- device building blocks of the NVFP4 quantizers
// ("nemo_automodel.components.quantization.nvfp4", quantize_nvfp4): block
// maxima taken on raw 16-bit patterns, the block scale and the binary64
// reciprocal of its divisor, the codes of one 8-element chunk, and the lane
// pair exchange of the 16-element blocks that two lanes share.
#pragma once

#include "mxq_kernel_common.h"

namespace mxq {

constexpr float kGlobalDiv = 2688.0f;         // E2M1_MAX * E4M3_MAX
constexpr double kHugeRecip = 0x1p800;        // stands in for 1 / 0 (see below)

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Magnitude maximum of 8 elements as a bit pattern that orders like the
// value: bfloat16 and float16 magnitudes order like their 15-bit patterns, so
// the maximum is taken on the raw data with packed 16-bit integer maxima (two
// elements per instruction); float32 uses the float maximum.
template <int DT>
__device__ __forceinline__ uint32_t amax8_bits(const Raw8<DT>& r) {
  if constexpr (DT == DT_F32) {
    float f[8];
    unpack8<DT>(r, f);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
    return fbits(a);
  } else {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 4; ++i)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return m.x > m.y ? m.x : m.y;
  }
}

template <int DT>
__device__ __forceinline__ float amax_from_bits(uint32_t b) {
  if constexpr (DT == DT_F32) return bitsf(b);
  else if constexpr (DT == DT_BF16) return bitsf(b << 16);
  else return f16_to_f32(b);
}

// Scale byte, and |1 / den| for den = e4m3(a / 6 / g) * g, of a block with
// amax `a`.  1 / den is correctly rounded in binary64.  den == 0 (only with
// g == 0 or a tiny given g) makes every non-zero element saturate and keeps
// 0 / 0 at code 0, as the float32 quotient would (inf -> code 7, NaN -> code
// 0); den == inf gives 0 (every finite element to code 0).  The magnitude is
// taken because a code's sign is its element's, whatever the sign of g.
constexpr int kClassZeroInf = (1 << 2) | (1 << 5) | (1 << 6) | (1 << 9);   // -inf -0 +0 +inf

__device__ __forceinline__ double nv_block_recip(float a, float g, double rg, uint32_t& sb) {
  float den;
  sb = nvfp4_block_scale(a, g, rg, &den);
  double r = recip64((double)den);
  if (__builtin_amdgcn_classf(den, kClassZeroInf)) r = (den == 0.0f) ? kHugeRecip : 0.0;
  return fabs(r);
}

// The same for a row scale g in [2^-100, 2^100]: den = sigma * g then lies in
// [2^-109, 2^109], finite, non-zero and positive, so none of the cases above
// arises.
__device__ __forceinline__ double nv_block_recip_normal(float a, float g, double rg, uint32_t& sb) {
  float den;
  sb = nvfp4_block_scale(a, g, rg, &den);
  return recip64((double)den);
}

__device__ __forceinline__ bool nv_g_normal(float g) {
  return g >= 0x1p-100f && g <= 0x1p100f;      // false for NaN
}

// The float32 quotient x / den of one element, rounded to nearest, then made
// ready for the round-to-nearest-even converter (e2m1_pack8_even) to round it
// half down.
__device__ __forceinline__ float nv_quotient(float x, double rden) {
  return half_down_for_rne((float)((double)x * rden));
}

// 8 codes (one dword) of a chunk, given 1 / den of its block.  This form --
// the quotient rounded up to 22 significant bits, then the tie-down multiply
// inside e2m1_pack8_rne -- takes one VALU instruction per element more than
// nv_quotient + e2m1_pack8_even and gives the same codes, yet the row
// quantizer ran 2-4% faster with it on the MoE sweep (interleaved A/B runs of
// both builds); the cache, static and KV kernels run the other form.
template <int DT>
__device__ __forceinline__ uint32_t nv_codes8(const Raw8<DT>& r, double rden) {
  float f[8];
  unpack8<DT>(r, f);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = ceil22((float)((double)f[i] * rden));
  return e2m1_pack8_rne(f, 1.0f);      // quotients near a midpoint are normal
}

// Lane exchanges within each pair of lanes (DPP quad_perm; every lane has a
// source): QP = kQuadSwap gives the partner's value (lane L ^ 1), kQuadEven
// the even lane's (L & ~1), kQuadOdd the odd lane's (L | 1).
constexpr int kQuadSwap = 0xB1;     // [1,0,3,2]
constexpr int kQuadEven = 0xA0;     // [0,0,2,2]
constexpr int kQuadOdd = 0xF5;      // [1,1,3,3]

template <int QP>
__device__ __forceinline__ uint32_t pair_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, QP, 0xF, 0xF, true);
}
template <int QP>
__device__ __forceinline__ double pair_lane(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  const uint64_t lo = pair_lane<QP>((uint32_t)u), hi = pair_lane<QP>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) { return pair_lane<kQuadSwap>(v); }

} // namespace mxq
