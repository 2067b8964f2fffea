// mxq_kernel_common.h -- device-only building blocks shared by the libmxq
// kernels: 16-byte vector loads and stores of 8-element chunks, and max
// reductions across small lane groups of a 64-wide wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.h"

namespace mxq {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ chunks
// A "chunk" is 8 consecutive elements.  16-bit inputs move one 16-byte vector
// per chunk, float32 inputs two.  Chunk c of a tensor starts at element 8c;
// every base pointer is 16-byte aligned (checked by the host layer).

template <int DT> struct Raw8;
template <> struct Raw8<DT_BF16> { u32x4 v; };
template <> struct Raw8<DT_F16> { u32x4 v; };
template <> struct Raw8<DT_F32> { u32x4 a, b; };

template <int DT>
__device__ __forceinline__ Raw8<DT> ld8(const void* base, int64_t chunk);

template <>
__device__ __forceinline__ Raw8<DT_BF16> ld8<DT_BF16>(const void* base, int64_t c) {
  return Raw8<DT_BF16>{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + c)};
}
template <>
__device__ __forceinline__ Raw8<DT_F16> ld8<DT_F16>(const void* base, int64_t c) {
  return Raw8<DT_F16>{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + c)};
}
template <>
__device__ __forceinline__ Raw8<DT_F32> ld8<DT_F32>(const void* base, int64_t c) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base) + 2 * c;
  return Raw8<DT_F32>{__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1)};
}

template <int DT>
__device__ __forceinline__ Raw8<DT> zero8() {
  Raw8<DT> r;
  memset(&r, 0, sizeof(r));
  return r;
}

__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = bitsf(w << 16);
  hi = bitsf(w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack_f16x2(uint32_t w, float& lo, float& hi) {
  lo = f16_to_f32(w & 0xFFFFu);
  hi = f16_to_f32(w >> 16);
}

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float f[8]);

template <>
__device__ __forceinline__ void unpack8<DT_BF16>(const Raw8<DT_BF16>& r, float f[8]) {
  unpack_bf16x2(r.v.x, f[0], f[1]);
  unpack_bf16x2(r.v.y, f[2], f[3]);
  unpack_bf16x2(r.v.z, f[4], f[5]);
  unpack_bf16x2(r.v.w, f[6], f[7]);
}
template <>
__device__ __forceinline__ void unpack8<DT_F16>(const Raw8<DT_F16>& r, float f[8]) {
  unpack_f16x2(r.v.x, f[0], f[1]);
  unpack_f16x2(r.v.y, f[2], f[3]);
  unpack_f16x2(r.v.z, f[4], f[5]);
  unpack_f16x2(r.v.w, f[6], f[7]);
}
template <>
__device__ __forceinline__ void unpack8<DT_F32>(const Raw8<DT_F32>& r, float f[8]) {
  f[0] = bitsf(r.a.x); f[1] = bitsf(r.a.y); f[2] = bitsf(r.a.z); f[3] = bitsf(r.a.w);
  f[4] = bitsf(r.b.x); f[5] = bitsf(r.b.y); f[6] = bitsf(r.b.z); f[7] = bitsf(r.b.w);
}

// Round 8 float32 values to DT (round to nearest even) and store them.
template <int DT>
__device__ __forceinline__ void st8(void* base, int64_t c, const float f[8]);

template <>
__device__ __forceinline__ void st8<DT_F32>(void* base, int64_t c, const float f[8]) {
  u32x4* p = reinterpret_cast<u32x4*>(base) + 2 * c;
  __builtin_nontemporal_store(u32x4{fbits(f[0]), fbits(f[1]), fbits(f[2]), fbits(f[3])}, p);
  __builtin_nontemporal_store(u32x4{fbits(f[4]), fbits(f[5]), fbits(f[6]), fbits(f[7])}, p + 1);
}
template <>
__device__ __forceinline__ void st8<DT_BF16>(void* base, int64_t c, const float f[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = f32_to_bf16_rne(f[2 * i]) | (f32_to_bf16_rne(f[2 * i + 1]) << 16);
  __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                              reinterpret_cast<u32x4*>(base) + c);
}
template <>
__device__ __forceinline__ void st8<DT_F16>(void* base, int64_t c, const float f[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = f32_to_f16_rne(f[2 * i]) | (f32_to_f16_rne(f[2 * i + 1]) << 16);
  __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                              reinterpret_cast<u32x4*>(base) + c);
}

// ------------------------------------------------------------------ reductions
// Max across aligned groups of G consecutive lanes (G a power of two <= 64),
// the result replicated in every lane of the group.  Values are non-negative
// floats, so the unsigned integer maximum of the bit patterns is the float
// maximum.  All lanes of a group must be active.  Lane exchange uses DPP
// inside rows of 16 (quad permutes, then the half-row and row mirrors, which
// pair up groups whose members already agree) and LDS permutes above that.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
  uint32_t v = fbits(x);
  if constexpr (G >= 2) v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  if constexpr (G >= 16) v = max(v, dpp_u32<0x140>(v));  // row_mirror
  if constexpr (G >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (G >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return bitsf(v);
}

// Same for a group size known only at run time (a power of two <= 64).
__device__ __forceinline__ float group_max_rt(float x, int G) {
  uint32_t v = fbits(x);
  for (int m = 1; m < G; m <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
  return bitsf(v);
}

} // namespace mxq
