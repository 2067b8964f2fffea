// k_mxfp8.hip -- MXFP8 (e4m3 elements, e8m0 block scales, block 32)
// quantize and dequantize kernels for gfx950.
//
// Method: Model-Optimizer tensor_quantizer.py, TensorQuantizer._real_quantize,
// the MX branch with e4m3 elements (block size 32).  The pages name the MXFP8
// tensor class without printing its arithmetic; the block scale is the
// power-of-two rule the pages print for fp8 blocks
// ("nemo_automodel.components.models.deepseek_v41.quantization",
// quantize_cache and _power_of_two_ceiling):
//   s    = pow2ceil(max(amax / 448, 2^-126)),  stored as the e8m0 byte of s
//   code = e4m3(x / s)    (round to nearest even; |x / s| <= 448 by
//                          construction; the sign bit is the input's)
//   y    = e4m3value(code) * 2^(b - 127) in float32, one rounding to dtype.
//
// Layout of the work is that of the MXFP4 kernels: 8-element chunks, a
// wavefront tile of kUnroll x 64 chunks with lane l owning chunk
// tile * kUnroll * 64 + u * 64 + l, four lanes per 32-element block (their
// maxima combined with two DPP quad permutes).  Codes leave as 8 bytes per
// lane and instruction, contiguous over the wave.
//
// The e4m3 encode uses the gfx950 fp8 converter (v_cvt_pk_fp8_f32) only on
// magnitudes clamped to [2^-9, 448], where it rounds to nearest even exactly
// (measured over every float32 of that range).  Magnitudes below 2^-9 have
// two candidates, 0 and 2^-9: those above 2^-10 round to 2^-9 (which the
// clamp gives), the others to zero (masked afterwards); sign bits are copied
// from the input.  x / s is the exact product x * 2^-k (below 2^-126 it may
// lose bits, far below any e4m3 decision).
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

#ifndef MXQ_MX8_UNROLL
#define MXQ_MX8_UNROLL 2
#endif
constexpr int kMx8Unroll = MXQ_MX8_UNROLL;
constexpr int kMx8TileChunks = kMx8Unroll * kWave;
constexpr int kMx8Waves = 4;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// e8m0 byte of the MXFP8 block scale pow2ceil(max(amax / 448, 2^-126)):
// the biased exponent of that power of two (1 .. 247 for finite amax).
__device__ __forceinline__ uint32_t mxfp8_scale_byte(float amax) {
  const float v = fmaxf(amax / 448.0f, 1.17549435e-38f);
  return fbits(pow2_ceil(v)) >> 23;
}

// Two e4m3 codes (bytes 0 and 1) of magnitudes m0, m1 (already divided by the
// block scale, each <= 448 up to one rounding) with sign bits s0, s1 (0/1).
__device__ __forceinline__ uint32_t e4m3_pair(float m0, float m1, uint32_t s0, uint32_t s1) {
  const float c0 = __builtin_amdgcn_fmed3f(m0, 0x1p-9f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(m1, 0x1p-9f, 448.0f);
  uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
  const uint32_t keep = (m0 > 0x1p-10f ? 0x00FFu : 0u) | (m1 > 0x1p-10f ? 0xFF00u : 0u);
  return (h & keep) | (s0 << 7) | (s1 << 15);
}

// 8 elements -> 8 e4m3 codes (element i in byte i of the pair of dwords).
__device__ __forceinline__ u32x2 e4m3_codes8(const float f[8], float inv) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = e4m3_pair(fabsf(f[2 * i]) * inv, fabsf(f[2 * i + 1]) * inv,
                     fbits(f[2 * i]) >> 31, fbits(f[2 * i + 1]) >> 31);
  return u32x2{p[0] | (p[1] << 16), p[2] | (p[3] << 16)};
}

template <int DT>
__global__ __launch_bounds__(64 * kMx8Waves) void k_mxfp8_quant(
    const void* __restrict__ x, u32x2* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t nchunks, int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < ntiles; t += nwaves) {
    const int64_t c0 = t * kMx8TileChunks + lane;
    Raw8<DT> r[kMx8Unroll];
#pragma unroll
    for (int u = 0; u < kMx8Unroll; ++u) {
      const int64_t c = c0 + u * kWave;
      r[u] = ld8_wave<DT>(x, c - lane, nchunks, lane);
    }
#pragma unroll
    for (int u = 0; u < kMx8Unroll; ++u) {
      const int64_t c = c0 + u * kWave;
      float f[8];
      unpack8<DT>(r[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
      a = group_max<4>(a);                       // amax of the 32-column block
      const uint32_t sb = mxfp8_scale_byte(a);
      const float inv = bitsf((254u - sb) << 23);  // 1 / s, exact
      const u32x2 w = e4m3_codes8(f, inv);
      if (c < nchunks) {
        stream_st(w, codes + c);
        if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)sb;
      }
    }
  }
}


template <int DT>
__global__ __launch_bounds__(64 * kMx8Waves) void k_mxfp8_dequant(
    const u32x2* __restrict__ codes, const uint8_t* __restrict__ scales,
    void* __restrict__ y, int64_t nchunks, int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < ntiles; t += nwaves) {
    const int64_t c0 = t * kMx8TileChunks + lane;
    u32x2 w[kMx8Unroll];
    uint32_t sb[kMx8Unroll];
#pragma unroll
    for (int u = 0; u < kMx8Unroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const bool ok = c < nchunks;
      w[u] = ok ? stream_ld(codes + c) : u32x2{0u, 0u};
      sb[u] = ok ? (uint32_t)scales[c >> 2] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kMx8Unroll; ++u) {
      const int64_t c = c0 + u * kWave;
      // e4m3 * 2^(b - 127) through the scaled fp8 converter, two codes per
      // instruction: the product of a 4-bit significand at or above 2^-9 and a
      // power of two at or above 2^-127 is an exact float32 (lowest bit >=
      // 2^-136), so the converter's result is exact; byte 255 is NaN.
      const float sc = e8m0_as_scale(sb[u]);
      float f[8];
      f32x2 v;
      v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[u].x, sc, false); f[0] = v.x; f[1] = v.y;
      v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[u].x, sc, true);  f[2] = v.x; f[3] = v.y;
      v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[u].y, sc, false); f[4] = v.x; f[5] = v.y;
      v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[u].y, sc, true);  f[6] = v.x; f[7] = v.y;
      if (sb[u] == 255u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = bitsf(0x7FC00000u);
      }
      st8_wave<DT>(y, c - lane, nchunks, lane, f);
    }
  }
}

static int mx8_grid(int64_t ntiles) {
#ifndef MXQ_MX8_UPW
#define MXQ_MX8_UPW MXQ_UNITS_PER_WAVE
#endif
  int64_t b = (ntiles + kMx8Waves * MXQ_MX8_UPW - 1) / (kMx8Waves * MXQ_MX8_UPW);
  return (int)(b < kMaxGridBlocks ? (b > 0 ? b : 1) : kMaxGridBlocks);
}

hipError_t launch_mxfp8_quant(const void* x, int dt, int64_t rows, int64_t K,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t ntiles = (nchunks + kMx8TileChunks - 1) / kMx8TileChunks;
  const dim3 grid(mx8_grid(ntiles)), block(64 * kMx8Waves);
  u32x2* c = reinterpret_cast<u32x2*>(codes);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_mxfp8_quant<DT_F32>, grid, block, 0, s, x, c, scales, nchunks, ntiles); break;
    case DT_BF16: hipLaunchKernelGGL(k_mxfp8_quant<DT_BF16>, grid, block, 0, s, x, c, scales, nchunks, ntiles); break;
    default: hipLaunchKernelGGL(k_mxfp8_quant<DT_F16>, grid, block, 0, s, x, c, scales, nchunks, ntiles); break;
  }
  return hipGetLastError();
}

hipError_t launch_mxfp8_dequant(const uint8_t* codes, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y, int dt,
                                hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t ntiles = (nchunks + kMx8TileChunks - 1) / kMx8TileChunks;
  const dim3 grid(mx8_grid(ntiles)), block(64 * kMx8Waves);
  const u32x2* c = reinterpret_cast<const u32x2*>(codes);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_mxfp8_dequant<DT_F32>, grid, block, 0, s, c, scales, y, nchunks, ntiles); break;
    case DT_BF16: hipLaunchKernelGGL(k_mxfp8_dequant<DT_BF16>, grid, block, 0, s, c, scales, y, nchunks, ntiles); break;
    default: hipLaunchKernelGGL(k_mxfp8_dequant<DT_F16>, grid, block, 0, s, c, scales, y, nchunks, ntiles); break;
  }
  return hipGetLastError();
}

} // namespace mxq
