// k_fp4_static.hip -- static two-level FP4 fake quantization for gfx950.
//
// Method: Model-Optimizer tensor_quantizer.py, StaticBlockScaleQuantizer:
// _block_scale_from_amax with FP8 (e4m3) block scales, _amax_to_scale,
// _clamp_scale, _FP8_E4M3_MIN_POSITIVE, and the division / fp4 cast /
// multiplication of _fake_quantize with one amax for the pre and the post
// scale.  Inputs: x [rows, K], one float32 amax per block of B consecutive
// columns ([rows, K / B]), one float32 global amax G (device memory).
// float32 arithmetic, left to right:
//   P  = G / 6,  replaced by 1e-8 when <= 1e-8          (per-tensor scale)
//   m  = c * P,  c = float32(2^-9 / 448)                (scale floor)
//   s  = a / 6,  replaced by m when <= m                (block scale)
//   t  = 448 / P;  sigma = e4m3(s * t);  s' = sigma / t (e4m3 fake quant)
//   y  = RN_dtype(e2m1(x / s') * s')
// with e2m1 rounding to nearest, ties to the smaller magnitude, and the sign
// of x on the code.
//
// Work layout: 8-element chunks, one chunk per lane per step, a wavefront
// tile of kUnroll x 64 consecutive chunks (contiguous loads and stores over
// the wave); B / 8 neighbouring lanes share a block and each of them derives
// the block's scale (a broadcast load of the same amax word, a handful of
// scalar-like float operations per 8 elements).
//
// Exactness.  s * t lies in [2^-9 (1 - 2^-21), 448 (1 + 2^-22)] or above
// (a block amax beyond G); clamping to [2^-9, 448] before the hardware e4m3
// converter (exact there) gives its round-to-nearest-even value with
// saturation.  The quotient x / s' is taken as the binary64 product with
// 1 / s' (hardware reciprocal, two Newton steps) rounded to float32: x has at
// most 24 significant bits and s' 24, so the e2m1 decisions of that product
// equal those of the float32 quotient (see nvfp4_quant8 in mxq_device.h);
// then the round-to-nearest-even converter, made to round half down by a
// one-unit step on the operands that need it (half_down_for_rne).
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

#ifndef MXQ_ST_UNROLL
#define MXQ_ST_UNROLL 2
#endif
constexpr int kStUnroll = MXQ_ST_UNROLL;
constexpr int kStTileChunks = kStUnroll * kWave;
constexpr int kStWaves = 4;

// float32(2^-9 / 448): the smallest e4m3 value over E4M3_MAX.
constexpr float kFp8FloorRatio = (float)(0x1p-9 / 448.0);

struct StaticTensorScale {
  float m;      // block-scale floor
  float t;      // 448 / P
};

__device__ __forceinline__ StaticTensorScale static_tensor_scale(float G) {
  float P = G / 6.0f;
  P = (P <= 1e-8f) ? 1e-8f : P;
  StaticTensorScale r;
  r.m = kFp8FloorRatio * P;
  r.t = 448.0f / P;
  return r;
}

// Dequantization-side block scale s' of a block with amax a.
__device__ __forceinline__ float static_block_scale(float a, const StaticTensorScale& ts) {
  float s = a / 6.0f;
  s = (s <= ts.m) ? ts.m : s;
  const float v = __builtin_amdgcn_fmed3f(s * ts.t, 0x1p-9f, 448.0f);
  float sigma;
  (void)e4m3_encode_clamped(v, &sigma);
  return sigma / ts.t;
}

template <int DT>
__global__ __launch_bounds__(64 * kStWaves) void k_fp4_static_qdq(
    const void* __restrict__ x, const float* __restrict__ block_amax,
    const float* __restrict__ global_amax, void* __restrict__ y,
    int64_t nchunks, int64_t ntiles, int cpb_log2) {
  const int lane = threadIdx.x & 63;
  const StaticTensorScale ts = static_tensor_scale(*global_amax);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < ntiles; t += nwaves) {
    const int64_t c0 = t * kStTileChunks + lane;
    Raw8<DT> r[kStUnroll];
    float a[kStUnroll];
#pragma unroll
    for (int u = 0; u < kStUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const bool ok = c < nchunks;
      r[u] = ld8_wave<DT>(x, c - lane, nchunks, lane);
      a[u] = ok ? block_amax[c >> cpb_log2] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kStUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const float sp = static_block_scale(a[u], ts);
      const double rs = recip64((double)sp);
      float f[8];
      unpack8<DT>(r[u], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = half_down_for_rne((float)((double)f[i] * rs));
      const uint32_t w = e2m1_canonical_zeros(e2m1_pack8_even(f, 1.0f));
      float o[8];
      e2m1_unpack8_f32_hw(w, 1.0f, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = o[i] * sp;   // one float32 rounding
      st8_wave<DT>(y, c - lane, nchunks, lane, o);
    }
  }
}

hipError_t launch_fp4_static_qdq(const void* x, int dt, int64_t rows, int64_t K,
                                 int block_size, const float* block_amax,
                                 const float* global_amax, void* y, hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t ntiles = (nchunks + kStTileChunks - 1) / kStTileChunks;
  int cpb_log2 = 0;
  while ((8 << cpb_log2) < block_size) ++cpb_log2;
// four tiles per wave: 370-378 us against 399 us for one tile per wave on a
// bf16 [36, 2048, 7168] round trip (the other streaming kernels are fastest
// at one unit per wave)
#ifndef MXQ_ST_UPW
#define MXQ_ST_UPW 4
#endif
  int64_t b = (ntiles + kStWaves * MXQ_ST_UPW - 1) / (kStWaves * MXQ_ST_UPW);
  b = b < kMaxGridBlocks ? (b > 0 ? b : 1) : kMaxGridBlocks;
  const dim3 grid((unsigned)b), block(64 * kStWaves);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_fp4_static_qdq<DT_F32>, grid, block, 0, s, x, block_amax, global_amax, y, nchunks, ntiles, cpb_log2); break;
    case DT_BF16: hipLaunchKernelGGL(k_fp4_static_qdq<DT_BF16>, grid, block, 0, s, x, block_amax, global_amax, y, nchunks, ntiles, cpb_log2); break;
    default: hipLaunchKernelGGL(k_fp4_static_qdq<DT_F16>, grid, block, 0, s, x, block_amax, global_amax, y, nchunks, ntiles, cpb_log2); break;
  }
  return hipGetLastError();
}

} // namespace mxq
