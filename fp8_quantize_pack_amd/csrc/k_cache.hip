// k_cache.hip -- cache quantize/dequantize round trip for gfx950.
//
// Method: "nemo_automodel.components.models.deepseek_v41.quantization",
// sections quantize_cache, _CacheQuantization.forward and
// _power_of_two_ceiling.  Channels are grouped in runs of block_size; each
// group gets one scale and every value is replaced by its quantize-then-
// dequantize image, in the input dtype:
//   fp8   : s = pow2ceil(max(amax / 448, 2^-126)),  y = e4m3(x / s) * s
//   mxfp4 : s = pow2ceil(max(amax / 6,   2^-126)),  y = e2m1(x / s) * s
//   nvfp4 : s = e4m3(clamp(amax / 6, 2^-9, 448)),   y = e2m1(x / s) * s
// A last partial group behaves as if padded with zeros.
//
// Fast path (B = block_size a power of two in 8..512, C % 8 == 0, 16-byte
// aligned pointers): B/8 neighbouring lanes own one group (DPP max), LPR lanes
// own one row (rows of up to 512 columns are covered in one step; 64/LPR rows
// per wavefront), the row's groups are padded to whole lane groups so that a
// partial last group simply has idle lanes that contribute 0 to its amax.
// Generic path (anything else): one thread per group, scalar loads.
//
// The e2m1 formats round with the gfx950 scaled fp4 converter (round half
// down through a one-ulp step toward zero and round-to-nearest-even; float32
// inputs and nvfp4 quotients rounded up to 22 significant bits first, which
// changes no decision) and decode with the exact fp4 dequantizer;
// the nvfp4 quotient x / sigma is taken as a binary64 product with 1 / sigma
// to about 2^-52: x has at most 24 significant bits and sigma 4, so x / sigma
// is never a float32 decision boundary and lies at least 2^-29 (relative)
// away from each, far beyond the product's error of about 2^-51.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

struct CacheGeom {
  int64_t rows;
  int64_t cpr;     // chunks per row = C / 8
  int64_t slots;   // chunk slots per row, padded to whole groups
  int lpr;         // lanes per row
  int niter;       // ceil(slots / lpr)
};

// Quantize-dequantize one 8-element chunk (index c, valid if ok) whose group
// spans G neighbouring lanes.  Every lane of the wave calls this together
// (the group amax is a DPP reduction); only valid chunks are stored.
template <int DT, int FMT, int G>
__device__ __forceinline__ void cache_chunk(const Raw8<DT>& raw, bool ok, void* __restrict__ y,
                                            int64_t c) {
  float f[8];
  unpack8<DT>(raw, f);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  a = group_max<G>(a);
  const CacheGroupScale gs = cache_scale(FMT, a);
  float o[8];
  if constexpr (FMT == FMT_FP8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = cache_qdq1(FMT, DT == DT_F32, f[i], gs);
  } else {
    // e2m1 formats: quantize with the scaled fp4 converter (round half
    // down), decode exactly with the fp4 dequantizer.
    float q[8];
    float cvt_scale;
    if constexpr (FMT == FMT_MXFP4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = (DT == DT_F32) ? ceil22(f[i]) : f[i];
      cvt_scale = gs.s;                         // power of two: x / s inside
    } else {
      // sigma: an e4m3 value in [2^-9, 448]; 1 / sigma to about 2^-52
      // (hardware reciprocal and two Newton steps), far inside the 2^-29
      // margin of the quotient (see the header)
      const double rs = recip64((double)gs.s);
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = half_down_for_rne((float)((double)f[i] * rs));
      cvt_scale = 1.0f;
    }
    // A midpoint tie is a float32 subnormal only under an mxfp4 scale
    // below 2^-124; waves holding one take the stochastic-rounding
    // converts, which need no tie-down step.
    const bool tiny = (FMT == FMT_MXFP4) && __any(gs.s < 0x1p-124f);
    const uint32_t w = e2m1_canonical_zeros(
        __builtin_expect(tiny, 0) ? e2m1_pack8_hw(q, cvt_scale)
        : FMT == FMT_MXFP4        ? e2m1_pack8_rne(q, cvt_scale)
                                  : e2m1_pack8_even(q, cvt_scale));
    if constexpr (FMT == FMT_MXFP4 && DT == DT_BF16) {
      if (ok) stream_st(e2m1_unpack8_bf16_hw(w, gs.s), reinterpret_cast<u32x4*>(y) + c);
      return;
    } else if constexpr (FMT == FMT_MXFP4) {
      e2m1_unpack8_f32_hw(w, gs.s, o);
    } else {
      e2m1_unpack8_f32_hw(w, 1.0f, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = o[i] * gs.s;  // exact
    }
  }
  if (ok) st8<DT>(y, c, o);
}

// Row groups in flight per wave (their loads are issued together).  One,
// with two row groups per wave in turn, measured fastest on the 32 to 128 MiB
// KV tensors (graphs of back-to-back launches over cold inputs): fp8 block
// 32 [16, 8192, 512] 43.4 us against 46.4 with two in flight, mxfp4 block 32
// [16, 8192, 128] 12.9 against 13.5 (the plain copy of the same bytes takes
// 12.2 to 12.9), nvfp4 block 16 [16, 2048, 512] unchanged at 13.7; four in
// flight was slower for all three.
#ifndef MXQ_CACHE_UNROLL
#define MXQ_CACHE_UNROLL 1
#endif
constexpr int kCacheUnroll = MXQ_CACHE_UNROLL;
#ifndef MXQ_CACHE_GROUPS_PER_WAVE
#define MXQ_CACHE_GROUPS_PER_WAVE (2 * MXQ_CACHE_UNROLL)
#endif
constexpr int64_t kCacheGroupsPerWave = MXQ_CACHE_GROUPS_PER_WAVE;

template <int DT, int FMT, int B>
__global__ __launch_bounds__(256) void k_cache_qdq(const void* __restrict__ x,
                                                   void* __restrict__ y,
                                                   CacheGeom geo) {
  constexpr int G = B / 8;   // lanes per group
  constexpr int U = kCacheUnroll;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (geo.lpr - 1);
  const int rows_per_wave = kWave / geo.lpr;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t ngroups = (geo.rows + rows_per_wave - 1) / rows_per_wave;
  for (int64_t wg0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       wg0 < ngroups; wg0 += nwaves * U) {
    for (int it = 0; it < geo.niter; ++it) {
      const int64_t j = sub + (int64_t)it * geo.lpr;
      Raw8<DT> r[U];
      bool ok[U];
      int64_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t row = (wg0 + u * nwaves) * rows_per_wave + lane / geo.lpr;
        ok[u] = row < geo.rows && j < geo.cpr;
        c[u] = row * geo.cpr + j;
        r[u] = ok[u] ? ld8<DT>(x, c[u]) : zero8<DT>();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) cache_chunk<DT, FMT, G>(r[u], ok[u], y, c[u]);
    }
  }
}

template <int DT>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (DT == DT_F32) return reinterpret_cast<const float*>(p)[i];
  const uint32_t h = reinterpret_cast<const uint16_t*>(p)[i];
  if constexpr (DT == DT_BF16) return bitsf(h << 16);
  return f16_to_f32(h);
}

template <int DT>
__device__ __forceinline__ void st1(void* p, int64_t i, float v) {
  if constexpr (DT == DT_F32) {
    reinterpret_cast<float*>(p)[i] = v;
  } else if constexpr (DT == DT_BF16) {
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(f16x2_rne(v, 0.0f) & 0xFFFFu);
  }
}

template <int DT, int FMT>
__global__ __launch_bounds__(256) void k_cache_qdq_generic(
    const void* __restrict__ x, void* __restrict__ y, int64_t rows, int64_t C,
    int64_t B, int64_t gpr) {
  const int64_t ngroups = rows * gpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < ngroups; gi += stride) {
    const int64_t row = gi / gpr, grp = gi - row * gpr;
    const int64_t c0 = grp * B;
    const int64_t n = (C - c0 < B) ? C - c0 : B;
    const int64_t base = row * C + c0;
    float a = 0.0f;
    for (int64_t k = 0; k < n; ++k) a = fmaxf(a, fabsf(ld1<DT>(x, base + k)));
    const CacheGroupScale gs = cache_scale(FMT, a);
    for (int64_t k = 0; k < n; ++k) st1<DT>(y, base + k, cache_qdq1(FMT, DT == DT_F32, ld1<DT>(x, base + k), gs));
  }
}

template <int DT, int FMT>
static hipError_t launch_fast(const void* x, void* y, const CacheGeom& geo,
                              int B, hipStream_t s) {
  const int64_t rows_per_wave = kWave / geo.lpr;
  const int64_t waves = (geo.rows + rows_per_wave - 1) / rows_per_wave;
  // about kCacheGroupsPerWave row groups per wave (two steps of kCacheUnroll):
  // measured best on 32 MiB to 128 MiB tensors over fixed grid caps, which
  // favoured small tensors or large ones but not both
  int64_t b = (waves + 4 * kCacheGroupsPerWave - 1) / (4 * kCacheGroupsPerWave);
  b = b < kCacheGridBlocks ? kCacheGridBlocks : b;
  b = b < (waves + 3) / 4 ? b : (waves + 3) / 4;
  b = b < kMaxGridBlocks ? (b > 0 ? b : 1) : kMaxGridBlocks;
  const dim3 grid((unsigned)b), block(256);
  switch (B) {
    case 8: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 8>), grid, block, 0, s, x, y, geo); break;
    case 16: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 16>), grid, block, 0, s, x, y, geo); break;
    case 32: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 32>), grid, block, 0, s, x, y, geo); break;
    case 64: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 64>), grid, block, 0, s, x, y, geo); break;
    case 128: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 128>), grid, block, 0, s, x, y, geo); break;
    case 256: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 256>), grid, block, 0, s, x, y, geo); break;
    default: hipLaunchKernelGGL((k_cache_qdq<DT, FMT, 512>), grid, block, 0, s, x, y, geo); break;
  }
  return hipGetLastError();
}

template <int DT, int FMT>
static hipError_t launch_one(const void* x, void* y, int64_t rows, int64_t C,
                             int B, hipStream_t s) {
  const bool pow2 = B >= 8 && B <= 512 && (B & (B - 1)) == 0;
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
  if (pow2 && aligned && C % 8 == 0) {
    CacheGeom geo;
    geo.rows = rows;
    geo.cpr = C / 8;
    const int64_t gpr = (C + B - 1) / B;
    geo.slots = gpr * (B / 8);
    int lpr = B / 8 > 2 ? B / 8 : 2;
    while (lpr < 64 && lpr < geo.slots) lpr <<= 1;
    geo.lpr = lpr;
    geo.niter = (int)((geo.slots + lpr - 1) / lpr);
    return launch_fast<DT, FMT>(x, y, geo, B, s);
  }
  const int64_t gpr = (C + B - 1) / B;
  const int64_t ngroups = rows * gpr;
  int64_t b = (ngroups + 255) / 256;
  const dim3 grid((unsigned)(b < 4096 ? b : 4096)), block(256);
  hipLaunchKernelGGL((k_cache_qdq_generic<DT, FMT>), grid, block, 0, s, x, y, rows, C, (int64_t)B, gpr);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const void* x, void* y, int64_t rows, int64_t C,
                            int fmt, int B, hipStream_t s) {
  switch (fmt) {
    case FMT_FP8: return launch_one<DT, FMT_FP8>(x, y, rows, C, B, s);
    case FMT_MXFP4: return launch_one<DT, FMT_MXFP4>(x, y, rows, C, B, s);
    default: return launch_one<DT, FMT_NVFP4>(x, y, rows, C, B, s);
  }
}

hipError_t launch_cache_qdq(const void* x, void* y, int dt, int64_t rows,
                            int64_t C, int fmt, int block_size, hipStream_t s) {
  switch (dt) {
    case DT_F32: return launch_dt<DT_F32>(x, y, rows, C, fmt, block_size, s);
    case DT_BF16: return launch_dt<DT_BF16>(x, y, rows, C, fmt, block_size, s);
    default: return launch_dt<DT_F16>(x, y, rows, C, fmt, block_size, s);
  }
}

} // namespace mxq
