// k_mxfp4.hip -- MXFP4 quantize-pack and dequantize kernels for gfx950.
//
// Method: "nemo_automodel.components.quantization.mxfp4", sections
// quantize_mxfp4 / dequantize_mxfp4 / Data.  Per 32-column block: scale
// 2^(floor(log2 amax) - 2) stored as an e8m0 byte, elements divided by it and
// rounded to the nearest e2m1 value (ties to the smaller magnitude), two codes
// per byte with the even column in the low nibble.
//
// Layout of the work.  Blocks never straddle rows (K % 32 == 0), so the tensor
// is a flat run of 8-element chunks.  A wavefront tile is kUnroll x 64 chunks:
// in step u lane l owns chunk tile*kUnroll*64 + u*64 + l, so every vector load and
// store instruction of the wave touches one contiguous 1 KiB (bf16 input) or
// 256 B (packed) range, and the 4 lanes of a quad own one 32-column block
// (their amax is combined with two DPP quad permutes).  With kUnroll = 2 a
// tile covers 32 blocks (1024 elements) and 32 contiguous scale bytes: small
// tiles and many workgroups balance best across the chip.
//
// Rounding and packing use the gfx950 scaled fp4 converts (see
// mxq_kernel_common.h): the quantizer divides by the block's power-of-two
// scale and, after a one-ulp step toward zero, rounds to nearest even --
// together round half down; the dequantizer multiplies back exactly.
// float32 inputs are first rounded up to 22 significant bits (ceil22), which
// changes no e2m1 decision; bfloat16 and float16 values already fit.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

#ifndef MXQ_MX_UNROLL
#define MXQ_MX_UNROLL 2
#endif
constexpr int kUnroll = MXQ_MX_UNROLL;
constexpr int kTileChunks = kUnroll * kWave;   // chunks per wavefront tile
#ifndef MXQ_MX_WAVES
#define MXQ_MX_WAVES 4
#endif
constexpr int kMxWaves = MXQ_MX_WAVES;         // waves per workgroup

// Both kernels touch the scale array with streaming (non-temporal) accesses,
// like every other stream of the codec.  Ordinary cached scale accesses were
// as fast for these kernels, but they left the chip in a state that slowed
// the NVFP4 quantizer launched after them for the whole of its run (on the
// MoE sweep 201-204 us per launch instead of 190-194; after the
// dequantizer, its place in the step; neither the memory footprint nor
// plain copy, read or fill passes did that).  With streaming scale accesses
// the quantizer costs 0.3% more, the dequantizer 1.3% more (its 16-byte
// scale loads cover a whole tile), and the step as a whole runs 1.1% faster.
template <int DT>
__global__ __launch_bounds__(64 * kMxWaves) void k_mxfp4_quant(
    const void* __restrict__ x, uint32_t* __restrict__ packed,
    uint8_t* __restrict__ scales, int64_t nchunks, int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < ntiles; t += nwaves) {
    const int64_t c0 = t * kTileChunks + lane;
    Raw8<DT> r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      r[u] = ld8_wave<DT>(x, c - lane, nchunks, lane);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      float f[8];
      unpack8<DT>(r[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
      a = group_max<4>(a);                      // amax of the 32-column block
      const uint32_t sb = mxfp4_scale_byte(a);  // e8m0 byte
      if constexpr (DT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = ceil22(f[i]);
      }
      // Scale bytes below 3 can put a midpoint tie on a float32 subnormal,
      // which the tie-down multiply cannot move: such waves (amax < 2^-121)
      // take the stochastic-rounding converts.
      const uint32_t word = __builtin_expect(__any(sb < 3u), 0)
                                ? e2m1_pack8_hw(f, e8m0_as_scale(sb))
                                : e2m1_pack8_rne(f, e8m0_as_scale(sb));
      if (c < nchunks) {
        stream_st(word, packed + c);
        // streaming store of the scale byte, like the codes (see kernel note)
        if ((lane & 3) == 0) __builtin_nontemporal_store((uint8_t)sb, scales + (c >> 2));
      }
    }
  }
}

template <int DT>
__global__ __launch_bounds__(64 * kMxWaves) void k_mxfp4_dequant(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    void* __restrict__ y, int64_t nchunks, int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < ntiles; t += nwaves) {
    const int64_t c0 = t * kTileChunks + lane;
    uint32_t w[kUnroll], sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const bool ok = c < nchunks;
      w[u] = ok ? stream_ld(packed + c) : 0u;
    }
    {
      // The tile's kUnroll * 16 scale bytes: one streaming 16-byte load per
      // unroll step (lanes 0 .. kUnroll-1), handed to every lane by readlanes
      // (lane l of step u needs byte 16 u + l / 4).  Partial tiles and
      // unaligned scale arrays load single bytes.  See the kernel note on
      // why the scale accesses stream.
      const int64_t sbase = t * (kTileChunks / 4);
      const bool full = ((reinterpret_cast<uintptr_t>(scales) & 15) == 0) && (t + 1) * kTileChunks <= nchunks;
      if (full) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (lane < kUnroll) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(scales + sbase) + lane);
        const int q = lane >> 4, sh = ((lane >> 2) & 3) * 8;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t d0 = __builtin_amdgcn_readlane(v.x, u), d1 = __builtin_amdgcn_readlane(v.y, u);
          const uint32_t d2 = __builtin_amdgcn_readlane(v.z, u), d3 = __builtin_amdgcn_readlane(v.w, u);
          const uint32_t d = q == 0 ? d0 : (q == 1 ? d1 : (q == 2 ? d2 : d3));
          sb[u] = (d >> sh) & 0xFFu;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int64_t c = c0 + u * kWave;
          sb[u] = c < nchunks ? (uint32_t)scales[c >> 2] : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const uint32_t wc = e2m1_canonical_zeros(w[u]);
      const float scale = e8m0_as_scale(sb[u]);
      const bool nan_scale = sb[u] == 255u;               // e8m0 NaN
      if constexpr (DT == DT_BF16) {
        u32x4 o = e2m1_unpack8_bf16_hw(wc, scale);
        if (nan_scale) o = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        if (c < nchunks) stream_st(o, reinterpret_cast<u32x4*>(y) + c);
      } else {
        // float32 (exact: a code times a power of two), then for float16 one
        // rounding to nearest even in st8
        float f[8];
        e2m1_unpack8_f32_hw(wc, scale, f);
        if (nan_scale) {
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = bitsf(0x7FC00000u);
        }
        st8_wave<DT>(y, c - lane, nchunks, lane, f);
      }
    }
  }
}

static int grid_for(int64_t ntiles) {
  // One tile per wave, kMxWaves waves per workgroup, up to the grid cap.
  const int64_t max_blocks = kMaxGridBlocks;
#ifndef MXQ_MX_UPW
#define MXQ_MX_UPW MXQ_UNITS_PER_WAVE
#endif
  int64_t b = (ntiles + kMxWaves * MXQ_MX_UPW - 1) / (kMxWaves * MXQ_MX_UPW);
  return (int)(b < max_blocks ? (b > 0 ? b : 1) : max_blocks);
}

// The quantizer runs at most seven of its workgroups per CU (see
// occupancy_lds): on the MoE sweep it took 185.6 us per 36-expert chunk
// against 190.9 at eight (what its registers allow) and 189 at six.  The
// dequantizer is fastest at eight.
#ifndef MXQ_MXQ_WG_PER_CU
#define MXQ_MXQ_WG_PER_CU 7
#endif
constexpr unsigned kMxQuantOccupancyLds = occupancy_lds(MXQ_MXQ_WG_PER_CU);

hipError_t launch_mxfp4_quant(const void* x, int dt, int64_t rows, int64_t K,
                              int8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t ntiles = (nchunks + kTileChunks - 1) / kTileChunks;
  const dim3 grid(grid_for(ntiles)), block(64 * kMxWaves);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_mxfp4_quant<DT_F32>, grid, block, kMxQuantOccupancyLds, s, x, p, scales, nchunks, ntiles); break;
    case DT_BF16: hipLaunchKernelGGL(k_mxfp4_quant<DT_BF16>, grid, block, kMxQuantOccupancyLds, s, x, p, scales, nchunks, ntiles); break;
    default: hipLaunchKernelGGL(k_mxfp4_quant<DT_F16>, grid, block, kMxQuantOccupancyLds, s, x, p, scales, nchunks, ntiles); break;
  }
  return hipGetLastError();
}

hipError_t launch_mxfp4_dequant(const int8_t* packed, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y, int dt,
                                hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t ntiles = (nchunks + kTileChunks - 1) / kTileChunks;
  const dim3 grid(grid_for(ntiles)), block(64 * kMxWaves);
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_mxfp4_dequant<DT_F32>, grid, block, 0, s, p, scales, y, nchunks, ntiles); break;
    case DT_BF16: hipLaunchKernelGGL(k_mxfp4_dequant<DT_BF16>, grid, block, 0, s, p, scales, y, nchunks, ntiles); break;
    default: hipLaunchKernelGGL(k_mxfp4_dequant<DT_F16>, grid, block, 0, s, p, scales, y, nchunks, ntiles); break;
  }
  return hipGetLastError();
}

} // namespace mxq
