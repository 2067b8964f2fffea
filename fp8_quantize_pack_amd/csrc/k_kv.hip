// k_kv.hip -- NVFP4 KV cache kernels for gfx950: dequantization of a paged
// cache into one contiguous tensor, and per-head quantization with k_smooth.
//
// Method: LongLive utils/quant.py, dequantize_kv_cache, k_smooth and
// quantize_kv, with the NVFP4 arithmetic of
// "nemo_automodel.components.quantization.nvfp4" (quantize_nvfp4,
// quantize_nvfp4_modelopt, dequantize_nvfp4).
//
// Paged dequantization.  Block b of the cache holds block_tokens * H rows of
// D values (row t * H + h: token t, head h) as packed e2m1 codes [rows, D/2],
// row-major e4m3 block scales [rows, D/16] and one float32 amax; its global
// scale is amax / (6 * 448).  The blocks are separate allocations reached
// through device arrays of pointers (the cache's block list); block b lands at
// tokens b * block_tokens .. of the output [blocks * block_tokens, H, D], so
// the output is the blocks' rows concatenated.  Each wavefront owns a tile of
// 2 x 64 consecutive 8-element chunks of one block: it reads the block's
// pointers and amax once (uniform), a packed dword and a scale byte per lane,
// and writes 16 bytes (bfloat16) per lane, contiguous over the wave.
//
// Quantization with k_smooth.  k [S, H, D], D a power of two in [16, 512].
// Each row (token, head) of D values is optionally smoothed: its mean is the
// binary32 pairwise sum (8 values in a lane, then a butterfly over the D / 8
// lanes of the row: the pairwise tree, since every addition is commutative)
// times 1 / D, rounded to the dtype; each value minus that mean is evaluated
// in binary32 and rounded to the dtype.  Every head's slice then gets one
// global scale g = amax(slice) / 2688 and the NVFP4 codes of the nvfp4 page.
// Pass 1 reduces the per-head maxima of the (smoothed) values: each
// workgroup owns a contiguous range of rows, folds them into per-head maxima
// in LDS, then issues one global atomic maximum per head; pass 2 recomputes
// the smoothed values (deterministic) and quantizes.  Rows are contiguous
// in memory, so every load and store of a wave is one contiguous range.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"
#include "mxq_nvfp4_common.h"

namespace mxq {

// ------------------------------------------------------------------ paged dequantization

constexpr int kKvUnroll = 2;
constexpr int kKvTileChunks = kKvUnroll * kWave;

template <int DT>
__global__ __launch_bounds__(256) void k_kv_pages_dequant(
    const uint8_t* const* __restrict__ values, const uint8_t* const* __restrict__ scales,
    const float* const* __restrict__ amax, int64_t cpb, int64_t tiles_per_block,
    int64_t ntiles, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < ntiles;
       t += nwaves) {
    const int64_t b = t / tiles_per_block;                 // uniform over the wave
    const int64_t c0 = (t - b * tiles_per_block) * kKvTileChunks + lane;
    const uint32_t* vb = reinterpret_cast<const uint32_t*>(values[b]);
    const uint8_t* sb = scales[b];
    const float g = *amax[b] / kGlobalDiv;
    uint32_t w[kKvUnroll], s[kKvUnroll];
#pragma unroll
    for (int u = 0; u < kKvUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const bool ok = c < cpb;
      w[u] = ok ? stream_ld(vb + c) : 0u;
      s[u] = ok ? (uint32_t)sb[c >> 1] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kKvUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const float sigma = e4m3_decode_any(s[u]);
      float f[8];
      e2m1_unpack8_f32_hw(e2m1_canonical_zeros(w[u]), 1.0f, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g;   // left to right, float32
      if (c < cpb) st8<DT>(y, b * cpb + c, f);
    }
  }
}

hipError_t launch_kv_pages_dequant(const uint8_t* const* values, const uint8_t* const* scales,
                                   const float* const* amax, int64_t nblocks,
                                   int64_t block_tokens, int64_t H, int64_t D, void* y, int dt,
                                   hipStream_t s) {
  const int64_t cpb = block_tokens * H * (D / 8);
  const int64_t tpb = (cpb + kKvTileChunks - 1) / kKvTileChunks;
  const int64_t ntiles = tpb * nblocks;
  int64_t g = (ntiles + 3) / 4;
  g = g < kMaxGridBlocks ? (g > 0 ? g : 1) : kMaxGridBlocks;
  const dim3 grid((unsigned)g), block(256);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_kv_pages_dequant<DT_F32>, grid, block, 0, s, values, scales, amax, cpb, tpb, ntiles, y); break;
    case DT_BF16: hipLaunchKernelGGL(k_kv_pages_dequant<DT_BF16>, grid, block, 0, s, values, scales, amax, cpb, tpb, ntiles, y); break;
    default: hipLaunchKernelGGL(k_kv_pages_dequant<DT_F16>, grid, block, 0, s, values, scales, amax, cpb, tpb, ntiles, y); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ k_smooth + per-head NVFP4

// Sum over aligned groups of G consecutive lanes, the result replicated in
// every lane of the group; the additions follow the pairwise tree over the
// lanes (each level adds two partial sums that every lane of both halves
// holds identically).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x = x + bitsf(dpp_u32<0xB1>(fbits(x)));    // lane ^ 1
  if constexpr (G >= 4) x = x + bitsf(dpp_u32<0x4E>(fbits(x)));    // lane ^ 2
  if constexpr (G >= 8) x = x + bitsf(dpp_u32<0x141>(fbits(x)));   // other quad of 8
  if constexpr (G >= 16) x = x + bitsf(dpp_u32<0x140>(fbits(x)));  // other half of 16
  if constexpr (G >= 32) x = x + __shfl_xor(x, 16);
  if constexpr (G >= 64) x = x + __shfl_xor(x, 32);
  return x;
}

template <int DT>
__device__ __forceinline__ float round_to_dt(float v) {
  if constexpr (DT == DT_BF16) return bitsf(f32_to_bf16_rne(v) << 16);
  else if constexpr (DT == DT_F16) return f16_to_f32(f32_to_f16_rne(v));
  else return v;
}

// k - mean(k) of the 8 values of this lane; the row spans L lanes.  Every
// lane of the wave must call this together.
template <int DT, int L>
__device__ __forceinline__ void k_smooth8(float f[8]) {
  float s = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
  s = group_sum<L>(s);
  const float m = round_to_dt<DT>(s * (1.0f / (float)(8 * L)));   // exact scaling
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = round_to_dt<DT>(f[i] - m);
}

struct KvGeom {
  int64_t rows;      // S * H
  int64_t rows_per_block;
  int H;
};

// Rows of this lane in iteration it of workgroup blk: a contiguous run of
// rows_per_block rows per workgroup, 4 waves x (64 / L) rows per iteration.
template <int L>
__device__ __forceinline__ int64_t kv_row(const KvGeom& geo, int it) {
  constexpr int kRpw = 64 / L;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  return (int64_t)blockIdx.x * geo.rows_per_block + (int64_t)it * (4 * kRpw) + wave * kRpw + lane / L;
}

template <int DT, bool SMOOTH, int L>
__global__ __launch_bounds__(256) void k_kv_head_amax(const void* __restrict__ k, KvGeom geo,
                                                      uint32_t* __restrict__ head_amax) {
  extern __shared__ uint32_t s_max[];
  constexpr int kRpw = 64 / L;
  for (int i = threadIdx.x; i < geo.H; i += blockDim.x) s_max[i] = 0u;
  __syncthreads();
  const int sub = threadIdx.x & (L - 1);
  const int64_t end0 = (int64_t)blockIdx.x * geo.rows_per_block + geo.rows_per_block;
  const int64_t end = end0 < geo.rows ? end0 : geo.rows;
  const int iters = (int)((geo.rows_per_block + 4 * kRpw - 1) / (4 * kRpw));
  const int64_t r0 = kv_row<L>(geo, 0);
  uint32_t h = (uint32_t)(r0 % geo.H);
  const uint32_t step = (uint32_t)((4 * kRpw) % geo.H);
  for (int it = 0; it < iters; ++it) {
    const int64_t row = r0 + (int64_t)it * (4 * kRpw);
    const bool ok = row < end;
    const Raw8<DT> raw = ok ? ld8<DT>(k, row * L + sub) : zero8<DT>();
    float f[8];
    unpack8<DT>(raw, f);
    if constexpr (SMOOTH) k_smooth8<DT, L>(f);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
    a = group_max<L>(a);
    if (ok && sub == 0) atomicMax(&s_max[h], fbits(a));
    h += step;
    h = h >= (uint32_t)geo.H ? h - geo.H : h;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < geo.H; i += blockDim.x)
    if (s_max[i] != 0u) atomicMax(&head_amax[i], s_max[i]);
}

template <int DT, bool SMOOTH, int L>
__global__ __launch_bounds__(256) void k_kv_quant(const void* __restrict__ k, KvGeom geo,
                                                  const uint32_t* __restrict__ head_amax,
                                                  uint32_t* __restrict__ packed,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ row_scale) {
  constexpr int kRpw = 64 / L;
  const int sub = threadIdx.x & (L - 1);
  const int64_t end0 = (int64_t)blockIdx.x * geo.rows_per_block + geo.rows_per_block;
  const int64_t end = end0 < geo.rows ? end0 : geo.rows;
  const int iters = (int)((geo.rows_per_block + 4 * kRpw - 1) / (4 * kRpw));
  const int64_t r0 = kv_row<L>(geo, 0);
  uint32_t h = (uint32_t)(r0 % geo.H);
  const uint32_t step = (uint32_t)((4 * kRpw) % geo.H);
  for (int it = 0; it < iters; ++it) {
    const int64_t row = r0 + (int64_t)it * (4 * kRpw);
    const bool ok = row < end;
    const Raw8<DT> raw = ok ? ld8<DT>(k, row * L + sub) : zero8<DT>();
    float f[8];
    unpack8<DT>(raw, f);
    if constexpr (SMOOTH) k_smooth8<DT, L>(f);
    // the 16-value block of this chunk is shared with lane ^ 1
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
    a = bitsf(max(fbits(a), pair_swap(fbits(a))));
    const float g = bitsf(head_amax[h]) / kGlobalDiv;
    const double rg = 1.0 / (double)g;
    uint32_t sb;
    const double rden = nv_block_recip(a, g, rg, sb);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = ceil22((float)((double)f[i] * rden));
    const uint32_t w = e2m1_pack8_rne(q, 1.0f);
    if (ok) {
      stream_st(w, packed + row * L + sub);
      if ((sub & 1) == 0) scales[row * (L / 2) + (sub >> 1)] = (uint8_t)sb;
      if (sub == 0) row_scale[row] = g;
    }
    h += step;
    h = h >= (uint32_t)geo.H ? h - geo.H : h;
  }
}

__global__ void k_fill_head_amax(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int DT, bool SMOOTH, int L>
static void launch_kv_quant_l(const void* k, const KvGeom& geo, int64_t nblk,
                              uint32_t* head_amax, uint32_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t s) {
  const size_t lds = sizeof(uint32_t) * (size_t)geo.H;
  hipLaunchKernelGGL((k_kv_head_amax<DT, SMOOTH, L>), dim3((unsigned)nblk), dim3(256), lds, s, k,
                     geo, head_amax);
  hipLaunchKernelGGL((k_kv_quant<DT, SMOOTH, L>), dim3((unsigned)nblk), dim3(256), 0, s, k, geo,
                     head_amax, packed, scales, row_scale);
}

template <int DT, bool SMOOTH>
static void launch_kv_quant_d(const void* k, const KvGeom& geo, int64_t nblk, int64_t D,
                              uint32_t* ha, uint32_t* p, uint8_t* sc, float* rs, hipStream_t s) {
  switch (D) {
    case 16: launch_kv_quant_l<DT, SMOOTH, 2>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 32: launch_kv_quant_l<DT, SMOOTH, 4>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 64: launch_kv_quant_l<DT, SMOOTH, 8>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 128: launch_kv_quant_l<DT, SMOOTH, 16>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 256: launch_kv_quant_l<DT, SMOOTH, 32>(k, geo, nblk, ha, p, sc, rs, s); break;
    default: launch_kv_quant_l<DT, SMOOTH, 64>(k, geo, nblk, ha, p, sc, rs, s); break;
  }
}

template <int DT>
static void launch_kv_quant_dt(const void* k, const KvGeom& geo, int64_t nblk, int64_t D,
                               bool smooth, uint32_t* ha, uint32_t* p, uint8_t* sc, float* rs,
                               hipStream_t s) {
  if (smooth) launch_kv_quant_d<DT, true>(k, geo, nblk, D, ha, p, sc, rs, s);
  else launch_kv_quant_d<DT, false>(k, geo, nblk, D, ha, p, sc, rs, s);
}

// Rows per workgroup: enough that the per-head atomics stay few, small
// enough that the grid has several workgroups per CU.
constexpr int64_t kKvRowsPerBlock = 512;

hipError_t launch_kv_quant(const void* k, int dt, int64_t S, int64_t H, int64_t D, int smooth,
                           float* head_amax, uint8_t* packed, uint8_t* scales,
                           float* row_scale, hipStream_t s) {
  KvGeom geo;
  geo.rows = S * H;
  geo.H = (int)H;
  geo.rows_per_block = kKvRowsPerBlock;
  const int64_t nblk = (geo.rows + kKvRowsPerBlock - 1) / kKvRowsPerBlock;
  uint32_t* ha = reinterpret_cast<uint32_t*>(head_amax);
  hipLaunchKernelGGL(k_fill_head_amax, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, s, ha, (int)H);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  switch (dt) {
    case DT_F32: launch_kv_quant_dt<DT_F32>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
    case DT_BF16: launch_kv_quant_dt<DT_BF16>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
    default: launch_kv_quant_dt<DT_F16>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
  }
  return hipGetLastError();
}

} // namespace mxq
