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
// 8 x 64 consecutive 8-element chunks of one block: it reads the block's
// pointers and amax once (uniform) and the tile's scale bytes as one dword
// per lane, then per step a packed dword per lane (and its scale byte from
// another lane's dword), and writes 16 bytes (bfloat16) per lane, contiguous
// over the wave.
//
// Quantization with k_smooth.  k [S, H, D], D a power of two in [16, 512].
// Each row (token, head) of D values is optionally smoothed: its mean is the
// binary32 pairwise sum (8 values in a lane, then a butterfly over the D / 8
// lanes of the row: the pairwise tree, since every addition is commutative)
// times 1 / D, rounded to the dtype; each value minus that mean is evaluated
// in binary32 and rounded to the dtype.  Every head's slice then gets one
// global scale g = amax(slice) / 2688 and the NVFP4 codes of the nvfp4 page.
// Both passes run on a fixed grid whose waves stride over tiles of 128
// chunks (lane l holds chunks l and 64 + l), loading the next step's tiles
// before the current step's arithmetic.  Pass 1 keeps the maxima of the
// (smoothed) values of its lane's two heads in registers, folds them in LDS
// and adds one atomic maximum per head and workgroup into one of 32 slots per
// head; pass 2 reduces the slots into per-head g and 1 / g tables in LDS,
// recomputes the smoothed values (deterministic) and quantizes, one binary64
// block reciprocal per lane pair and 16 values (as in the NVFP4 row kernel).
// Every load and store instruction of a wave covers one contiguous range.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"
#include "mxq_nvfp4_common.h"

namespace mxq {

// ------------------------------------------------------------------ paged dequantization

// 8 x 64 chunks per wave tile: 4 KiB of codes and 16 KiB of bfloat16 output
// per wave, so that the two dependent loads of the block's pointers and amax
// are amortized and enough loads are in flight.
#ifndef MXQ_KV_PAGE_UNROLL
#define MXQ_KV_PAGE_UNROLL 8
#endif
constexpr int kKvUnroll = MXQ_KV_PAGE_UNROLL;
constexpr int kKvTileChunks = kKvUnroll * kWave;

typedef const uint32_t __attribute__((address_space(1))) GlobalU32;
typedef const uint8_t __attribute__((address_space(1))) GlobalU8;
typedef const float __attribute__((address_space(1))) GlobalF32;

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
    // pointers read from memory are generic; the block arrays live in global
    // memory, so address them as such (global rather than flat loads)
    const GlobalU32* vb = (const GlobalU32*)(values[b]);
    const GlobalU8* sb = (const GlobalU8*)(scales[b]);
    const float g = *(const GlobalF32*)(amax[b]) / kGlobalDiv;
    uint32_t w[kKvUnroll], s[kKvUnroll];
    // A whole tile's 256 scale bytes are contiguous (16-byte aligned): lane l
    // loads dword l and step u takes the byte of chunk c0 + 64 u -- byte
    // 32 u + l / 2, in dword 8 u + l / 8 -- by a lane permute instead of a
    // byte load of its own.  A partial last tile loads bytes.
    static_assert(kKvUnroll == 8, "one scale dword per lane covers the tile");
    const bool full = c0 - lane + kKvTileChunks <= cpb;   // uniform over the wave
    if (full) {
      const uint32_t sd = __builtin_nontemporal_load((const GlobalU32*)(sb + ((c0 - lane) >> 1)) + lane);
      const int sh = 8 * ((lane >> 1) & 3);
#pragma unroll
      for (int u = 0; u < kKvUnroll; ++u) {
        w[u] = __builtin_nontemporal_load(vb + c0 + u * kWave);
        s[u] = ((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (8 * u + (lane >> 3)), (int)sd) >> sh) & 0xFFu;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kKvUnroll; ++u) {
        const int64_t c = c0 + u * kWave;
        const bool ok = c < cpb;
        w[u] = ok ? __builtin_nontemporal_load(vb + c) : 0u;
        s[u] = ok ? (uint32_t)sb[c >> 1] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kKvUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const float sigma = e4m3_decode_any(s[u]);
      float f[8];
      e2m1_unpack8_f32_hw(e2m1_canonical_zeros(w[u]), 1.0f, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g;   // left to right, float32
      st8_wave<DT>(y, b * cpb + c - lane, b * cpb + cpb, lane, f);
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
#ifndef MXQ_KVP_UPW
#define MXQ_KVP_UPW MXQ_UNITS_PER_WAVE
#endif
  int64_t g = (ntiles + 4 * MXQ_KVP_UPW - 1) / (4 * MXQ_KVP_UPW);
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
  // G == 1: the lane holds the whole row
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
  if constexpr (DT == DT_BF16) return bitsf(bf16x2_rne(v, 0.0f) << 16);
  else if constexpr (DT == DT_F16) return f16_to_f32(f16x2_rne(v, 0.0f) & 0xFFFFu);
  else return v;
}

// k - mean(k) of the 8 values of this lane; the row spans L lanes (L
// consecutive chunks).  Every lane of the wave must call this together.  The
// in-lane sum is the pairwise tree over the 8 values and the lanes continue
// it.  bfloat16 rounds through the hardware pair converter (round to nearest
// even, two values per instruction); each difference is a float32 value
// first.
template <int DT, int L>
__device__ __forceinline__ void k_smooth8(float f[8]) {
  float s = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
  s = group_sum<L>(s);
  const float m = round_to_dt<DT>(s * (1.0f / (float)(8 * L)));   // exact scaling
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float d0 = f[i] - m, d1 = f[i + 1] - m;
      unpack_bf16x2(bf16x2_rne(d0, d1), f[i], f[i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = round_to_dt<DT>(f[i] - m);
  }
}

// Work layout of both passes: a wavefront tile is 128 consecutive chunks of
// 8 values; lane l holds chunks l and 64 + l, so each of the two load (and
// store) instructions covers one contiguous 1 KiB (bfloat16) range.  A row of
// D values is L = D / 8 consecutive chunks and never straddles the two
// halves (L divides 64); the 16-value blocks are lane pairs.  The grid is a
// fixed number of workgroups whose waves stride over the tiles, so that each
// workgroup's set-up (LDS tables, the final atomics) is paid once.  The host
// makes the stride (in rows) a multiple of the head count, so the heads of a
// lane's two rows are the same in every tile it visits: a lane keeps its
// running maxima (pass 1) and its heads' scales (pass 2) in registers.
// Workgroups of each pass (at most; rounded up as the launcher explains).
// Pass 1 ends with one atomic per head and workgroup, so it takes fewer.
#ifndef MXQ_KV_AMAX_GRID_BLOCKS
#define MXQ_KV_AMAX_GRID_BLOCKS 1024
#endif
#ifndef MXQ_KV_QUANT_GRID_BLOCKS
#define MXQ_KV_QUANT_GRID_BLOCKS 1536
#endif
constexpr int64_t kKvAmaxGridBlocks = MXQ_KV_AMAX_GRID_BLOCKS;
constexpr int64_t kKvQuantGridBlocks = MXQ_KV_QUANT_GRID_BLOCKS;
#ifndef MXQ_KV_ROW_UNROLL
#define MXQ_KV_ROW_UNROLL 2
#endif
// tiles a wave works on per step; the next step's tiles are loaded before
// this step's arithmetic, so 2 * kKvRowUnroll tiles are in registers
constexpr int kKvRowUnroll = MXQ_KV_ROW_UNROLL;

struct KvGeom {
  int64_t nchunks;   // S * H * D / 8
  int64_t tiles;     // ceil(nchunks / 128)
  int H;
};

// Each head's maximum is spread over kKvAmaxSlots words (workgroup b folds
// into slot b % kKvAmaxSlots), which keeps the atomics on one address few.
// The scratch is slot-major, word s * H + h, so that the slots of one head
// lie in different cache lines (atomics on one line serialize); slot 0 of
// head h, word h, holds the head's maximum after the quantize pass.
#ifndef MXQ_KV_AMAX_SLOTS
#define MXQ_KV_AMAX_SLOTS 32
#endif
constexpr int kKvAmaxSlots = MXQ_KV_AMAX_SLOTS;

// First tile, tile stride, first row of this lane's chunk l, and the heads of
// its two rows (row_a and row_a + 64 / L), which the stride leaves unchanged.
template <int L>
struct KvRows {
  int64_t tile, stride, row_a;
  uint32_t h_a, h_b;
  __device__ __forceinline__ KvRows(const KvGeom& geo) {
    constexpr int R = 128 / L;                           // rows per tile
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    tile = (int64_t)blockIdx.x * 4 + wave;
    stride = (int64_t)gridDim.x * 4;
    row_a = tile * R + lane / L;
    h_a = (uint32_t)(row_a % geo.H);
    h_b = (uint32_t)((row_a + R / 2) % geo.H);
  }
};

template <int DT>
struct KvTile { Raw8<DT> c0, c1; };

// FULL: every chunk of the tile is in range (no guards, so that the loads and
// stores of a step are unconditional and the compiler can wait for exactly
// the loads a step needs while the next step's are in flight).
template <int DT, bool FULL>
__device__ __forceinline__ KvTile<DT> kv_tile_load(const void* k, const KvGeom& geo, int64_t tile) {
  const int64_t c = tile * 128 + (threadIdx.x & 63);
  KvTile<DT> t;
  t.c0 = (FULL || c < geo.nchunks) ? ld8<DT>(k, c) : zero8<DT>();
  t.c1 = (FULL || c + 64 < geo.nchunks) ? ld8<DT>(k, c + 64) : zero8<DT>();
  return t;
}

// Whether tiles tile, tile + stride, ..., tile + (n - 1) * stride all lie
// wholly in range (uniform over the wave).
__device__ __forceinline__ bool kv_tiles_full(const KvGeom& geo, int64_t tile, int64_t stride, int n) {
  return (tile + (n - 1) * stride) * 128 + 128 <= geo.nchunks;
}

// Pass 1 on one tile: the running maxima of the lane's two rows.
template <int DT, bool SMOOTH, int L>
__device__ __forceinline__ void kv_amax_tile(const KvTile<DT>& t, float& m0, float& m1) {
  float f0[8], f1[8];
  unpack8<DT>(t.c0, f0);
  unpack8<DT>(t.c1, f1);
  if constexpr (SMOOTH) {
    k_smooth8<DT, L>(f0);
    k_smooth8<DT, L>(f1);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m0 = fmaxf(m0, fabsf(f0[i]));
    m1 = fmaxf(m1, fabsf(f1[i]));
  }
}

template <int DT, bool SMOOTH, int L>
__global__ __launch_bounds__(256) void k_kv_head_amax(const void* __restrict__ k, KvGeom geo,
                                                      uint32_t* __restrict__ head_amax) {
  extern __shared__ uint32_t s_max[];
  constexpr int U = kKvRowUnroll;
  for (int i = threadIdx.x; i < geo.H; i += blockDim.x) s_max[i] = 0u;
  __syncthreads();
  const KvRows<L> rr(geo);
  const int64_t st = rr.stride;
  float m0 = 0.0f, m1 = 0.0f;           // running maxima of the lane's two rows' heads
  // chunks past the end load as zeros, which leave a maximum unchanged
  KvTile<DT> t[U];
#pragma unroll
  for (int u = 0; u < U; ++u) t[u] = kv_tile_load<DT, false>(k, geo, rr.tile + u * st);
  // the next step's loads go out before this step's arithmetic; steps whose
  // next tiles are all in range first (one loop without guards), then the rest
  int64_t tile = rr.tile;
  for (; tile < geo.tiles && kv_tiles_full(geo, tile + U * st, st, U); tile += U * st) {
    KvTile<DT> n[U];
#pragma unroll
    for (int u = 0; u < U; ++u) n[u] = kv_tile_load<DT, true>(k, geo, tile + (U + u) * st);
#pragma unroll
    for (int u = 0; u < U; ++u) kv_amax_tile<DT, SMOOTH, L>(t[u], m0, m1);
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = n[u];
  }
  for (; tile < geo.tiles; tile += U * st) {
    KvTile<DT> n[U];
#pragma unroll
    for (int u = 0; u < U; ++u) n[u] = kv_tile_load<DT, false>(k, geo, tile + (U + u) * st);
#pragma unroll
    for (int u = 0; u < U; ++u) kv_amax_tile<DT, SMOOTH, L>(t[u], m0, m1);
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = n[u];
  }
  m0 = group_max<L>(m0);
  m1 = group_max<L>(m1);
  if ((threadIdx.x & (L - 1)) == 0) {                   // first lane of its row
    atomicMax(&s_max[rr.h_a], fbits(m0));
    atomicMax(&s_max[rr.h_b], fbits(m1));
  }
  __syncthreads();
  const int slot = blockIdx.x % kKvAmaxSlots;
  for (int i = threadIdx.x; i < geo.H; i += blockDim.x)
    if (s_max[i] != 0u) atomicMax(&head_amax[slot * geo.H + i], s_max[i]);
}

// Pass 2 on one tile: k_smooth, block maxima (the block is the lane pair),
// one block scale per lane (the even lane's for chunk 0's block, the odd
// lane's for chunk 1's), both reciprocals by one pair exchange, codes, and
// the stores.  Every lane of a row writes its row scale (the same value).
template <int DT, bool SMOOTH, int L, bool FULL>
__device__ __forceinline__ void kv_quant_tile(const KvTile<DT>& t, const KvGeom& geo, int64_t tile,
                                              float g_a, float g_b, float g_m, double rg_m,
                                              uint32_t* __restrict__ packed,
                                              uint8_t* __restrict__ scales,
                                              float* __restrict__ row_scale) {
  constexpr int R = 128 / L;
  const int lane = threadIdx.x & 63;
  const bool odd = lane & 1;
  const int64_t c = tile * 128 + lane;
  float f0[8], f1[8];
  unpack8<DT>(t.c0, f0);
  unpack8<DT>(t.c1, f1);
  if constexpr (SMOOTH) {
    k_smooth8<DT, L>(f0);
    k_smooth8<DT, L>(f1);
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0 = fmaxf(a0, fabsf(f0[i]));
    a1 = fmaxf(a1, fabsf(f1[i]));
  }
  a0 = bitsf(max(fbits(a0), pair_swap(fbits(a0))));
  a1 = bitsf(max(fbits(a1), pair_swap(fbits(a1))));
  uint32_t sb;
  const double mine = nv_block_recip(odd ? a1 : a0, g_m, rg_m, sb);
  // chunk 0 lies in the even lane's block, chunk 1 in the odd lane's
  const double r0 = pair_lane<kQuadEven>(mine), r1 = pair_lane<kQuadOdd>(mine);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = nv_quotient(f0[i], r0);
  const uint32_t w0 = e2m1_pack8_even(q, 1.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = nv_quotient(f1[i], r1);
  const uint32_t w1 = e2m1_pack8_even(q, 1.0f);
  const int64_t cm = odd ? c + 64 : c;                // chunk of this lane's block
  const int64_t row = tile * R + lane / L;
  if (FULL || c < geo.nchunks) stream_st(w0, packed + c);
  if (FULL || c + 64 < geo.nchunks) stream_st(w1, packed + c + 64);
  if (FULL || cm < geo.nchunks) scales[cm >> 1] = (uint8_t)sb;
  if (FULL || c < geo.nchunks) row_scale[row] = g_a;
  if (FULL || c + 64 < geo.nchunks) row_scale[row + R / 2] = g_b;
}

template <int DT, bool SMOOTH, int L>
__global__ __launch_bounds__(256) void k_kv_quant(const void* __restrict__ k, KvGeom geo,
                                                  uint32_t* __restrict__ head_amax,
                                                  uint32_t* __restrict__ packed,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ row_scale) {
  // per-head amax (the maximum over its slots; workgroup 0 writes it back to
  // slot 0, which leaves every reader's maximum unchanged), g = amax / 2688
  // and its correctly rounded binary64 reciprocal
  extern __shared__ double s_rg[];
  float* s_g = reinterpret_cast<float*>(s_rg + geo.H);
  for (int i = threadIdx.x; i < geo.H; i += blockDim.x) {
    uint32_t m = 0u;
    for (int j = 0; j < kKvAmaxSlots; ++j) m = max(m, head_amax[j * geo.H + i]);
    if (blockIdx.x == 0) head_amax[i] = m;
    const float g = bitsf(m) / kGlobalDiv;
    s_g[i] = g;
    s_rg[i] = 1.0 / (double)g;
  }
  __syncthreads();
  constexpr int U = kKvRowUnroll;
  const bool odd = threadIdx.x & 1;
  const KvRows<L> rr(geo);
  const int64_t st = rr.stride;
  const float g_a = s_g[rr.h_a], g_b = s_g[rr.h_b];
  const float g_m = odd ? g_b : g_a;
  const double rg_m = s_rg[odd ? rr.h_b : rr.h_a];
  KvTile<DT> t[U];
#pragma unroll
  for (int u = 0; u < U; ++u) t[u] = kv_tile_load<DT, false>(k, geo, rr.tile + u * st);
  // as in pass 1: steps whose tiles and next tiles are all in range run
  // without guards, then the rest
  int64_t tile = rr.tile;
  for (; tile < geo.tiles && kv_tiles_full(geo, tile, st, 2 * U); tile += U * st) {
    KvTile<DT> n[U];
#pragma unroll
    for (int u = 0; u < U; ++u) n[u] = kv_tile_load<DT, true>(k, geo, tile + (U + u) * st);
#pragma unroll
    for (int u = 0; u < U; ++u)
      kv_quant_tile<DT, SMOOTH, L, true>(t[u], geo, tile + u * st, g_a, g_b, g_m, rg_m,
                                         packed, scales, row_scale);
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = n[u];
  }
  for (; tile < geo.tiles; tile += U * st) {
    KvTile<DT> n[U];
#pragma unroll
    for (int u = 0; u < U; ++u) n[u] = kv_tile_load<DT, false>(k, geo, tile + (U + u) * st);
#pragma unroll
    for (int u = 0; u < U; ++u)
      kv_quant_tile<DT, SMOOTH, L, false>(t[u], geo, tile + u * st, g_a, g_b, g_m, rg_m,
                                          packed, scales, row_scale);
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = n[u];
  }
}

__global__ void k_fill_head_amax(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int DT, bool SMOOTH, int L>
static void launch_kv_quant_l(const void* k, const KvGeom& geo, const int64_t nblk[2],
                              uint32_t* head_amax, uint32_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t s) {
  const size_t lds_max = sizeof(uint32_t) * (size_t)geo.H;
  const size_t lds_g = (sizeof(double) + sizeof(float)) * (size_t)geo.H;
  hipLaunchKernelGGL((k_kv_head_amax<DT, SMOOTH, L>), dim3((unsigned)nblk[0]), dim3(256), lds_max, s,
                     k, geo, head_amax);
  hipLaunchKernelGGL((k_kv_quant<DT, SMOOTH, L>), dim3((unsigned)nblk[1]), dim3(256), lds_g, s, k,
                     geo, head_amax, packed, scales, row_scale);
}

template <int DT, bool SMOOTH>
static void launch_kv_quant_d(const void* k, const KvGeom& geo, const int64_t nblk[2], int64_t D,
                              uint32_t* ha, uint32_t* p, uint8_t* sc, float* rs, hipStream_t s) {
  switch (D) {     // chunks (lanes) per row
    case 16: launch_kv_quant_l<DT, SMOOTH, 2>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 32: launch_kv_quant_l<DT, SMOOTH, 4>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 64: launch_kv_quant_l<DT, SMOOTH, 8>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 128: launch_kv_quant_l<DT, SMOOTH, 16>(k, geo, nblk, ha, p, sc, rs, s); break;
    case 256: launch_kv_quant_l<DT, SMOOTH, 32>(k, geo, nblk, ha, p, sc, rs, s); break;
    default: launch_kv_quant_l<DT, SMOOTH, 64>(k, geo, nblk, ha, p, sc, rs, s); break;
  }
}

template <int DT>
static void launch_kv_quant_dt(const void* k, const KvGeom& geo, const int64_t nblk[2], int64_t D,
                               bool smooth, uint32_t* ha, uint32_t* p, uint8_t* sc, float* rs,
                               hipStream_t s) {
  if (smooth) launch_kv_quant_d<DT, true>(k, geo, nblk, D, ha, p, sc, rs, s);
  else launch_kv_quant_d<DT, false>(k, geo, nblk, D, ha, p, sc, rs, s);
}

hipError_t launch_kv_quant(const void* k, int dt, int64_t S, int64_t H, int64_t D, int smooth,
                           float* head_amax, uint8_t* packed, uint8_t* scales,
                           float* row_scale, hipStream_t s) {
  KvGeom geo;
  geo.nchunks = S * H * (D / 8);
  geo.tiles = (geo.nchunks + 127) / 128;
  geo.H = (int)H;
  // workgroups of each pass: up to its cap (fewer for small tensors), then
  // rounded up to a multiple of q = H / gcd(4 * rows per tile, H), so that
  // the stride of the grid's 4 * nblk waves, 4 * nblk * rows per tile rows,
  // is a multiple of H
  const int64_t rows_per_tile = 1024 / D;
  int64_t a = 4 * rows_per_tile, b = H;
  while (b != 0) { const int64_t r = a % b; a = b; b = r; }
  const int64_t q = H / a;
  const int64_t want = (geo.tiles + 3) / 4;
  const int64_t caps[2] = {kKvAmaxGridBlocks, kKvQuantGridBlocks};
  int64_t nblk[2];
  for (int i = 0; i < 2; ++i) {
    const int64_t n = want < caps[i] ? want : caps[i];
    nblk[i] = (n + q - 1) / q * q;
  }
  uint32_t* ha = reinterpret_cast<uint32_t*>(head_amax);
  const int nslots = (int)H * kKvAmaxSlots;
  hipLaunchKernelGGL(k_fill_head_amax, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, s, ha, nslots);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  switch (dt) {
    case DT_F32: launch_kv_quant_dt<DT_F32>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
    case DT_BF16: launch_kv_quant_dt<DT_BF16>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
    default: launch_kv_quant_dt<DT_F16>(k, geo, nblk, D, smooth != 0, ha, p, scales, row_scale, s); break;
  }
  return hipGetLastError();
}

} // namespace mxq
