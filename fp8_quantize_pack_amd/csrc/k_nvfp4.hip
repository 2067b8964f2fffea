// k_nvfp4.hip -- NVFP4 (ModelOpt layout) quantize-pack and dequantize
// kernels for gfx950.
//
// Method: "nemo_automodel.components.quantization.nvfp4", sections
// quantize_nvfp4, quantize_nvfp4_modelopt, dequantize_nvfp4, Data:
//   g           = amax(row) / (6 * 448)     (or a given / whole-tensor value)
//   block scale = e4m3(amax(block) / 6 / g) per 16 columns
//   code        = round_to_e2m1(x / (block scale * g))
//   decode      = e2m1 * e4m3 * g in float32, then one rounding to dtype.
//
// Layout of the work.  Rows of 64 blocks or more are cut into segments of 64
// blocks (1024 elements).  A wavefront reads a segment with two loads that are
// each contiguous over the wave: lane L takes chunks L and 64 + L (8 elements
// each), i.e. one half of blocks L/2 and 32 + L/2, whose other halves sit in
// lane L ^ 1.  The pair combines its half-block maxima with one DPP swap; the
// even lane derives the scale of block L/2, the odd lane that of block
// 32 + L/2, and one more swap hands each lane both reciprocals -- so a wave
// still computes one scale per lane for 1024 elements.  Codes leave as one
// dword per lane and instruction, contiguous again.  A row is owned by WPR
// waves of the workgroup (segments w, w + WPR, ... go to wave w), which
// combine their row maxima through LDS; with NIT > 0 every wave keeps its
// NIT segments in registers between the row-amax reduction and the
// quantization (HBM is read once); NIT == 0 is the fallback for very long
// rows, which reads the row twice.  Rows of fewer than 64 blocks take one
// block per lane, several rows per wave.
//
// Exactness of the element step: q = RN(x / den) is needed only through the
// e2m1 decisions q > m.  The kernel forms the binary64 product x * (1 / den)
// (1 / den correctly rounded), rounds it to float32 -- which lands on the same
// side of every decision boundary as x / den (see nvfp4_quant8 in
// mxq_device.h) -- rounds that up to 22 significant bits (ceil22, again
// decision-preserving) and lets the fp4 converter round half down
// (e2m1_pack8_rne).
#include "mxq_kernel_common.h"
#include "mxq_launch.h"
#include "mxq_nvfp4_common.h"

namespace mxq {

__device__ __forceinline__ float nv_row_scale(int mode, float row_amax,
                                              const float* given,
                                              int64_t given_stride, int64_t row,
                                              const uint32_t* tensor_amax) {
  if (mode == 1) return given[row * given_stride];
  if (mode == 2) return bitsf(*tensor_amax) / kGlobalDiv;
  return row_amax / kGlobalDiv;
}

struct NvSegGeom {
  int64_t rows;
  int64_t bpr;      // 16-column blocks per row = K / 16
  int64_t cpr;      // 8-column chunks per row = 2 * bpr
  int nseg;         // 64-block segments per row = ceil(bpr / 64)
};

// One segment's two chunks of this lane (zero outside the row) and their
// magnitude maxima as ordered bit patterns (amax8_bits), taken once: the row
// maximum and the block maxima both use them.
template <int DT>
struct SegChunks { Raw8<DT> c0, c1; uint32_t m0, m1; };

// With FULL (every segment of a row has 64 blocks) the guards depend only on
// the row and the segment, which are uniform over the wave.
template <int DT, bool FULL>
__device__ __forceinline__ SegChunks<DT> seg_load(const void* x, const NvSegGeom& geo,
                                                  bool row_ok, int64_t cbase, int seg, int lane) {
  const int64_t ch0 = (int64_t)seg * 128 + lane;       // chunk index within the row
  const bool ok0 = FULL ? (row_ok && seg < geo.nseg) : (row_ok && ch0 < geo.cpr);
  const bool ok1 = FULL ? ok0 : (row_ok && ch0 + 64 < geo.cpr);
  SegChunks<DT> c;
  // (float32 rows keep the per-lane loads: the half exchange of ld8_wave made
  // this kernel, which holds a whole row in registers, 22% slower)
  c.c0 = ok0 ? ld8<DT>(x, cbase + ch0) : zero8<DT>();
  c.c1 = ok1 ? ld8<DT>(x, cbase + ch0 + 64) : zero8<DT>();
  c.m0 = amax8_bits<DT>(c.c0);
  c.m1 = amax8_bits<DT>(c.c1);
  return c;
}

// Quantize one loaded segment: block maxima from the pair, one scale per lane,
// codes of both chunks, stores.
template <int DT, bool FULL, bool NORMAL>
__device__ __forceinline__ void seg_quant(const SegChunks<DT>& c, const NvSegGeom& geo,
                                          bool row_ok, int64_t row, int seg, int lane,
                                          float g, double rg, uint32_t* __restrict__ packed,
                                          uint8_t* __restrict__ scales) {
  const uint32_t p0 = max(c.m0, pair_swap(c.m0));      // block of chunk 0
  const uint32_t p1 = max(c.m1, pair_swap(c.m1));      // block of chunk 1
  const bool odd = lane & 1;
  uint32_t sb;
  const float a = amax_from_bits<DT>(odd ? p1 : p0);
  const double mine = NORMAL ? nv_block_recip_normal(a, g, rg, sb) : nv_block_recip(a, g, rg, sb);
  const double other = pair_lane<kQuadSwap>(mine);
  const uint32_t w0 = nv_codes8<DT>(c.c0, odd ? other : mine);
  const uint32_t w1 = nv_codes8<DT>(c.c1, odd ? mine : other);
  const int64_t ch0 = (int64_t)seg * 128 + lane;
  const int64_t cbase = row * geo.cpr;
  const int64_t blk = (int64_t)seg * 64 + (odd ? 32 : 0) + (lane >> 1);
  const bool ok0 = FULL ? (row_ok && seg < geo.nseg) : (row_ok && ch0 < geo.cpr);
  const bool ok1 = FULL ? ok0 : (row_ok && ch0 + 64 < geo.cpr);
  const bool okb = FULL ? ok0 : (row_ok && blk < geo.bpr);
  if (ok0) stream_st(w0, packed + cbase + ch0);
  if (ok1) stream_st(w1, packed + cbase + ch0 + 64);
  if (okb) scales[row * geo.bpr + blk] = (uint8_t)sb;
}

template <int DT, int NIT, int WPR, bool FULL>
__global__ __launch_bounds__(256) void k_nvfp4_quant_seg(
    const void* __restrict__ x, NvSegGeom geo, int mode,
    const float* __restrict__ given, int64_t given_stride,
    const uint32_t* __restrict__ tensor_amax, uint32_t* __restrict__ packed,
    uint8_t* __restrict__ scales, float* __restrict__ row_scale) {
  __shared__ uint32_t part[2][4];              // partial row maxima, double-buffered
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int wir = wave % WPR;                  // wave within its row
  constexpr int rows_per_block = 4 / WPR;
  const int64_t ngroups = (geo.rows + rows_per_block - 1) / rows_per_block;
  int buf = 0;
  for (int64_t bg = blockIdx.x; bg < ngroups; bg += gridDim.x) {
    const int64_t row = bg * rows_per_block + wave / WPR;
    const bool row_ok = row < geo.rows;
    const int64_t cbase = row * geo.cpr;
    SegChunks<DT> c[NIT > 0 ? NIT : 1];
    float amax = 0.0f;
    if constexpr (NIT > 0) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) c[it] = seg_load<DT, FULL>(x, geo, row_ok, cbase, wir + it * WPR, lane);
      if (mode == 0) {
        uint32_t m = 0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) m = max(m, max(c[it].m0, c[it].m1));
        amax = amax_from_bits<DT>(m);
      }
    } else {
      if (mode == 0) {
        uint32_t m = 0;
        for (int seg = wir; seg < geo.nseg; seg += WPR) {
          const SegChunks<DT> t = seg_load<DT, FULL>(x, geo, row_ok, cbase, seg, lane);
          m = max(m, max(t.m0, t.m1));
        }
        amax = amax_from_bits<DT>(m);
      }
    }
    if (mode == 0) {
      amax = group_max<64>(amax);
      if constexpr (WPR > 1) {
        // One barrier per row group: a wave can rewrite part[buf] only after
        // the next group's barrier, which every reader of it has passed.
        if (lane == 0) part[buf][wave] = fbits(amax);
        __syncthreads();
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < WPR; ++w) m = max(m, part[buf][(wave / WPR) * WPR + w]);
        amax = bitsf(m);
        buf ^= 1;
      }
    }
    float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
    g = bitsf(__builtin_amdgcn_readfirstlane(fbits(g)));   // the same in every lane
    const double rg = 1.0 / (double)g;
    if (row_ok && wir == 0 && lane == 0) row_scale[row] = g;
    if (nv_g_normal(g)) {
      if constexpr (NIT > 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
          seg_quant<DT, FULL, true>(c[it], geo, row_ok, row, wir + it * WPR, lane, g, rg, packed, scales);
      } else {
        for (int seg = wir; seg < geo.nseg; seg += WPR)
          seg_quant<DT, FULL, true>(seg_load<DT, FULL>(x, geo, row_ok, cbase, seg, lane), geo, row_ok,
                                    row, seg, lane, g, rg, packed, scales);
      }
    } else {
      if constexpr (NIT > 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
          seg_quant<DT, FULL, false>(c[it], geo, row_ok, row, wir + it * WPR, lane, g, rg, packed, scales);
      } else {
        for (int seg = wir; seg < geo.nseg; seg += WPR)
          seg_quant<DT, FULL, false>(seg_load<DT, FULL>(x, geo, row_ok, cbase, seg, lane), geo, row_ok,
                                     row, seg, lane, g, rg, packed, scales);
      }
    }
  }
}

// Rows of fewer than 64 blocks: lane `sub` of the LPR lanes (a power of two
// >= blocks per row) of a row owns block `sub` (16 elements, 32 bytes of
// bfloat16), 64 / LPR rows per wave.
template <int DT>
__global__ __launch_bounds__(256) void k_nvfp4_quant_short(
    const void* __restrict__ x, int64_t rows, int64_t bpr, int lpr, int mode,
    const float* __restrict__ given, int64_t given_stride,
    const uint32_t* __restrict__ tensor_amax, u32x2* __restrict__ packed,
    uint8_t* __restrict__ scales, float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (lpr - 1);
  const int rows_per_wave = kWave / lpr;
  const int rows_per_block = 4 * rows_per_wave;
  const int row_in_block = (threadIdx.x >> 6) * rows_per_wave + lane / lpr;
  const int64_t ngroups = (rows + rows_per_block - 1) / rows_per_block;
  for (int64_t bg = blockIdx.x; bg < ngroups; bg += gridDim.x) {
    const int64_t row = bg * rows_per_block + row_in_block;
    const bool ok = row < rows && sub < bpr;
    const int64_t blk = row * bpr + sub;
    const Raw8<DT> lo = ok ? ld8<DT>(x, 2 * blk) : zero8<DT>();
    const Raw8<DT> hi = ok ? ld8<DT>(x, 2 * blk + 1) : zero8<DT>();
    const float ba = amax_from_bits<DT>(max(amax8_bits<DT>(lo), amax8_bits<DT>(hi)));
    const float amax = (mode == 0) ? group_max_rt(ba, lpr) : 0.0f;
    const bool row_ok = row < rows;
    const float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
    const double rg = 1.0 / (double)g;
    if (row_ok && sub == 0) row_scale[row] = g;
    if (ok) {
      uint32_t sb;
      const double rden = nv_block_recip(ba, g, rg, sb);
      stream_st(u32x2{nv_codes8<DT>(lo, rden), nv_codes8<DT>(hi, rden)}, packed + blk);
      scales[blk] = (uint8_t)sb;
    }
  }
}

// Whole-tensor amax for the one-tensor-scale mode: a grid-stride max over all
// chunks, reduced per wave and combined with an integer atomic max on the bit
// patterns (non-negative floats order like their patterns).
// Whole-tensor amax: a grid-stride pass (magnitude maxima on the raw 16-bit
// patterns); the waves of a workgroup combine through LDS and issue one
// atomic maximum (atomics on one address serialize, so their number is kept
// to the workgroup count).  One workgroup per CU with eight chunks in flight
// per lane reads fastest (measured on a 1 GB bf16 tensor: 148 us, against
// 194 us with 4096 workgroups of four chunks per lane).
#ifndef MXQ_TENSOR_AMAX_BLOCKS
#define MXQ_TENSOR_AMAX_BLOCKS 256
#endif
constexpr int64_t kTensorAmaxBlocks = MXQ_TENSOR_AMAX_BLOCKS;
#ifndef MXQ_TENSOR_AMAX_UNROLL
#define MXQ_TENSOR_AMAX_UNROLL 8
#endif
constexpr int kTensorAmaxUnroll = MXQ_TENSOR_AMAX_UNROLL;   // loads in flight per thread

template <int DT>
__global__ __launch_bounds__(256) void k_tensor_amax(const void* __restrict__ x,
                                                     int64_t nchunks,
                                                     uint32_t* __restrict__ out) {
  constexpr int U = kTensorAmaxUnroll;
  uint32_t m = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; c + (U - 1) * stride < nchunks; c += U * stride) {
    Raw8<DT> r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = ld8<DT>(x, c + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) m = max(m, amax8_bits<DT>(r[u]));
  }
  for (; c < nchunks; c += stride) m = max(m, amax8_bits<DT>(ld8<DT>(x, c)));
  __shared__ uint32_t s_wave[4];
  const float amax = group_max<64>(amax_from_bits<DT>(m));
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = fbits(amax);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t w = max(max(s_wave[0], s_wave[1]), max(s_wave[2], s_wave[3]));
    atomicMax(out, w);
  }
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

// Dequantization of short rows (fewer than kDqSegChunks chunks): the tensor
// is a flat run of 8-element chunks (rows are contiguous and hold an even
// number of chunks, so chunk c's scale byte is c / 2).  A wavefront owns
// kDqFlatUnroll x 64 consecutive chunks, every load and store instruction
// contiguous over the wave; each lane finds the row of its first chunk with
// one division and advances it by a fixed quotient and remainder per step.
#ifndef MXQ_NVD_FLAT_UNROLL
#define MXQ_NVD_FLAT_UNROLL 8
#endif
constexpr int kDqFlatUnroll = MXQ_NVD_FLAT_UNROLL;
constexpr int kDqFlatTile = kDqFlatUnroll * kWave;

struct NvFlatGeom {
  int64_t nchunks;
  int64_t cpr;      // chunks per row (even, < kDqSegChunks)
  int64_t ntiles;
  int32_t drow;     // 64 / cpr
  int32_t drem;     // 64 % cpr
};

template <int DT>
__global__ __launch_bounds__(256) void k_nvfp4_dequant_flat(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ row_scale, NvFlatGeom geo, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < geo.ntiles;
       t += nwaves) {
    const int64_t c0 = t * kDqFlatTile + lane;
    int64_t row = c0 / geo.cpr;
    int32_t rem = (int32_t)(c0 - row * geo.cpr);
    uint32_t w[kDqFlatUnroll], sb[kDqFlatUnroll];
    float g[kDqFlatUnroll];
#pragma unroll
    for (int u = 0; u < kDqFlatUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      const bool ok = c < geo.nchunks;
      w[u] = ok ? stream_ld(packed + c) : 0u;
      sb[u] = ok ? (uint32_t)scales[c >> 1] : 0u;
      g[u] = ok ? row_scale[row] : 0.0f;
      row += geo.drow;
      rem += geo.drem;
      if (rem >= geo.cpr) { rem -= (int32_t)geo.cpr; ++row; }
    }
#pragma unroll
    for (int u = 0; u < kDqFlatUnroll; ++u) {
      const int64_t c = c0 + u * kWave;
      float f[8];
      const float sigma = e4m3_decode_any(sb[u]);
      e2m1_unpack8_f32_hw(e2m1_canonical_zeros(w[u]), 1.0f, f);   // exact e2m1
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g[u];     // exact, then RN
      st8_wave<DT>(y, c - lane, geo.nchunks, lane, f);
    }
  }
}

// Dequantization of rows of at least kDqSegChunks chunks: a wave owns one
// segment of kDqSegChunks consecutive chunks of a row (lane l takes chunks
// l, l + 64, ...), so every load and store instruction is contiguous, the
// row and its scale are the same for the whole wave (scalar), and the grid
// has many small units that the dispatcher spreads evenly.
constexpr int kDqSegUnroll = 2;
constexpr int kDqSegChunks = kDqSegUnroll * kWave;

template <int DT>
__global__ __launch_bounds__(256) void k_nvfp4_dequant_seg(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ row_scale, int64_t rows, int64_t cpr, int64_t nseg,
    void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t units = rows * nseg;
  for (int64_t unit = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       unit < units; unit += nwaves) {
    const int64_t row = unit / nseg;                     // uniform
    const int64_t seg = unit - row * nseg;
    const float g = row_scale[row];
    const int64_t rbase = row * cpr;
    uint32_t w[kDqSegUnroll], sb[kDqSegUnroll];
#pragma unroll
    for (int u = 0; u < kDqSegUnroll; ++u) {
      const int64_t j = seg * kDqSegChunks + u * kWave + lane;
      const bool ok = j < cpr;
      w[u] = ok ? stream_ld(packed + rbase + j) : 0u;
      sb[u] = ok ? (uint32_t)scales[(rbase + j) >> 1] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kDqSegUnroll; ++u) {
      const int64_t j = seg * kDqSegChunks + u * kWave + lane;
      float f[8];
      const float sigma = e4m3_decode_any(sb[u]);
      e2m1_unpack8_f32_hw(e2m1_canonical_zeros(w[u]), 1.0f, f);   // exact e2m1
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g;        // exact, then RN
      st8_wave<DT>(y, rbase + j - lane, rbase + cpr, lane, f);
    }
  }
}

// Segments a wave may hold in registers (1, 2, 4 or 8; 8 by default, so that
// one wave owns a whole row of up to 8192 columns: no LDS exchange, no
// barrier, no wave idling on a shorter share of the row); rows needing more
// than 4 waves x this many segments take the two-pass fallback.
#ifndef MXQ_NV_MAX_NIT
#define MXQ_NV_MAX_NIT 8
#endif

// A row kernel holding 5 to 8 segments per wave runs four of its workgroups
// per CU, one wave per SIMD each (see occupancy_lds): on the MoE sweep (rows
// of 7168 columns, 7 segments) it ran at 199 us per 36-expert chunk with four
// waves per SIMD, 209 with five (what its registers allow) and 216 with
// three.  With 4 segments (rows of 4096) it ran 2% faster uncapped.
#ifndef MXQ_NV_SEG_WG_PER_CU
#define MXQ_NV_SEG_WG_PER_CU 4
#endif
constexpr unsigned kNvSegOccupancyLds = occupancy_lds(MXQ_NV_SEG_WG_PER_CU);

template <int DT, int NIT, int WPR, bool FULL>
static void launch_seg_k(dim3 grid, hipStream_t s, const void* x, const NvSegGeom& geo,
                         int mode, const float* given, int64_t gs, const uint32_t* ta,
                         uint32_t* p, uint8_t* sc, float* rs) {
  const unsigned lds = NIT >= 5 ? kNvSegOccupancyLds : 0u;
  hipLaunchKernelGGL((k_nvfp4_quant_seg<DT, NIT, WPR, FULL>), grid, dim3(256), lds, s, x,
                     geo, mode, given, gs, ta, p, sc, rs);
}

// Every segment count a wave can hold has its own instantiation, so no wave
// keeps registers for, or computes, a segment past the end of its row (at
// K = 7168, 7 segments in 8 slots took 2% longer).  Waves that share a row
// hold more than MXQ_NV_MAX_NIT / 2 segments, since shorter rows take fewer
// waves; any count without a kernel here goes to NIT = 0, which serves every
// row length.
template <int DT, int WPR, bool FULL>
static void launch_seg_f(int nit, dim3 grid, hipStream_t s, const void* x,
                         const NvSegGeom& geo, int mode, const float* given,
                         int64_t gs, const uint32_t* ta, uint32_t* p,
                         uint8_t* sc, float* rs) {
#define MXQ_SEG_CASE(n)                                                              \
  case n:                                                                            \
    if constexpr (n <= MXQ_NV_MAX_NIT && (WPR == 1 || 2 * n > MXQ_NV_MAX_NIT)) {      \
      launch_seg_k<DT, n, WPR, FULL>(grid, s, x, geo, mode, given, gs, ta, p, sc, rs); \
      return;                                                                        \
    }                                                                                \
    break;
  switch (nit) {
    MXQ_SEG_CASE(1) MXQ_SEG_CASE(2) MXQ_SEG_CASE(3) MXQ_SEG_CASE(4)
    MXQ_SEG_CASE(5) MXQ_SEG_CASE(6) MXQ_SEG_CASE(7) MXQ_SEG_CASE(8)
    default: break;
  }
#undef MXQ_SEG_CASE
  launch_seg_k<DT, 0, WPR, FULL>(grid, s, x, geo, mode, given, gs, ta, p, sc, rs);
}

template <int DT, int WPR>
static void launch_seg_w(int nit, dim3 grid, hipStream_t s, const void* x,
                         const NvSegGeom& geo, int mode, const float* given,
                         int64_t gs, const uint32_t* ta, uint32_t* p,
                         uint8_t* sc, float* rs) {
  if (geo.bpr % 64 == 0) launch_seg_f<DT, WPR, true>(nit, grid, s, x, geo, mode, given, gs, ta, p, sc, rs);
  else launch_seg_f<DT, WPR, false>(nit, grid, s, x, geo, mode, given, gs, ta, p, sc, rs);
}

template <int DT>
static void launch_seg(int nit, int wpr, dim3 grid, hipStream_t s, const void* x,
                       const NvSegGeom& geo, int mode, const float* given,
                       int64_t gs, const uint32_t* ta, uint32_t* p,
                       uint8_t* sc, float* rs) {
  switch (wpr) {
    case 1: launch_seg_w<DT, 1>(nit, grid, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 2: launch_seg_w<DT, 2>(nit, grid, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    default: launch_seg_w<DT, 4>(nit, grid, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
  }
}

#ifndef MXQ_NVQ_UPW
#define MXQ_NVQ_UPW MXQ_UNITS_PER_WAVE
#endif
#ifndef MXQ_NVD_UPW
#define MXQ_NVD_UPW MXQ_UNITS_PER_WAVE
#endif
static dim3 grid_of(int64_t units) {
  return dim3((unsigned)(units < kMaxGridBlocks ? (units > 0 ? units : 1) : kMaxGridBlocks));
}

hipError_t launch_nvfp4_quant(const void* x, int dt, int64_t rows, int64_t K,
                              int mode, const float* given,
                              int64_t given_stride, float* scratch,
                              uint8_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t s) {
  uint32_t* ta = reinterpret_cast<uint32_t*>(scratch);
  if (mode == 2) {
    const int64_t nchunks = rows * (K / 8);
    int64_t b = (nchunks + 255) / 256;
    const int gb = (int)(b < kTensorAmaxBlocks ? b : kTensorAmaxBlocks);
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, s, ta, 0u);
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL(k_tensor_amax<DT_F32>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
      case DT_BF16: hipLaunchKernelGGL(k_tensor_amax<DT_BF16>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
      default: hipLaunchKernelGGL(k_tensor_amax<DT_F16>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
    }
  }
  const int64_t bpr = K / 16;
  if (bpr < 64) {
    int lpr = 1;
    while (lpr < bpr) lpr <<= 1;
    const int64_t rows_per_block = 4 * (kWave / lpr);
    const dim3 grid = grid_of(((rows + rows_per_block - 1) / rows_per_block + MXQ_NVQ_UPW - 1) / MXQ_NVQ_UPW);
    u32x2* p = reinterpret_cast<u32x2*>(packed);
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL(k_nvfp4_quant_short<DT_F32>, grid, dim3(256), 0, s, x, rows, bpr, lpr, mode, given, given_stride, ta, p, scales, row_scale); break;
      case DT_BF16: hipLaunchKernelGGL(k_nvfp4_quant_short<DT_BF16>, grid, dim3(256), 0, s, x, rows, bpr, lpr, mode, given, given_stride, ta, p, scales, row_scale); break;
      default: hipLaunchKernelGGL(k_nvfp4_quant_short<DT_F16>, grid, dim3(256), 0, s, x, rows, bpr, lpr, mode, given, given_stride, ta, p, scales, row_scale); break;
    }
    return hipGetLastError();
  }
  NvSegGeom geo;
  geo.rows = rows;
  geo.bpr = bpr;
  geo.cpr = 2 * bpr;
  geo.nseg = (int)((bpr + 63) / 64);
  // waves per row: the fewest (1, 2, 4) that leave each wave at most
  // MXQ_NV_MAX_NIT segments; NIT = that many segments per wave.
  int wpr = 1;
  while (wpr < 4 && geo.nseg > MXQ_NV_MAX_NIT * wpr) wpr <<= 1;
  int nit = (geo.nseg + wpr - 1) / wpr;
  if (nit > MXQ_NV_MAX_NIT) { nit = 0; wpr = 4; }         // two passes over the row
  const int64_t rows_per_block = 4 / wpr;
  const dim3 grid = grid_of(((rows + rows_per_block - 1) / rows_per_block + MXQ_NVQ_UPW - 1) / MXQ_NVQ_UPW);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  switch (dt) {
    case DT_F32: launch_seg<DT_F32>(nit, wpr, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
    case DT_BF16: launch_seg<DT_BF16>(nit, wpr, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
    default: launch_seg<DT_F16>(nit, wpr, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t rows,
                                int64_t K, void* y, int dt, hipStream_t s) {
  const int64_t cpr = K / 8;
  if (cpr >= kDqSegChunks) {
    const int64_t nseg = (cpr + kDqSegChunks - 1) / kDqSegChunks;
    const dim3 grid = grid_of((rows * nseg + 4 * MXQ_NVD_UPW - 1) / (4 * MXQ_NVD_UPW)), block(256);
    const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL(k_nvfp4_dequant_seg<DT_F32>, grid, block, 0, s, p, scales, row_scale, rows, cpr, nseg, y); break;
      case DT_BF16: hipLaunchKernelGGL(k_nvfp4_dequant_seg<DT_BF16>, grid, block, 0, s, p, scales, row_scale, rows, cpr, nseg, y); break;
      default: hipLaunchKernelGGL(k_nvfp4_dequant_seg<DT_F16>, grid, block, 0, s, p, scales, row_scale, rows, cpr, nseg, y); break;
    }
    return hipGetLastError();
  }
  NvFlatGeom geo;
  geo.nchunks = rows * cpr;
  geo.cpr = cpr;
  geo.ntiles = (geo.nchunks + kDqFlatTile - 1) / kDqFlatTile;
  geo.drow = (int32_t)(kWave / cpr);
  geo.drem = (int32_t)(kWave % cpr);
  const dim3 grid = grid_of((geo.ntiles + 4 * MXQ_NVD_UPW - 1) / (4 * MXQ_NVD_UPW)), block(256);
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_nvfp4_dequant_flat<DT_F32>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    case DT_BF16: hipLaunchKernelGGL(k_nvfp4_dequant_flat<DT_BF16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    default: hipLaunchKernelGGL(k_nvfp4_dequant_flat<DT_F16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
  }
  return hipGetLastError();
}

} // namespace mxq
