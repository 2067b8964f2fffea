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
// Layout of the work.  One lane owns one 16-column block at a time (32 bytes
// of bfloat16 in, 8 bytes of codes and one scale byte out), so the block amax
// and the block scale need no lane exchange.  A row is owned by LPR lanes (a
// power of two, 64 once the row has 64 blocks or more), i.e. 64/LPR rows per
// wavefront; lane `sub` owns the blocks sub, sub + LPR, ...  With NIT > 0 the
// whole row stays in registers between the row-amax reduction and the
// quantization (HBM is read once); NIT == 0 is the fallback for very long
// rows, which reads the row twice.
//
// Exactness of the element step: q = RN(x / den) is needed only through the
// e2m1 decisions q > m.  The kernel forms the binary64 product x * (1 / den)
// (1 / den correctly rounded), rounds it to float32 -- which lands on the same
// side of every decision boundary as x / den (see nvfp4_quant8 in
// mxq_device.h) -- rounds that up to 22 significant bits (ceil22, again
// decision-preserving) and lets the scaled fp4 converter round half down.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

constexpr float kGlobalDiv = 2688.0f;         // E2M1_MAX * E4M3_MAX
constexpr double kHugeRecip = 0x1p800;        // stands in for 1 / 0 (see below)

struct NvRowGeom {
  int64_t rows;
  int64_t bpr;      // 16-column blocks per row = K / 16
  int lpr;          // lanes per row
  int niter;        // block iterations per lane = ceil(bpr / lpr)
};

// 16 elements (one block) as two 8-element chunks.
template <int DT> struct Raw16 { Raw8<DT> lo, hi; };

template <int DT>
__device__ __forceinline__ Raw16<DT> ld16(const void* x, int64_t blk) {
  return Raw16<DT>{ld8<DT>(x, 2 * blk), ld8<DT>(x, 2 * blk + 1)};
}
template <int DT>
__device__ __forceinline__ Raw16<DT> zero16() {
  return Raw16<DT>{zero8<DT>(), zero8<DT>()};
}

__device__ __forceinline__ float nv_row_scale(int mode, float row_amax,
                                              const float* given,
                                              int64_t given_stride, int64_t row,
                                              const uint32_t* tensor_amax) {
  if (mode == 1) return given[row * given_stride];
  if (mode == 2) return bitsf(*tensor_amax) / kGlobalDiv;
  return row_amax / kGlobalDiv;
}

template <int DT>
__device__ __forceinline__ float amax16(const Raw16<DT>& r) {
  float f[8], h[8];
  unpack8<DT>(r.lo, f);
  unpack8<DT>(r.hi, h);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fmaxf(fabsf(f[i]), fabsf(h[i])));
  return a;
}

// Quantize one block: returns the 16 codes (two words) and the scale byte.
template <int DT>
__device__ __forceinline__ void nv_quant_block(const Raw16<DT>& r, float g, double rg,
                                               uint32_t& w0, uint32_t& w1, uint32_t& sb) {
  float f[8], h[8];
  unpack8<DT>(r.lo, f);
  unpack8<DT>(r.hi, h);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fmaxf(fabsf(f[i]), fabsf(h[i])));
  float den;
  sb = nvfp4_block_scale(a, g, rg, &den);
  // 1 / den, correctly rounded; den == 0 (only with g == 0) makes every
  // non-zero element saturate and keeps 0 / 0 at code 0, as the float32
  // quotient would (inf -> code 7, NaN -> code 0).
  const double rden = (den == 0.0f) ? kHugeRecip : 1.0 / (double)den;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = ceil22((float)((double)f[i] * rden));
    h[i] = ceil22((float)((double)h[i] * rden));
  }
  w0 = e2m1_pack8_hw(f, 1.0f);
  w1 = e2m1_pack8_hw(h, 1.0f);
}

template <int DT, int NIT>
__global__ __launch_bounds__(256) void k_nvfp4_quant(
    const void* __restrict__ x, NvRowGeom geo, int mode,
    const float* __restrict__ given, int64_t given_stride,
    const uint32_t* __restrict__ tensor_amax, uint2* __restrict__ packed,
    uint8_t* __restrict__ scales, float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (geo.lpr - 1);
  const int rows_per_wave = kWave / geo.lpr;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t ngroups = (geo.rows + rows_per_wave - 1) / rows_per_wave;
  for (int64_t wg = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       wg < ngroups; wg += nwaves) {
    const int64_t row = wg * rows_per_wave + lane / geo.lpr;
    const bool row_ok = row < geo.rows;
    const int64_t rbase = row * geo.bpr;
    if constexpr (NIT > 0) {
      Raw16<DT> r[NIT];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        r[it] = (row_ok && j < geo.bpr) ? ld16<DT>(x, rbase + j) : zero16<DT>();
      }
      float amax = 0.0f;
      if (mode == 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) amax = fmaxf(amax, amax16<DT>(r[it]));
        amax = group_max_rt(amax, geo.lpr);
      }
      const float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
      const double rg = 1.0 / (double)g;
      if (row_ok && sub == 0) row_scale[row] = g;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        if (row_ok && j < geo.bpr) {
          uint32_t w0, w1, sb;
          nv_quant_block<DT>(r[it], g, rg, w0, w1, sb);
          __builtin_nontemporal_store(w0, &packed[rbase + j].x);
          __builtin_nontemporal_store(w1, &packed[rbase + j].y);
          scales[rbase + j] = (uint8_t)sb;
        }
      }
    } else {
      float amax = 0.0f;
      if (mode == 0) {
        for (int it = 0; it < geo.niter; ++it) {
          const int64_t j = sub + (int64_t)it * geo.lpr;
          if (row_ok && j < geo.bpr) amax = fmaxf(amax, amax16<DT>(ld16<DT>(x, rbase + j)));
        }
        amax = group_max_rt(amax, geo.lpr);
      }
      const float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
      const double rg = 1.0 / (double)g;
      if (row_ok && sub == 0) row_scale[row] = g;
      for (int it = 0; it < geo.niter; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        if (row_ok && j < geo.bpr) {
          uint32_t w0, w1, sb;
          nv_quant_block<DT>(ld16<DT>(x, rbase + j), g, rg, w0, w1, sb);
          __builtin_nontemporal_store(w0, &packed[rbase + j].x);
          __builtin_nontemporal_store(w1, &packed[rbase + j].y);
          scales[rbase + j] = (uint8_t)sb;
        }
      }
    }
  }
}

// Whole-tensor amax for the one-tensor-scale mode: a grid-stride max over all
// chunks, reduced per wave and combined with an integer atomic max on the bit
// patterns (non-negative floats order like their patterns).
template <int DT>
__global__ __launch_bounds__(256) void k_tensor_amax(const void* __restrict__ x,
                                                     int64_t nchunks,
                                                     uint32_t* __restrict__ out) {
  float amax = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    float f[8];
    unpack8<DT>(ld8<DT>(x, c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = group_max<64>(amax);
  if ((threadIdx.x & 63) == 0) atomicMax(out, fbits(amax));
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

// Dequantization works on 8-element chunks (one packed dword, half a block)
// so that every load and store instruction of a wavefront is contiguous:
// lane `sub` of a row owns the chunks sub, sub + LPR, ..., kDqUnroll of them
// in flight at a time.
struct NvChunkGeom {
  int64_t rows;
  int64_t cpr;      // 8-element chunks per row = K / 8
  int lpr;          // lanes per row (>= 2, a power of two)
  int niter;        // ceil(cpr / lpr)
};

constexpr int kDqUnroll = 4;

template <int DT>
__global__ __launch_bounds__(256) void k_nvfp4_dequant(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ row_scale, NvChunkGeom geo, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (geo.lpr - 1);
  const int rows_per_wave = kWave / geo.lpr;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t ngroups = (geo.rows + rows_per_wave - 1) / rows_per_wave;
  for (int64_t wg = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       wg < ngroups; wg += nwaves) {
    const int64_t row = wg * rows_per_wave + lane / geo.lpr;
    if (row >= geo.rows) continue;
    const int64_t rbase = row * geo.cpr;
    const float g = row_scale[row];
    for (int it0 = 0; it0 < geo.niter; it0 += kDqUnroll) {
      uint32_t w[kDqUnroll], sb[kDqUnroll];
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t j = sub + (int64_t)(it0 + u) * geo.lpr;
        const bool ok = j < geo.cpr;
        w[u] = ok ? __builtin_nontemporal_load(packed + rbase + j) : 0u;
        sb[u] = ok ? (uint32_t)scales[(rbase + j) >> 1] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t j = sub + (int64_t)(it0 + u) * geo.lpr;
        if (j >= geo.cpr) continue;
        float f[8];
        if constexpr (DT == DT_F16) {
          nvfp4_dequant8(w[u], sb[u], g, f);
        } else {
          const float sigma = e4m3_decode_any(sb[u]);
          e2m1_unpack8_f32_hw(e2m1_canonical_zeros(w[u]), 1.0f, f);   // exact e2m1
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g;        // exact, then RN
        }
        st8<DT>(y, rbase + j, f);
      }
    }
  }
}

static NvRowGeom nv_geom(int64_t rows, int64_t K) {
  NvRowGeom g;
  g.rows = rows;
  g.bpr = K / 16;
  int lpr = 1;
  while (lpr < 64 && lpr < g.bpr) lpr <<= 1;
  g.lpr = lpr;
  g.niter = (int)((g.bpr + lpr - 1) / lpr);
  return g;
}

static int nv_grid(const NvRowGeom& g) {
  const int64_t rows_per_wave = kWave / g.lpr;
  const int64_t waves = (g.rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t max_blocks = 256 * 8;
  int64_t b = (waves + 3) / 4;
  return (int)(b < max_blocks ? (b > 0 ? b : 1) : max_blocks);
}

template <int DT>
static void launch_nvq(int nit, dim3 grid, hipStream_t s, const void* x,
                       NvRowGeom geo, int mode, const float* given,
                       int64_t gs, const uint32_t* ta, uint2* p,
                       uint8_t* sc, float* rs) {
  const dim3 block(256);
  switch (nit) {
    case 1: hipLaunchKernelGGL((k_nvfp4_quant<DT, 1>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 2: hipLaunchKernelGGL((k_nvfp4_quant<DT, 2>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 4: hipLaunchKernelGGL((k_nvfp4_quant<DT, 4>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 8: hipLaunchKernelGGL((k_nvfp4_quant<DT, 8>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    default: hipLaunchKernelGGL((k_nvfp4_quant<DT, 0>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
  }
}

hipError_t launch_nvfp4_quant(const void* x, int dt, int64_t rows, int64_t K,
                              int mode, const float* given,
                              int64_t given_stride, float* scratch,
                              uint8_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t s) {
  const NvRowGeom geo = nv_geom(rows, K);
  uint32_t* ta = reinterpret_cast<uint32_t*>(scratch);
  if (mode == 2) {
    const int64_t nchunks = rows * (K / 8);
    int64_t b = (nchunks + 255) / 256;
    const int gb = (int)(b < 1024 ? b : 1024);
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, s, ta, 0u);
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL(k_tensor_amax<DT_F32>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
      case DT_BF16: hipLaunchKernelGGL(k_tensor_amax<DT_BF16>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
      default: hipLaunchKernelGGL(k_tensor_amax<DT_F16>, dim3(gb), dim3(256), 0, s, x, nchunks, ta); break;
    }
  }
  // registers per lane hold NIT blocks (16 elements each): up to 8 (rows of
  // 8192 columns when LPR = 64); longer rows take the two-pass fallback.
  int nit = 1;
  while (nit < geo.niter) nit <<= 1;
  const int nit_max = (dt == DT_F32) ? 4 : 8;
  if (nit > nit_max) nit = 0;
  const dim3 grid(nv_grid(geo));
  uint2* p = reinterpret_cast<uint2*>(packed);
  switch (dt) {
    case DT_F32: launch_nvq<DT_F32>(nit, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
    case DT_BF16: launch_nvq<DT_BF16>(nit, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
    default: launch_nvq<DT_F16>(nit, grid, s, x, geo, mode, given, given_stride, ta, p, scales, row_scale); break;
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t rows,
                                int64_t K, void* y, int dt, hipStream_t s) {
  NvChunkGeom geo;
  geo.rows = rows;
  geo.cpr = K / 8;
  int lpr = 2;
  while (lpr < 64 && lpr < geo.cpr) lpr <<= 1;
  geo.lpr = lpr;
  geo.niter = (int)((geo.cpr + lpr - 1) / lpr);
  const int64_t waves = (rows + (kWave / lpr) - 1) / (kWave / lpr);
  int64_t nb = (waves + 3) / 4;
  const dim3 grid((unsigned)(nb < 2048 ? (nb > 0 ? nb : 1) : 2048)), block(256);
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_nvfp4_dequant<DT_F32>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    case DT_BF16: hipLaunchKernelGGL(k_nvfp4_dequant<DT_BF16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    default: hipLaunchKernelGGL(k_nvfp4_dequant<DT_F16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
  }
  return hipGetLastError();
}

} // namespace mxq
