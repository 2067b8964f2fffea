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
// Layout of the work.  A row is owned by LPR lanes (a power of two, 64 for
// rows of 512 columns or more), i.e. 64/LPR rows per wavefront; lane `sub` of
// a row owns the chunks sub, sub + LPR, ...  Two neighbouring lanes own one
// 16-column block.  With NIT > 0 the whole row stays in registers between the
// row-amax reduction and the quantization (HBM is read once); NIT == 0 is the
// fallback for very long rows, which reads the row twice.
#include "mxq_kernel_common.h"
#include "mxq_launch.h"

namespace mxq {

constexpr float kE4m3MinSub = 0.001953125f;   // 2^-9, E4M3_MIN_SUBNORMAL
constexpr float kE4m3Max = 448.0f;            // E4M3_MAX
constexpr float kGlobalDiv = 2688.0f;         // E2M1_MAX * E4M3_MAX

struct NvRowGeom {
  int64_t rows;
  int64_t cpr;      // chunks (of 8 elements) per row = K / 8
  int lpr;          // lanes per row
  int niter;        // chunk iterations per lane = ceil(cpr / lpr)
};

// Quantize one 8-element chunk whose 16-column block is shared with the
// neighbouring lane; returns the packed word and the block-scale byte.
__device__ __forceinline__ uint32_t nv_quant_chunk(const float f[8], float g,
                                                   uint32_t& sb_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  a = group_max<2>(a);                               // 16-column block amax
  float den;
  sb_out = nvfp4_block_scale(a, g, &den);
  return nvfp4_quant8(f, den);
}

__device__ __forceinline__ float nv_row_scale(int mode, float row_amax,
                                              const float* given,
                                              int64_t given_stride, int64_t row,
                                              const uint32_t* tensor_amax) {
  if (mode == 1) return given[row * given_stride];
  if (mode == 2) return bitsf(*tensor_amax) / kGlobalDiv;
  return row_amax / kGlobalDiv;
}

template <int DT, int NIT>
__global__ __launch_bounds__(256) void k_nvfp4_quant(
    const void* __restrict__ x, NvRowGeom geo, int mode,
    const float* __restrict__ given, int64_t given_stride,
    const uint32_t* __restrict__ tensor_amax, uint32_t* __restrict__ packed,
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
    const int64_t rbase = row * geo.cpr;
    if constexpr (NIT > 0) {
      Raw8<DT> r[NIT];
      float amax = 0.0f;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        r[it] = (row_ok && j < geo.cpr) ? ld8<DT>(x, rbase + j) : zero8<DT>();
      }
      if (mode == 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          float f[8];
          unpack8<DT>(r[it], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
        }
        amax = group_max_rt(amax, geo.lpr);
      }
      const float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
      if (row_ok && sub == 0) row_scale[row] = g;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        if (it * geo.lpr >= geo.cpr) break;          // uniform across the wave
        float f[8];
        unpack8<DT>(r[it], f);
        uint32_t sb;
        const uint32_t word = nv_quant_chunk(f, g, sb);
        if (row_ok && j < geo.cpr) {
          __builtin_nontemporal_store(word, packed + rbase + j);
          if ((sub & 1) == 0) scales[(rbase + j) >> 1] = (uint8_t)sb;
        }
      }
    } else {
      float amax = 0.0f;
      if (mode == 0) {
        for (int it = 0; it < geo.niter; ++it) {
          const int64_t j = sub + (int64_t)it * geo.lpr;
          if (row_ok && j < geo.cpr) {
            float f[8];
            unpack8<DT>(ld8<DT>(x, rbase + j), f);
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
          }
        }
        amax = group_max_rt(amax, geo.lpr);
      }
      const float g = row_ok ? nv_row_scale(mode, amax, given, given_stride, row, tensor_amax) : 1.0f;
      if (row_ok && sub == 0) row_scale[row] = g;
      for (int it = 0; it < geo.niter; ++it) {
        const int64_t j = sub + (int64_t)it * geo.lpr;
        const bool ok = row_ok && j < geo.cpr;
        float f[8];
        unpack8<DT>(ok ? ld8<DT>(x, rbase + j) : zero8<DT>(), f);
        uint32_t sb;
        const uint32_t word = nv_quant_chunk(f, g, sb);
        if (ok) {
          __builtin_nontemporal_store(word, packed + rbase + j);
          if ((sub & 1) == 0) scales[(rbase + j) >> 1] = (uint8_t)sb;
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

template <int DT>
__global__ __launch_bounds__(256) void k_nvfp4_dequant(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ row_scale, NvRowGeom geo, void* __restrict__ y) {
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
    for (int it = 0; it < geo.niter; ++it) {
      const int64_t j = sub + (int64_t)it * geo.lpr;
      if (j >= geo.cpr) break;
      const uint32_t w = __builtin_nontemporal_load(packed + rbase + j);
      float f[8];
      nvfp4_dequant8(w, scales[(rbase + j) >> 1], g, f);
      st8<DT>(y, rbase + j, f);
    }
  }
}

static NvRowGeom nv_geom(int64_t rows, int64_t K) {
  NvRowGeom g;
  g.rows = rows;
  g.cpr = K / 8;
  int lpr = 2;
  while (lpr < 64 && lpr < g.cpr) lpr <<= 1;
  g.lpr = lpr;
  g.niter = (int)((g.cpr + lpr - 1) / lpr);
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
                       int64_t gs, const uint32_t* ta, uint32_t* p,
                       uint8_t* sc, float* rs) {
  const dim3 block(256);
  switch (nit) {
    case 1: hipLaunchKernelGGL((k_nvfp4_quant<DT, 1>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 2: hipLaunchKernelGGL((k_nvfp4_quant<DT, 2>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 4: hipLaunchKernelGGL((k_nvfp4_quant<DT, 4>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 8: hipLaunchKernelGGL((k_nvfp4_quant<DT, 8>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
    case 16: hipLaunchKernelGGL((k_nvfp4_quant<DT, 16>), grid, block, 0, s, x, geo, mode, given, gs, ta, p, sc, rs); break;
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
  // registers per lane hold NIT chunks: 16-bit inputs up to 16, float32 up to 8
  int nit = 1;
  while (nit < geo.niter) nit <<= 1;
  const int nit_max = (dt == DT_F32) ? 8 : 16;
  if (nit > nit_max) nit = 0;
  const dim3 grid(nv_grid(geo));
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
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
  const NvRowGeom geo = nv_geom(rows, K);
  const dim3 grid(nv_grid(geo)), block(256);
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(k_nvfp4_dequant<DT_F32>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    case DT_BF16: hipLaunchKernelGGL(k_nvfp4_dequant<DT_BF16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
    default: hipLaunchKernelGGL(k_nvfp4_dequant<DT_F16>, grid, block, 0, s, p, scales, row_scale, geo, y); break;
  }
  return hipGetLastError();
}

} // namespace mxq
