// k_roofline_ref.hip -- plain streaming kernels that give the practical HBM
// ceiling the codec kernels are compared with: copy (read + write), read only
// and write only; and a shader clock probe.  They move 16-byte chunks with the same non-temporal vector
// accesses and the same wave-tile mapping as the codec kernels (in step u of
// a tile lane l owns chunk tile * U * 64 + u * 64 + l, so every wave
// instruction touches one contiguous 1 KiB range; four waves per workgroup,
// one tile per wave, one workgroup per four tiles up to the grid cap), and do
// no arithmetic.  They are measurement references, not part of the codec.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_roofline.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int64_t kMaxBlocks = 256 * 1024;

template <int U>
__global__ __launch_bounds__(64 * kWaves) void k_copy(const v4u* __restrict__ src,
                                                      v4u* __restrict__ dst, int64_t nchunks,
                                                      int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < ntiles; t += nw) {
    const int64_t c0 = t * (U * kWave) + lane;
    v4u r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      r[u] = c < nchunks ? __builtin_nontemporal_load(src + c) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < nchunks) __builtin_nontemporal_store(r[u], dst + c);
    }
  }
}

// Reads every chunk and folds it into an XOR that is stored only when it
// equals `magic` (which the caller picks so that it practically never does):
// the loads cannot be dropped, and nothing is written.
template <int U>
__global__ __launch_bounds__(64 * kWaves) void k_read(const v4u* __restrict__ src,
                                                      int64_t nchunks, int64_t ntiles,
                                                      uint32_t magic, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  uint32_t acc = 0u;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < ntiles; t += nw) {
    const int64_t c0 = t * (U * kWave) + lane;
    v4u r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      r[u] = c < nchunks ? __builtin_nontemporal_load(src + c) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  if (acc == magic) sink[0] = acc;
}

template <int U>
__global__ __launch_bounds__(64 * kWaves) void k_fill(v4u* __restrict__ dst, int64_t nchunks,
                                                      int64_t ntiles, uint32_t value) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const v4u v = {value, value, value, value};
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < ntiles; t += nw) {
    const int64_t c0 = t * (U * kWave) + lane;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave;
      if (c < nchunks) __builtin_nontemporal_store(v, dst + c);
    }
  }
}

// Shader clock probe: every workgroup (one wave) reads the shader cycle
// counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around
// a chain of `iters` dependent VALU operations; lane 0 stores both
// differences, so that their ratio is the mean shader clock over the window.
__global__ __launch_bounds__(64) void k_clock(uint64_t* __restrict__ out, int32_t iters) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float v = (float)threadIdx.x;
  for (int32_t i = 0; i < iters; ++i) v = __builtin_fmaf(v, 0.999f, 0.5f);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (v == -1.0f) out[0] = 0;      // keeps the chain; v stays positive
}

int grid_for(int64_t ntiles) {
  const int64_t b = (ntiles + kWaves - 1) / kWaves;
  return (int)(b < kMaxBlocks ? (b > 0 ? b : 1) : kMaxBlocks);
}

int check(const void* p, int64_t bytes, int32_t unroll) {
  if (bytes < 0 || bytes % 16) return MXQ_REF_E_SHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return MXQ_REF_E_UNROLL;
  if (bytes && !p) return MXQ_REF_E_NULL;
  if (reinterpret_cast<uintptr_t>(p) % 16) return MXQ_REF_E_ALIGN;
  return MXQ_REF_OK;
}

#define MXQ_REF_DISPATCH(KERNEL, U, ...)                                              \
  switch (U) {                                                                        \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;                        \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;                        \
    case 4: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;                        \
    default: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;                       \
  }

}  // namespace

extern "C" {

int mxq_ref_copy(const void* src, void* dst, int64_t bytes, int32_t unroll,
                 hipStream_t stream) {
  int st = check(src, bytes, unroll);
  if (st == MXQ_REF_OK) st = check(dst, bytes, unroll);
  if (st != MXQ_REF_OK || bytes == 0) return st;
  const int64_t n = bytes / 16, tiles = (n + unroll * kWave - 1) / (unroll * kWave);
  MXQ_REF_DISPATCH(k_copy, unroll, dim3(grid_for(tiles)), dim3(64 * kWaves), 0, stream,
                   static_cast<const v4u*>(src), static_cast<v4u*>(dst), n, tiles);
  return hipGetLastError() == hipSuccess ? MXQ_REF_OK : MXQ_REF_E_LAUNCH;
}

int mxq_ref_read(const void* src, int64_t bytes, int32_t unroll, uint32_t magic,
                 uint32_t* sink, hipStream_t stream) {
  int st = check(src, bytes, unroll);
  if (st == MXQ_REF_OK && !sink) st = MXQ_REF_E_NULL;
  if (st != MXQ_REF_OK || bytes == 0) return st;
  const int64_t n = bytes / 16, tiles = (n + unroll * kWave - 1) / (unroll * kWave);
  MXQ_REF_DISPATCH(k_read, unroll, dim3(grid_for(tiles)), dim3(64 * kWaves), 0, stream,
                   static_cast<const v4u*>(src), n, tiles, magic, sink);
  return hipGetLastError() == hipSuccess ? MXQ_REF_OK : MXQ_REF_E_LAUNCH;
}

int mxq_ref_fill(void* dst, int64_t bytes, uint32_t value, int32_t unroll,
                 hipStream_t stream) {
  const int st = check(dst, bytes, unroll);
  if (st != MXQ_REF_OK || bytes == 0) return st;
  const int64_t n = bytes / 16, tiles = (n + unroll * kWave - 1) / (unroll * kWave);
  MXQ_REF_DISPATCH(k_fill, unroll, dim3(grid_for(tiles)), dim3(64 * kWaves), 0, stream,
                   static_cast<v4u*>(dst), n, tiles, value);
  return hipGetLastError() == hipSuccess ? MXQ_REF_OK : MXQ_REF_E_LAUNCH;
}

int mxq_ref_clock(uint64_t* out, int32_t blocks, int32_t iters, hipStream_t stream) {
  if (!out) return MXQ_REF_E_NULL;
  if (reinterpret_cast<uintptr_t>(out) % 8) return MXQ_REF_E_ALIGN;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24)) return MXQ_REF_E_SHAPE;
  hipLaunchKernelGGL(k_clock, dim3(blocks), dim3(64), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? MXQ_REF_OK : MXQ_REF_E_LAUNCH;
}

}  // extern "C"
