// mxq_launch.h -- host-side launchers of the libmxq kernels (internal).
// Arguments are already validated by the C ABI layer; each launcher enqueues
// its kernels on stream `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

hipError_t launch_mxfp4_quant(const void* x, int dt, int64_t rows, int64_t K,
                              int8_t* packed, uint8_t* scales, hipStream_t s);
hipError_t launch_mxfp4_dequant(const int8_t* packed, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y, int dt,
                                hipStream_t s);
hipError_t launch_nvfp4_quant(const void* x, int dt, int64_t rows, int64_t K,
                              int mode, const float* given,
                              int64_t given_stride, float* scratch,
                              uint8_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t s);
hipError_t launch_nvfp4_dequant(const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t rows,
                                int64_t K, void* y, int dt, hipStream_t s);
hipError_t launch_cache_qdq(const void* x, void* y, int dt, int64_t rows,
                            int64_t C, int fmt, int block_size, hipStream_t s);
hipError_t launch_mxfp8_quant(const void* x, int dt, int64_t rows, int64_t K,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_mxfp8_dequant(const uint8_t* codes, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y, int dt,
                                hipStream_t s);
hipError_t launch_fp4_static_qdq(const void* x, int dt, int64_t rows, int64_t K,
                                 int block_size, const float* block_amax,
                                 const float* global_amax, void* y, hipStream_t s);
hipError_t launch_kv_pages_dequant(const uint8_t* const* values, const uint8_t* const* scales,
                                   const float* const* amax, int64_t nblocks,
                                   int64_t block_tokens, int64_t H, int64_t D, void* y, int dt,
                                   hipStream_t s);
hipError_t launch_kv_quant(const void* k, int dt, int64_t S, int64_t H, int64_t D, int smooth,
                           float* head_amax, uint8_t* packed, uint8_t* scales,
                           float* row_scale, hipStream_t s);

} // namespace mxq
