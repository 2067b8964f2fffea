// mxq_launch_gemm.h -- host-side launcher of the grouped GEMM (internal).
// Arguments are already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// fmt: FMT_MXFP4 or FMT_NVFP4; trans 0: y = x W_e^T, 1: y = x W_e.
hipError_t launch_grouped_mm(const void* x, int64_t T, const uint8_t* packed,
                             const uint8_t* scales, const float* row_scale,
                             int64_t E, int64_t N, int64_t K, const int32_t* offs,
                             int fmt, int trans, void* y, hipStream_t s);

}  // namespace mxq
