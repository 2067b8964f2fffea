// mxq_api_util.h -- argument checks shared by the C ABI translation units
// (internal; host code only).
#pragma once

#include <stdint.h>

#include "mxq.h"

namespace mxq {
namespace api {

inline bool bad_dtype(mxq_dtype d) { return d != MXQ_F32 && d != MXQ_BF16 && d != MXQ_F16; }

// Device pointers handed to the vector kernels must be 16-byte aligned.
inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// a * b overflows int64 (both non-negative).
inline bool mul_overflows(int64_t a, int64_t b) { return a != 0 && b > INT64_MAX / a; }

inline mxq_status launched(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_E_LAUNCH; }

}  // namespace api
}  // namespace mxq
