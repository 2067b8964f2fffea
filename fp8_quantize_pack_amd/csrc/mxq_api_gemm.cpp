// mxq_api_gemm.cpp -- C ABI of the grouped GEMM over packed fp4 expert
// weights (declared in include/mxq.h): argument validation on the host, then
// one launch.  No allocation, no synchronization, no global state.
#include "mxq.h"

#include <stdint.h>

#include "mxq_api_util.h"
#include "mxq_launch_gemm.h"

using namespace mxq::api;

namespace {

constexpr int64_t kTile = 128;            // N and K are whole numbers of output / reduction tiles
constexpr int64_t kMaxOutputTiles = 65535;

mxq_status check(const void* x, mxq_dtype xdt, int64_t T, const void* packed,
                 const void* scales, int64_t E, int64_t N, int64_t K,
                 const int32_t* offs, int32_t transpose, const void* y) {
  if (T < 0 || E < 0 || N <= 0 || K <= 0 || N % kTile != 0 || K % kTile != 0) return MXQ_E_SHAPE;
  if ((transpose ? K : N) / kTile > kMaxOutputTiles) return MXQ_E_SHAPE;
  if (xdt != MXQ_BF16) return MXQ_E_DTYPE;
  if (transpose != 0 && transpose != 1) return MXQ_E_MODE;
  if (mul_overflows(E, N) || mul_overflows(E * N, K) || mul_overflows(T, N > K ? N : K) ||
      T > INT32_MAX)
    return MXQ_E_SIZE;
  // one workgroup per (token-tile slot, output tile) in a 1-D grid
  if (((T + kTile - 1) / kTile + E) * ((transpose ? K : N) / kTile) > INT32_MAX) return MXQ_E_SIZE;
  if (T == 0 || E == 0) return MXQ_OK;
  if (!x || !packed || !scales || !offs || !y) return MXQ_E_NULL;
  if (misaligned(x) || misaligned(packed) || misaligned(y)) return MXQ_E_ALIGN;
  return MXQ_OK;
}

}  // namespace

extern "C" {

mxq_status mxq_grouped_mm_mxfp4(const void* x, mxq_dtype xdt, int64_t tokens,
                                const int8_t* packed, const uint8_t* scales,
                                int64_t experts, int64_t N, int64_t K,
                                const int32_t* offs, int32_t transpose, void* y,
                                hipStream_t stream) {
  const mxq_status st = check(x, xdt, tokens, packed, scales, experts, N, K, offs, transpose, y);
  if (st != MXQ_OK || tokens == 0 || experts == 0) return st;
  return launched(mxq::launch_grouped_mm(x, tokens, reinterpret_cast<const uint8_t*>(packed),
                                         scales, nullptr, experts, N, K, offs, 1, transpose, y,
                                         stream));
}

mxq_status mxq_grouped_mm_nvfp4(const void* x, mxq_dtype xdt, int64_t tokens,
                                const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t experts, int64_t N,
                                int64_t K, const int32_t* offs, int32_t transpose,
                                void* y, hipStream_t stream) {
  const mxq_status st = check(x, xdt, tokens, packed, scales, experts, N, K, offs, transpose, y);
  if (st != MXQ_OK || tokens == 0 || experts == 0) return st;
  if (!row_scale) return MXQ_E_NULL;
  return launched(mxq::launch_grouped_mm(x, tokens, packed, scales, row_scale, experts, N, K,
                                         offs, 2, transpose, y, stream));
}

}  // extern "C"
