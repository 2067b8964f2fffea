// mxq_api_ext.cpp -- C ABI of the MXFP8 and static two-level FP4 calls
// (declared in include/mxq.h): host-side validation, then one launcher per
// call.  No allocation, no synchronization, no global state.
#include "mxq.h"

#include <stdint.h>

#include "mxq_launch.h"

namespace {

bool bad_dtype(mxq_dtype d) { return d != MXQ_F32 && d != MXQ_BF16 && d != MXQ_F16; }
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool mul_overflows(int64_t a, int64_t b) { return a != 0 && b > INT64_MAX / a; }
mxq_status launched(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_E_LAUNCH; }

}  // namespace

extern "C" {

mxq_status mxq_quantize_mxfp8(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 32 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(xdt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !codes || !scales) return MXQ_E_NULL;
  if (misaligned(x) || misaligned(codes)) return MXQ_E_ALIGN;
  return launched(mxq::launch_mxfp8_quant(x, (int)xdt, rows, K, codes, scales, stream));
}

mxq_status mxq_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y,
                                mxq_dtype ydt, hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 32 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(ydt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!codes || !scales || !y) return MXQ_E_NULL;
  if (misaligned(codes) || misaligned(y)) return MXQ_E_ALIGN;
  return launched(mxq::launch_mxfp8_dequant(codes, scales, rows, K, y, (int)ydt, stream));
}

mxq_status mxq_fake_quantize_fp4_static(const void* x, mxq_dtype dt, int64_t rows,
                                        int64_t K, int32_t block_size,
                                        const float* block_amax,
                                        const float* global_amax, void* y,
                                        hipStream_t stream) {
  if (block_size < 8 || block_size > 1024 || (block_size & (block_size - 1)) != 0)
    return MXQ_E_BLOCK;
  if (rows < 0 || K < 0 || K % block_size != 0) return MXQ_E_SHAPE;
  if (bad_dtype(dt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !block_amax || !global_amax || !y) return MXQ_E_NULL;
  if (misaligned(x) || misaligned(y)) return MXQ_E_ALIGN;
  return launched(mxq::launch_fp4_static_qdq(x, (int)dt, rows, K, block_size, block_amax,
                                             global_amax, y, stream));
}

}  // extern "C"
