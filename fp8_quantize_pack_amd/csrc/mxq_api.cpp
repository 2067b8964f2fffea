// mxq_api.cpp -- the C ABI of libmxq (declared in include/mxq.h): argument
// validation on the host, then one launcher per call.  No allocation, no
// synchronization, no global state.
#include "mxq.h"

#include <stdint.h>

#include "mxq_api_util.h"
#include "mxq_launch.h"

using namespace mxq::api;

extern "C" {

int32_t mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_E_NULL: return "a required pointer is NULL";
    case MXQ_E_SHAPE: return "invalid shape: negative size or last dim not a whole number of blocks";
    case MXQ_E_DTYPE: return "unknown dtype";
    case MXQ_E_FORMAT: return "unknown cache format";
    case MXQ_E_BLOCK: return "block_size out of the range the call accepts";
    case MXQ_E_SIZE: return "rows * K overflows int64";
    case MXQ_E_LAUNCH: return "kernel launch failed";
    case MXQ_E_MODE: return "unknown NVFP4 scale mode";
    case MXQ_E_ALIGN: return "pointer not 16-byte aligned";
    case MXQ_E_SCRATCH: return "the call needs more than its static device scratch";
  }
  return "unknown status";
}

mxq_status mxq_quantize_mxfp4(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, int8_t* packed, uint8_t* scales,
                              hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 32 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(xdt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !packed || !scales) return MXQ_E_NULL;
  if (misaligned(x) || misaligned(packed)) return MXQ_E_ALIGN;
  return launched(mxq::launch_mxfp4_quant(x, (int)xdt, rows, K, packed, scales, stream));
}

mxq_status mxq_dequantize_mxfp4(const int8_t* packed, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y,
                                mxq_dtype ydt, hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 32 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(ydt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!packed || !scales || !y) return MXQ_E_NULL;
  if (misaligned(packed) || misaligned(y)) return MXQ_E_ALIGN;
  return launched(mxq::launch_mxfp4_dequant(packed, scales, rows, K, y, (int)ydt, stream));
}

mxq_status mxq_quantize_nvfp4(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, mxq_nv_mode mode, const float* given,
                              int64_t given_stride, float* scratch,
                              uint8_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 16 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(xdt)) return MXQ_E_DTYPE;
  if (mode != MXQ_NV_ROW_AMAX && mode != MXQ_NV_GIVEN && mode != MXQ_NV_TENSOR_AMAX)
    return MXQ_E_MODE;
  if (mode == MXQ_NV_GIVEN && (given_stride != 0 && given_stride != 1)) return MXQ_E_SHAPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!x || !packed || !scales || !row_scale) return MXQ_E_NULL;
  if (mode == MXQ_NV_GIVEN && !given) return MXQ_E_NULL;
  if (mode == MXQ_NV_TENSOR_AMAX && !scratch) return MXQ_E_NULL;
  if (misaligned(x) || misaligned(packed)) return MXQ_E_ALIGN;
  return launched(mxq::launch_nvfp4_quant(x, (int)xdt, rows, K, (int)mode, given,
                                          given_stride, scratch, packed, scales,
                                          row_scale, stream));
}

mxq_status mxq_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t rows,
                                int64_t K, void* y, mxq_dtype ydt,
                                hipStream_t stream) {
  if (rows < 0 || K < 0 || K % 16 != 0) return MXQ_E_SHAPE;
  if (bad_dtype(ydt)) return MXQ_E_DTYPE;
  if (mul_overflows(rows, K)) return MXQ_E_SIZE;
  if (rows == 0 || K == 0) return MXQ_OK;
  if (!packed || !scales || !row_scale || !y) return MXQ_E_NULL;
  if (misaligned(packed) || misaligned(y)) return MXQ_E_ALIGN;
  return launched(mxq::launch_nvfp4_dequant(packed, scales, row_scale, rows, K, y,
                                            (int)ydt, stream));
}

mxq_status mxq_quantize_cache(const void* x, void* y, mxq_dtype dt,
                              int64_t rows, int64_t C, mxq_format fmt,
                              int32_t block_size, hipStream_t stream) {
  if (rows < 0 || C < 0) return MXQ_E_SHAPE;
  if (bad_dtype(dt)) return MXQ_E_DTYPE;
  if (fmt != MXQ_FMT_FP8 && fmt != MXQ_FMT_MXFP4 && fmt != MXQ_FMT_NVFP4) return MXQ_E_FORMAT;
  if (block_size < 1) return MXQ_E_BLOCK;
  if (mul_overflows(rows, C)) return MXQ_E_SIZE;
  if (rows == 0 || C == 0) return MXQ_OK;
  if (!x || !y) return MXQ_E_NULL;
  return launched(mxq::launch_cache_qdq(x, y, (int)dt, rows, C, (int)fmt, block_size, stream));
}

}  // extern "C"
