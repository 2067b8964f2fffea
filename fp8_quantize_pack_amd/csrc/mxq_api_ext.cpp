// mxq_api_ext.cpp -- C ABI of the MXFP8, static two-level FP4 and NVFP4 KV
// cache calls (declared in include/mxq.h): host-side validation, then one
// launcher per call.  No allocation, no synchronization, no global state.
#include "mxq.h"

#include <stdint.h>

#include "mxq_api_util.h"
#include "mxq_launch.h"

using namespace mxq::api;

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

mxq_status mxq_dequantize_kv_pages_nvfp4(const uint8_t* const* values,
                                         const uint8_t* const* scales,
                                         const float* const* amax, int64_t num_blocks,
                                         int64_t block_tokens, int64_t heads,
                                         int64_t head_dim, void* y, mxq_dtype ydt,
                                         hipStream_t stream) {
  if (num_blocks < 0 || block_tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 16 != 0)
    return MXQ_E_SHAPE;
  if (bad_dtype(ydt)) return MXQ_E_DTYPE;
  if (mul_overflows(num_blocks, block_tokens) || mul_overflows(num_blocks * block_tokens, heads) ||
      mul_overflows(num_blocks * block_tokens * heads, head_dim))
    return MXQ_E_SIZE;
  if (num_blocks == 0 || block_tokens == 0 || heads == 0 || head_dim == 0) return MXQ_OK;
  if (!values || !scales || !amax || !y) return MXQ_E_NULL;
  if (misaligned(y)) return MXQ_E_ALIGN;
  return launched(mxq::launch_kv_pages_dequant(values, scales, amax, num_blocks, block_tokens,
                                               heads, head_dim, y, (int)ydt, stream));
}

mxq_status mxq_quantize_kv_nvfp4(const void* k, mxq_dtype dt, int64_t tokens, int64_t heads,
                                 int64_t head_dim, int32_t smooth, float* head_amax,
                                 uint8_t* packed, uint8_t* scales, float* row_scale,
                                 hipStream_t stream) {
  if (tokens < 0 || heads < 0 || heads > 4096) return MXQ_E_SHAPE;
  if (head_dim < 16 || head_dim > 512 || (head_dim & (head_dim - 1)) != 0) return MXQ_E_SHAPE;
  if (bad_dtype(dt)) return MXQ_E_DTYPE;
  if (smooth != 0 && smooth != 1) return MXQ_E_MODE;
  if (mul_overflows(tokens, heads) || mul_overflows(tokens * heads, head_dim)) return MXQ_E_SIZE;
  if (tokens == 0 || heads == 0) return MXQ_OK;
  if (!k || !head_amax || !packed || !scales || !row_scale) return MXQ_E_NULL;
  if (misaligned(k) || misaligned(packed)) return MXQ_E_ALIGN;
  return launched(mxq::launch_kv_quant(k, (int)dt, tokens, heads, head_dim, smooth, head_amax,
                                       packed, scales, row_scale, stream));
}

}  // extern "C"
