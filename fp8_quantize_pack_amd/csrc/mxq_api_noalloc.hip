// mxq_api_noalloc.hip -- mxq_quantize_kv_nvfp4_noalloc (include/mxq.h): the
// per-head NVFP4 KV quantization with its per-head amax scratch taken from a
// library-owned device array instead of a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, serving loops, harnesses
// that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol, so the address the
// kernels get is looked up once per device with hipGetSymbolAddress and
// cached; the kernels receive that pointer exactly as they receive the
// caller's workspace in mxq_quantize_kv_nvfp4.  The quantizer clears the
// scratch words itself with a fill kernel on every call (no memset), so the
// contents a previous call left behind do not matter; calls that overlap on
// one GPU (different streams at the same time) share the array and race.
#include <mutex>

#include "mxq.h"
#include "mxq_api_util.h"
#include "mxq_launch.h"

// Scratch words per head: the quantizer gathers each head's maximum in 32
// slots (slot-major), 128 KiB for MXQ_NOALLOC_KV_MAX_HEADS = 1024 heads.
static __device__ __align__(256) float scratch[MXQ_NOALLOC_KV_MAX_HEADS * 32];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current); nullptr if the runtime cannot give it.
float* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = static_cast<float*>(p);
  }
  return g_ptr[dev];
}

}  // namespace

using namespace mxq::api;

extern "C" mxq_status mxq_quantize_kv_nvfp4_noalloc(const void* k, mxq_dtype dt, int64_t tokens,
                                                    int64_t heads, int64_t head_dim,
                                                    int32_t smooth, uint8_t* packed,
                                                    uint8_t* scales, float* row_scale,
                                                    hipStream_t stream) {
  if (tokens < 0 || heads < 0 || heads > 4096) return MXQ_E_SHAPE;
  if (head_dim < 16 || head_dim > 512 || (head_dim & (head_dim - 1)) != 0) return MXQ_E_SHAPE;
  if (bad_dtype(dt)) return MXQ_E_DTYPE;
  if (smooth != 0 && smooth != 1) return MXQ_E_MODE;
  if (mul_overflows(tokens, heads) || mul_overflows(tokens * heads, head_dim)) return MXQ_E_SIZE;
  if (heads > MXQ_NOALLOC_KV_MAX_HEADS) return MXQ_E_SCRATCH;
  if (tokens == 0 || heads == 0) return MXQ_OK;
  if (!k || !packed || !scales || !row_scale) return MXQ_E_NULL;
  if (misaligned(k) || misaligned(packed)) return MXQ_E_ALIGN;
  float* ha = device_scratch();
  if (!ha) return MXQ_E_LAUNCH;
  return launched(mxq::launch_kv_quant(k, (int)dt, tokens, heads, head_dim, smooth, ha, packed,
                                       scales, row_scale, stream));
}
