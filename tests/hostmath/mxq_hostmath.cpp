// mxq_hostmath.cpp -- host build of the libmxq per-chunk arithmetic
// (fp8_quantize_pack_amd/csrc/mxq_device.h), driven in the same block
// structure as the gfx950 kernels.  The CPU test-suite compares it with the
// oracle on exhaustive and edge-case inputs; the GPU tests then only have to
// establish that the kernels distribute that arithmetic over lanes correctly
// and that the GPU's IEEE operations agree with the host's.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "mxq_device.h"

using namespace mxq;

static float ld(const void* x, int dt, int64_t i) {
  if (dt == DT_F32) return ((const float*)x)[i];
  uint32_t h = ((const uint16_t*)x)[i];
  return dt == DT_BF16 ? bitsf(h << 16) : f16_to_f32(h);
}

static void st(void* y, int dt, int64_t i, float v) {
  if (dt == DT_F32) ((float*)y)[i] = v;
  else if (dt == DT_BF16) ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_rne(v);
  else ((uint16_t*)y)[i] = (uint16_t)f32_to_f16_rne(v);
}

static void put_word(uint8_t* p, uint32_t w) { memcpy(p, &w, 4); }
static uint32_t get_word(const uint8_t* p) { uint32_t w; memcpy(&w, p, 4); return w; }

extern "C" {

void hm_quantize_mxfp4(const void* x, int dt, int64_t rows, int64_t K,
                       uint8_t* packed, uint8_t* scales) {
  const int64_t nblk = rows * K / 32;
  for (int64_t b = 0; b < nblk; ++b) {
    float f[32];
    float a = 0.0f;
    for (int i = 0; i < 32; ++i) { f[i] = ld(x, dt, 32 * b + i); a = fmaxf(a, fabsf(f[i])); }
    const uint32_t sb = mxfp4_scale_byte(a);
    scales[b] = (uint8_t)sb;
    for (int c = 0; c < 4; ++c) put_word(packed + 16 * b + 4 * c, mxfp4_quant8(f + 8 * c, sb, dt == DT_F32));
  }
}

void hm_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                         int64_t K, void* y, int dt) {
  const int64_t nchunks = rows * K / 8;
  for (int64_t c = 0; c < nchunks; ++c) {
    float f[8];
    mxfp4_dequant8(get_word(packed + 4 * c), scales[c / 4], f);
    for (int i = 0; i < 8; ++i) st(y, dt, 8 * c + i, f[i]);
  }
}

void hm_quantize_nvfp4(const void* x, int dt, int64_t rows, int64_t K, int mode,
                       const float* given, int64_t given_stride, uint8_t* packed,
                       uint8_t* scales, float* row_scale) {
  float tensor_amax = 0.0f;
  if (mode == 2)
    for (int64_t i = 0; i < rows * K; ++i) tensor_amax = fmaxf(tensor_amax, fabsf(ld(x, dt, i)));
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) amax = fmaxf(amax, fabsf(ld(x, dt, r * K + k)));
    const float g = mode == 1 ? given[r * given_stride]
                  : mode == 2 ? tensor_amax / 2688.0f : amax / 2688.0f;
    row_scale[r] = g;
    for (int64_t b = 0; b < K / 16; ++b) {
      float f[16];
      float a = 0.0f;
      for (int i = 0; i < 16; ++i) { f[i] = ld(x, dt, r * K + 16 * b + i); a = fmaxf(a, fabsf(f[i])); }
      float den;
      scales[r * (K / 16) + b] = (uint8_t)nvfp4_block_scale(a, g, &den);
      for (int c = 0; c < 2; ++c)
        put_word(packed + r * (K / 2) + 8 * b + 4 * c, nvfp4_quant8(f + 8 * c, den));
    }
  }
}

void hm_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales,
                         const float* row_scale, int64_t rows, int64_t K, void* y, int dt) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < K / 8; ++j) {
      const int64_t c = r * (K / 8) + j;
      float f[8];
      nvfp4_dequant8(get_word(packed + 4 * c), scales[c / 2], row_scale[r], f);
      for (int i = 0; i < 8; ++i) st(y, dt, 8 * c + i, f[i]);
    }
}

void hm_quantize_cache(const void* x, void* y, int dt, int64_t rows, int64_t C,
                       int fmt, int64_t B) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c0 = 0; c0 < C; c0 += B) {
      const int64_t n = C - c0 < B ? C - c0 : B;
      float a = 0.0f;
      for (int64_t k = 0; k < n; ++k) a = fmaxf(a, fabsf(ld(x, dt, r * C + c0 + k)));
      const CacheGroupScale gs = cache_scale(fmt, a);
      for (int64_t k = 0; k < n; ++k)
        st(y, dt, r * C + c0 + k, cache_qdq1(fmt, dt == DT_F32, ld(x, dt, r * C + c0 + k), gs));
    }
}

// element helpers over arrays
void hm_e4m3_encode_pos(const float* u, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)e4m3_encode_pos(u[i]);
}
void hm_e4m3_round_value(const float* r, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_round_value(r[i]);
}
void hm_pow2_ceil(const float* v, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = pow2_ceil(v[i]);
}
void hm_bf16_rne(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)f32_to_bf16_rne(v[i]);
}

}  // extern "C"
