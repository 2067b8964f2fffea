// mxq_hostmath.cpp -- host build of the libmxq per-chunk arithmetic
// (fp8_quantize_pack_amd/csrc/mxq_device.h), driven in the same block
// structure as the gfx950 kernels.  The CPU test-suite compares it with the
// oracle on exhaustive and edge-case inputs; the GPU tests then only have to
// establish that the kernels distribute that arithmetic over lanes correctly
// and that the GPU's IEEE operations agree with the host's.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <thread>
#include <vector>

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
    const double rg = 1.0 / (double)g;
    for (int64_t b = 0; b < K / 16; ++b) {
      float f[16];
      float a = 0.0f;
      for (int i = 0; i < 16; ++i) { f[i] = ld(x, dt, r * K + 16 * b + i); a = fmaxf(a, fabsf(f[i])); }
      float den;
      scales[r * (K / 16) + b] = (uint8_t)nvfp4_block_scale(a, g, rg, &den);
      for (int c = 0; c < 2; ++c)
        put_word(packed + r * (K / 2) + 8 * b + 4 * c, nvfp4_quant8(f + 8 * c, 1.0 / (double)den));
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

extern "C" void hm_f16_rne(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)mxq::f32_to_f16_rne(v[i]);
}

// Stress of the NVFP4 division shortcuts against IEEE float32 division on the
// host: random (x, den) pairs plus pairs built to sit on or next to an e2m1
// rounding boundary.  Returns the number of disagreements.
static uint64_t splitmix(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
extern "C" int64_t hm_nv_division_stress(int64_t n, uint64_t seed, int wide) {
  static const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  int64_t bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t r = splitmix(seed);
    // den: random float32 in [2^-40, 2^20], or sigma * 2^k (exact e4m3 times pow2)
    float den;
    if (r & 1) den = bitsf((uint32_t)(((r >> 8) % (60u << 23)) + (87u << 23)));
    else den = e4m3_decode_pos(1 + (uint32_t)((r >> 8) % 126)) * bitsf((uint32_t)((100 + (r >> 20) % 40) << 23));
    float x;
    const int kind = (int)((r >> 40) % 4);
    const float m = mids[(r >> 44) % 7];
    float t = m * den;                                 // near a midpoint
    if (kind == 0) x = bitsf((uint32_t)(splitmix(seed) % 0x7F7FFFFFu)) ;   // random
    else x = t;
    if (!wide) x = bitsf(fbits(x) & 0xFFFF0000u);      // bf16 input
    if (kind == 2) x = bitsf(fbits(x) + (wide ? 1u : 0x10000u));
    if (kind == 3) x = bitsf(fbits(x) - (wide ? 1u : 0x10000u));
    if (!(x == x) || x > 3e38f) continue;
    const float q_ref = fabsf(x) / den;
    const uint32_t want = e2m1_mag_f32(q_ref == q_ref ? q_ref : 0.0f);
    float q = (float)((double)fabsf(x) * (1.0 / (double)den));
    q = (q == q) ? q : 0.0f;
    if (e2m1_mag_f32(q) != want) ++bad;
    // block-scale chain: (a / 6) / g
    const float g = den;
    const float u_ref = (fabsf(x) / 6.0f) / g;
    const float u = (float)((double)div6_rn(fabsf(x)) * (1.0 / (double)g));
    if (fbits(u) != fbits(u_ref) && u_ref >= 1.17549435e-38f) ++bad;
  }
  return bad;
}

// Model of the gfx950 fp4 converter's rounding at scale 1 (measured on the
// chip: exact round to nearest, ties to the even code, saturating at 6):
// the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 to |q|, on a tie the one whose
// code is even.  Written from that definition, independently of
// e2m1_mag_f32.
static uint32_t e2m1_mag_rne_model(float q) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double a = fabs((double)q);
  if (a >= 6.0) return 7;                      // saturation, infinities included
  uint32_t best = 0;
  for (uint32_t c = 1; c < 8; ++c) {
    const double dc = fabs(a - grid[c]), db = fabs(a - grid[best]);
    if (dc < db || (dc == db && (c & 1u) == 0)) best = c;
  }
  return best;
}

// Every float32 magnitude below 16, both signs, and the infinities: the
// converter's ties-to-even rounding of half_down_for_rne(q) gives the
// round-half-down code of q (e2m1_mag_f32), with the sign of q.  Returns the
// number of disagreements.
static int64_t half_down_range(uint32_t b0, uint32_t b1) {
  int64_t bad = 0;
  for (uint32_t b = b0; b < b1; ++b) {
    for (uint32_t s = 0; s < 2; ++s) {
      const float q = bitsf(b | (s << 31));
      const float v = half_down_for_rne(q);
      if (e2m1_mag_rne_model(v) != e2m1_mag_f32(fabsf(q))) ++bad;
      if ((fbits(v) ^ fbits(q)) >> 31) ++bad;
    }
  }
  return bad;
}

extern "C" int64_t hm_half_down_check(void) {
  constexpr uint32_t kEnd = 0x41800001u;       // every magnitude up to 16
  constexpr int kParts = 8;
  int64_t part[kParts] = {};
  std::vector<std::thread> pool;
  for (int t = 0; t < kParts; ++t)
    pool.emplace_back([&part, t] {
      part[t] = half_down_range((uint32_t)((uint64_t)kEnd * t / kParts),
                                (uint32_t)((uint64_t)kEnd * (t + 1) / kParts));
    });
  int64_t bad = 0;
  for (int t = 0; t < kParts; ++t) { pool[t].join(); bad += part[t]; }
  if (e2m1_mag_rne_model(half_down_for_rne(bitsf(0x7F800000u))) != 7u) ++bad;
  if (e2m1_mag_rne_model(half_down_for_rne(bitsf(0xFF800000u))) != 7u) ++bad;
  return bad;
}

// The model above against the definition it states, on the grid values and
// midpoints themselves: returns the number of mismatches.
extern "C" int64_t hm_rne_model_check(void) {
  static const float pts[] = {0.0f, 0.25f, 0.5f, 0.75f, 1.0f, 1.25f, 1.5f, 1.75f,
                              2.0f, 2.5f, 3.0f, 3.5f, 4.0f, 5.0f, 6.0f, 7.0f, 100.0f};
  static const uint32_t want[] = {0, 0, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 7, 7};
  int64_t bad = 0;
  for (int i = 0; i < (int)(sizeof(pts) / sizeof(pts[0])); ++i)
    if (e2m1_mag_rne_model(pts[i]) != want[i]) ++bad;
  return bad;
}

// Every non-negative float32 below 16 (and +inf): the e2m1 code of ceil22(q)
// equals the code of q.  Returns the number of disagreements.
extern "C" int64_t hm_ceil22_check(void) {
  int64_t bad = 0;
  for (uint32_t b = 0; b <= 0x41800000u; ++b) {
    const float q = bitsf(b);
    if (e2m1_mag_f32(ceil22(q)) != e2m1_mag_f32(q)) ++bad;
    const float nq = ceil22(-q);                     // sign kept, same magnitude rounding
    if (!signbit(nq) || e2m1_mag_f32(fabsf(nq)) != e2m1_mag_f32(q)) ++bad;
  }
  if (e2m1_mag_f32(ceil22(bitsf(0x7F800000u))) != 7u) ++bad;
  return bad;
}

// Every non-negative finite float32 a: the cache scales' binary64-product
// quotients against IEEE float32 division.  a / 6 (div6_rn) must be equal for
// every a; a / 448 (div448_rn_normal) must be equal whenever the quotient is
// at least 2^-126, and in every case after the clamp to 2^-126 that follows
// it.  Returns the number of disagreements.
static int64_t scale_division_range(uint32_t lo, uint32_t hi) {
  int64_t bad = 0;
  const float tiny = 1.17549435e-38f;
  for (uint32_t b = lo; b < hi; ++b) {
    const float a = bitsf(b);
    if (fbits(div6_rn(a)) != fbits(a / 6.0f)) ++bad;
    const float q = a / 448.0f, p = div448_rn_normal(a);
    if (q >= tiny && fbits(p) != fbits(q)) ++bad;
    if (fbits(fmaxf(p, tiny)) != fbits(fmaxf(q, tiny))) ++bad;
  }
  return bad;
}

extern "C" int64_t hm_scale_division_check(void) {
  constexpr uint32_t kEnd = 0x7F800000u;       // every finite non-negative float32
  constexpr int kParts = 8;
  int64_t part[kParts] = {};
  std::vector<std::thread> pool;
  for (int t = 0; t < kParts; ++t)
    pool.emplace_back([&part, t] {
      part[t] = scale_division_range((uint32_t)((uint64_t)kEnd * t / kParts),
                                     (uint32_t)((uint64_t)kEnd * (t + 1) / kParts));
    });
  int64_t bad = 0;
  for (int t = 0; t < kParts; ++t) { pool[t].join(); bad += part[t]; }
  return bad;
}
