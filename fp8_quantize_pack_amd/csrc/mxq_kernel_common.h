// mxq_kernel_common.h -- device-only building blocks shared by the libmxq
// kernels: 16-byte vector loads and stores of 8-element chunks, and max
// reductions across small lane groups of a 64-wide wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.h"

namespace mxq {

constexpr int kWave = 64;

// Grid size of the streaming kernels: workgroups of 256 threads (4 waves).
// The weight kernels launch one workgroup per unit of work, up to
// kMaxGridBlocks, and loop only beyond that: with more workgroups than fit on
// the chip at once the dispatcher hands out work as CUs free up, which
// balances the XCDs and leaves no tail of workgroups that did not fit in the
// first round (a grid of exactly the resident count is right only while the
// register budget allows that many).  The cache kernels give each wave a few
// row groups, with at least kCacheGridBlocks workgroups when there is work
// for that many.
#ifndef MXQ_BLOCKS_PER_CU
#define MXQ_BLOCKS_PER_CU 1024
#endif
constexpr int64_t kMaxGridBlocks = 256 * MXQ_BLOCKS_PER_CU;
#ifndef MXQ_CACHE_BLOCKS_PER_CU
#define MXQ_CACHE_BLOCKS_PER_CU 8
#endif
constexpr int64_t kCacheGridBlocks = 256 * MXQ_CACHE_BLOCKS_PER_CU;
// Work units (wave tiles or row groups) each wave of a streaming kernel takes
// in turn; the grid has units / (units per wave) waves.  One unit per wave
// measured fastest for every kernel but the static FP4 round trip (which
// sets its own).
#ifndef MXQ_UNITS_PER_WAVE
#define MXQ_UNITS_PER_WAVE 1
#endif

// Dynamic LDS to ask for at launch, never touched by the kernel, so that at
// most `wg` workgroups share a CU's 160 KB (a multiple of the 512-byte LDS
// allocation granule).  Registers alone let most streaming kernels run eight
// waves per SIMD; the two quantizers that measured faster with fewer take this.
constexpr unsigned occupancy_lds(unsigned wg) { return (160u * 1024u / wg) & ~511u; }

// Streaming inputs and outputs are touched once: their global accesses carry
// the non-temporal hint unless MXQ_TEMPORAL is defined.
template <typename T>
__device__ __forceinline__ T stream_ld(const T* p) {
#ifdef MXQ_TEMPORAL
  return *p;
#else
  return __builtin_nontemporal_load(p);
#endif
}
template <typename T>
__device__ __forceinline__ void stream_st(T v, T* p) {
#ifdef MXQ_TEMPORAL
  *p = v;
#else
  __builtin_nontemporal_store(v, p);
#endif
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 value of an e4m3fn byte, branch-free: the hardware e4m3 converter
// on the magnitude (exact for every finite byte; NaN for 0x7F) and the sign
// set by hand, so that 0x80 is -0.  Finite bytes decode bit for bit as
// e4m3_decode_any does; a NaN byte gives the hardware's NaN, which every
// product with it propagates whatever the payload.  For code that must stay
// one basic block (the GEMM's dequantization between its MFMAs): the case
// split of e4m3_decode_any compiles to divergent branches, which there cost
// 17% of the NVFP4 GEMM, while in the memory-bound dequantizers the branches
// (skipped whole by waves without NaN or subnormal scales) are cheaper than
// the converter.
__device__ __forceinline__ float e4m3_decode_hw(uint32_t b) {
  const uint32_t d = fbits(__builtin_amdgcn_cvt_f32_fp8((int)(b & 0x7Fu), 0));
  return bitsf(d | ((b & 0x80u) << 24));
}

// ------------------------------------------------------------------ chunks
// A "chunk" is 8 consecutive elements.  16-bit inputs move one 16-byte vector
// per chunk, float32 inputs two.  Chunk c of a tensor starts at element 8c;
// every base pointer is 16-byte aligned (checked by the host layer).

template <int DT> struct Raw8;
template <> struct Raw8<DT_BF16> { u32x4 v; };
template <> struct Raw8<DT_F16> { u32x4 v; };
template <> struct Raw8<DT_F32> { u32x4 a, b; };

template <int DT>
__device__ __forceinline__ Raw8<DT> ld8(const void* base, int64_t chunk);

template <>
__device__ __forceinline__ Raw8<DT_BF16> ld8<DT_BF16>(const void* base, int64_t c) {
  return Raw8<DT_BF16>{stream_ld(reinterpret_cast<const u32x4*>(base) + c)};
}
template <>
__device__ __forceinline__ Raw8<DT_F16> ld8<DT_F16>(const void* base, int64_t c) {
  return Raw8<DT_F16>{stream_ld(reinterpret_cast<const u32x4*>(base) + c)};
}
template <>
__device__ __forceinline__ Raw8<DT_F32> ld8<DT_F32>(const void* base, int64_t c) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base) + 2 * c;
  return Raw8<DT_F32>{stream_ld(p), stream_ld(p + 1)};
}

template <int DT>
__device__ __forceinline__ Raw8<DT> zero8() {
  Raw8<DT> r;
  memset(&r, 0, sizeof(r));
  return r;
}

__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = bitsf(w << 16);
  hi = bitsf(w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack_f16x2(uint32_t w, float& lo, float& hi) {
  lo = f16_to_f32(w & 0xFFFFu);
  hi = f16_to_f32(w >> 16);
}

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float f[8]);

template <>
__device__ __forceinline__ void unpack8<DT_BF16>(const Raw8<DT_BF16>& r, float f[8]) {
  unpack_bf16x2(r.v.x, f[0], f[1]);
  unpack_bf16x2(r.v.y, f[2], f[3]);
  unpack_bf16x2(r.v.z, f[4], f[5]);
  unpack_bf16x2(r.v.w, f[6], f[7]);
}
template <>
__device__ __forceinline__ void unpack8<DT_F16>(const Raw8<DT_F16>& r, float f[8]) {
  unpack_f16x2(r.v.x, f[0], f[1]);
  unpack_f16x2(r.v.y, f[2], f[3]);
  unpack_f16x2(r.v.z, f[4], f[5]);
  unpack_f16x2(r.v.w, f[6], f[7]);
}
template <>
__device__ __forceinline__ void unpack8<DT_F32>(const Raw8<DT_F32>& r, float f[8]) {
  f[0] = bitsf(r.a.x); f[1] = bitsf(r.a.y); f[2] = bitsf(r.a.z); f[3] = bitsf(r.a.w);
  f[4] = bitsf(r.b.x); f[5] = bitsf(r.b.y); f[6] = bitsf(r.b.z); f[7] = bitsf(r.b.w);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi);

// Round 8 float32 values to DT (round to nearest even) and store them.
template <int DT>
__device__ __forceinline__ void st8(void* base, int64_t c, const float f[8]);

template <>
__device__ __forceinline__ void st8<DT_F32>(void* base, int64_t c, const float f[8]) {
  u32x4* p = reinterpret_cast<u32x4*>(base) + 2 * c;
  stream_st(u32x4{fbits(f[0]), fbits(f[1]), fbits(f[2]), fbits(f[3])}, p);
  stream_st(u32x4{fbits(f[4]), fbits(f[5]), fbits(f[6]), fbits(f[7])}, p + 1);
}
template <>
__device__ __forceinline__ void st8<DT_BF16>(void* base, int64_t c, const float f[8]) {
  stream_st(u32x4{bf16x2_rne(f[0], f[1]), bf16x2_rne(f[2], f[3]),
                                    bf16x2_rne(f[4], f[5]), bf16x2_rne(f[6], f[7])},
                              reinterpret_cast<u32x4*>(base) + c);
}
__device__ __forceinline__ uint32_t f16x2_rne(float lo, float hi);

template <>
__device__ __forceinline__ void st8<DT_F16>(void* base, int64_t c, const float f[8]) {
  stream_st(u32x4{f16x2_rne(f[0], f[1]), f16x2_rne(f[2], f[3]),
                  f16x2_rne(f[4], f[5]), f16x2_rne(f[6], f[7])},
            reinterpret_cast<u32x4*>(base) + c);
}

// Load chunk cw + l into lane l of a wave (cw uniform over the wave; zeros at
// or past `end`).  Every lane of the wave must call this together.  For
// float32 the two load instructions read one contiguous 1 KiB each (chunks
// cw .. cw + 31, then cw + 32 .. cw + 63; lane l: half l % 2 of chunk l / 2)
// and the lanes trade halves through ds_bpermute, instead of each
// instruction reading every other 16 bytes of the wave's 2 KiB.  16-bit
// inputs load per lane, as ld8 does.
template <int DT>
__device__ __forceinline__ Raw8<DT> ld8_wave(const void* base, int64_t cw, int64_t end, int lane) {
  if constexpr (DT != DT_F32) {
    return (cw + lane < end) ? ld8<DT>(base, cw + lane) : zero8<DT>();
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(base) + 2 * cw;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 a = (cw + (lane >> 1) < end) ? stream_ld(p + lane) : z;
    const u32x4 b = (cw + 32 + (lane >> 1) < end) ? stream_ld(p + 64 + lane) : z;
    // chunk cw + lane: its halves sit at positions 2 lane and 2 lane + 1 of
    // (a of lanes 0..63, then b of lanes 0..63)
    const int s0 = ((2 * lane) & 63) << 2, s1 = ((2 * lane + 1) & 63) << 2;
    const bool from_a = lane < 32;
    auto pull = [&](int src, uint32_t av, uint32_t bv) -> uint32_t {
      const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)av);
      const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)bv);
      return from_a ? x : y;
    };
    Raw8<DT_F32> r;
    r.a = u32x4{pull(s0, a.x, b.x), pull(s0, a.y, b.y), pull(s0, a.z, b.z), pull(s0, a.w, b.w)};
    r.b = u32x4{pull(s1, a.x, b.x), pull(s1, a.y, b.y), pull(s1, a.z, b.z), pull(s1, a.w, b.w)};
    return r;
  }
}

// Store the 8 results of every lane of a wave whose lane l holds chunk
// cw + l (cw uniform over the wave); chunks at or past `end` are not stored.
// Every lane of the wave must call this together.  A float32 chunk is 32
// bytes: stored by its own lane as two 16-byte halves, each store
// instruction would write every other 16 bytes of the wave's 2 KiB (measured
// at 0.35 of the HBM peak, against 0.80 for the 16-bit outputs).  Instead the
// lanes trade halves through the LDS crossbar (ds_bpermute, no LDS memory):
// the first instruction writes chunks cw .. cw + 31 and the second cw + 32 ..
// cw + 63, each one contiguous 1 KiB (lane l: half l % 2 of chunk l / 2).
template <int DT>
__device__ __forceinline__ void st8_wave(void* base, int64_t cw, int64_t end, int lane,
                                         const float f[8]) {
  if constexpr (DT != DT_F32) {
    if (cw + lane < end) st8<DT>(base, cw + lane, f);
  } else {
    const int half = lane & 1;
    const int src_a = (lane >> 1) << 2, src_b = (32 + (lane >> 1)) << 2;   // byte lane addresses
    uint32_t a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t alo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_a, (int)fbits(f[k]));
      const uint32_t ahi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_a, (int)fbits(f[4 + k]));
      const uint32_t blo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_b, (int)fbits(f[k]));
      const uint32_t bhi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_b, (int)fbits(f[4 + k]));
      a[k] = half ? ahi : alo;
      b[k] = half ? bhi : blo;
    }
    u32x4* p = reinterpret_cast<u32x4*>(base);
    const int64_t ca = cw + (lane >> 1), cb = cw + 32 + (lane >> 1);
    if (ca < end) stream_st(u32x4{a[0], a[1], a[2], a[3]}, p + 2 * ca + half);
    if (cb < end) stream_st(u32x4{b[0], b[1], b[2], b[3]}, p + 2 * cb + half);
  }
}

// ------------------------------------------------------------------ gfx950 converts
// The CDNA4 scaled fp4 converts.  Their scale operand is read as a power of
// two taken from the float's exponent field (an e8m0 byte b is passed as the
// float with bit pattern b << 23; byte 0 means 2^-127).  Quantizing converts
// divide by that power of two, dequantizing converts multiply by it.
// Measured properties this file relies on (exhaustively over every bfloat16
// value under every e8m0 scale, and over float32 values adjacent to every
// e2m1 midpoint):
//  * the stochastic-rounding quantizer adds a fixed "random" operand below
//    the kept mantissa bit and truncates; with the operands below it rounds
//    half down, i.e. to the nearest e2m1 value with ties to the smaller
//    magnitude, for operands with at most 22 significant bits (see ceil22).
//    The two elements of a pair read different bits of the operand, so each
//    pair is converted twice and the correct nibble of each kept;
//  * the sign nibble bit is the operand's sign bit (also for zeros);
//  * the dequantizers are exact, including subnormal results, except that
//    code 8 decodes to -0.0 (callers clear those sign bits first).

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kSrHalfDownEven = 0x7FFFFC00u;   // element 0 of a pair
constexpr uint32_t kSrHalfDownOdd = 0x3FFFFF00u;    // element 1 of a pair

__device__ __forceinline__ float e8m0_as_scale(uint32_t b) { return bitsf(b << 23); }

// One pair through the stochastic-rounding quantizer, result in byte 0.
// (This builtin's "old" operand is not tied to its result by the compiler, so
// its byte-select forms cannot be chained; every pair is converted into byte
// 0 of a fresh value and the bytes are assembled with v_perm_b32.  The
// round-to-nearest-even form below is tied and is chained.)
__device__ __forceinline__ uint32_t sr_fp4_pair(float a, float b, uint32_t seed, float scale) {
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2{a, b}, seed, scale, 0);
}

// Byte 0 of each of p0..p3 -> bytes 0..3 of the result.
__device__ __forceinline__ uint32_t gather_byte0(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
  const uint32_t lo = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);   // [p0.b0, p1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);   // [0, 0, p2.b0, p3.b0]
  return lo | hi;
}

// 8 values (at most 22 significant bits each) -> 8 e2m1 codes, element i in
// nibble i, each value first divided by the power of two `scale`.
__device__ __forceinline__ uint32_t e2m1_pack8_hw(const float f[8], float scale) {
  const uint32_t e = gather_byte0(sr_fp4_pair(f[0], f[1], kSrHalfDownEven, scale),
                                  sr_fp4_pair(f[2], f[3], kSrHalfDownEven, scale),
                                  sr_fp4_pair(f[4], f[5], kSrHalfDownEven, scale),
                                  sr_fp4_pair(f[6], f[7], kSrHalfDownEven, scale));
  const uint32_t o = gather_byte0(sr_fp4_pair(f[0], f[1], kSrHalfDownOdd, scale),
                                  sr_fp4_pair(f[2], f[3], kSrHalfDownOdd, scale),
                                  sr_fp4_pair(f[4], f[5], kSrHalfDownOdd, scale),
                                  sr_fp4_pair(f[6], f[7], kSrHalfDownOdd, scale));
  return o ^ ((e ^ o) & 0x0F0F0F0Fu);          // low nibbles from e, high from o
}

// Round to nearest with ties to the smaller magnitude through the round-to-
// nearest-even converter (one instruction per pair instead of two
// stochastic-rounding ones, at a higher issue rate).  Each value is first
// multiplied by kTieDown = 1 - 2^-24, which maps every normal float32 to its
// neighbour one ulp closer to zero and keeps zeros: a value / scale exactly
// on an e2m1 midpoint then lies just below it and rounds down, and one at
// least 2 ulps above a midpoint (or anywhere below it) keeps its side.
// Callers guarantee that spacing (values with at most 22 significant bits,
// e.g. after ceil22, or widened bfloat16 / float16) and that values on a
// midpoint are normal float32 numbers (for a power-of-two scale, scale >=
// 2^-124).  The converter itself rounds every float32 exactly to nearest
// even (checked on all |value / scale| < 8 for several scales).
constexpr float kTieDown = 0x1.fffffep-1f;

// Pair k of the 8 values goes to byte k of one register: the converter's
// byte select writes that byte and keeps the others.  The four calls write
// all four bytes, so the register they start from is irrelevant: it is f[0]'s
// own (dead after its product is taken), which saves zeroing one.
__device__ __forceinline__ uint32_t e2m1_pack8_rne(const float f[8], float scale) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(fbits(f[0]), f[0] * kTieDown, f[1] * kTieDown, scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2] * kTieDown, f[3] * kTieDown, scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4] * kTieDown, f[5] * kTieDown, scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6] * kTieDown, f[7] * kTieDown, scale, 3);
}

// The converter's own rounding, to nearest with ties to even, chained the same
// way.  With operands passed through half_down_for_rne it rounds half down on
// every float32, whatever its number of significant bits.
__device__ __forceinline__ uint32_t e2m1_pack8_even(const float f[8], float scale) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(fbits(f[0]), f[0], f[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], scale, 3);
}

// Clear the sign bit of every zero-magnitude nibble (code 8 -> 0), so that it
// decodes to +0.0 as the e2m1 table prescribes.
__device__ __forceinline__ uint32_t e2m1_canonical_zeros(uint32_t w) {
  const uint32_t nz = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
  return w & (nz | 0x77777777u);
}

// 8 codes -> 8 float32 values e2m1 * scale (exact).  Code 8 gives -0 unless
// w is canonical (e2m1_canonical_zeros).
__device__ __forceinline__ void e2m1_unpack8_f32_hw(uint32_t w, float scale, float out[8]) {
  f32x2 v;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0); out[0] = v.x; out[1] = v.y;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1); out[2] = v.x; out[3] = v.y;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2); out[4] = v.x; out[5] = v.y;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3); out[6] = v.x; out[7] = v.y;
}

// 8 codes -> 8 bfloat16 values (4 packed dwords) e2m1 * scale (exact).
__device__ __forceinline__ u32x4 e2m1_unpack8_bf16_hw(uint32_t w, float scale) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

// Two float32 -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32,
// IEEE with subnormals; measured bit-exact).  Written as one vector
// conversion so that both halves go through a single instruction: two scalar
// casts compile to one conversion each plus a shift and an OR.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2v));
}

// Two float32 -> packed float16 pair, round to nearest even, IEEE overflow to
// infinity, subnormals kept (v_cvt_pk_f16_f32 in the default float mode):
// the same values as f32_to_f16_rne, a NaN staying a quiet NaN.  The empty
// asm hands the conversion finished float32 values: it keeps the compiler
// from fusing it with the product that made them into one mixed-precision
// multiply-add, which would round once instead of twice and turn -0 into +0.
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2_rne(float lo, float hi) {
  asm volatile("" : "+v"(lo), "+v"(hi));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2v));
}

// ------------------------------------------------------------------ reductions
// Max across aligned groups of G consecutive lanes (G a power of two <= 64),
// the result replicated in every lane of the group.  Values are non-negative
// floats, so the unsigned integer maximum of the bit patterns is the float
// maximum.  All lanes of a group must be active.  Lane exchange uses DPP
// inside rows of 16 (quad permutes, then the half-row and row mirrors, which
// pair up groups whose members already agree) and LDS permutes above that.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
  uint32_t v = fbits(x);
  if constexpr (G >= 2) v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  if constexpr (G >= 16) v = max(v, dpp_u32<0x140>(v));  // row_mirror
  if constexpr (G >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (G >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return bitsf(v);
}

// Same for a group size known only at run time (a power of two <= 64).
__device__ __forceinline__ float group_max_rt(float x, int G) {
  uint32_t v = fbits(x);
  for (int m = 1; m < G; m <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
  return bitsf(v);
}

} // namespace mxq
