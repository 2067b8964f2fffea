/*
 * mxq.h -- C ABI of libmxq: block-scaled microscaling quantization on AMD
 * Instinct MI355X (gfx950).
 *
 * Three operations along the last dimension of a contiguous row-major
 * [rows, K] tensor:
 *   - quantize-pack into e2m1 (fp4) nibbles plus per-block scales
 *     (MXFP4: one e8m0 scale per 32 columns; NVFP4: one e4m3 scale per 16
 *     columns plus one float32 scale per row),
 *   - dequantize back to a floating dtype,
 *   - the quantize/dequantize round trip used for cache values (fp8 e4m3,
 *     mxfp4 or nvfp4 groups of any block size).
 *
 * Further calls: MXFP8 quantize / dequantize, static two-level FP4 fake
 * quantization with caller-given amax values, the NVFP4 KV cache (paged
 * dequantization, per-head quantization with k_smooth), and the grouped
 * GEMM over packed fp4 expert weights.
 *
 * Sources, cited by page title and section:
 *   [mxfp4 page] "nemo_automodel.components.quantization.mxfp4"
 *   [nvfp4 page] "nemo_automodel.components.quantization.nvfp4"
 *   [cache page] "nemo_automodel.components.models.deepseek_v41.quantization"
 *   [modelopt]   Model-Optimizer "tensor_quantizer.py" (TensorQuantizer,
 *                StaticBlockScaleQuantizer)
 *   [longlive]   LongLive "utils/quant.py" (dequantize_kv_cache, k_smooth,
 *                quantize_kv)
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer to contiguous row-major memory
 *     owned by the caller; the library allocates nothing and keeps no state.
 *     "rows" is the product of all leading dimensions.
 *   - Alignment: float/bfloat16/float16 tensors and packed arrays must be
 *     16-byte aligned for the weight calls (MXQ_E_ALIGN otherwise); the cache
 *     call accepts any alignment (it takes a slower path when x or y is not
 *     16-byte aligned or C is not a multiple of 8).
 *   - Calls are asynchronous on `stream` (0 = the null stream): argument
 *     validation happens synchronously on the host and returns an error
 *     status before anything is launched; a successful call returns MXQ_OK
 *     once its kernels are enqueued and never synchronizes.  A launch failure
 *     reported by the runtime returns MXQ_E_LAUNCH.
 *   - rows == 0 or K == 0 is valid and launches nothing.
 *   - Inputs are never written.  Outputs must not overlap inputs.
 *   - Input elements must be finite.  The pages define nothing for NaN or
 *     infinite elements; for them the codes and scales are unspecified (every
 *     access stays in bounds and the call still returns MXQ_OK).  Degenerate
 *     but finite cases are specified: all-zero blocks and rows, zero, tiny,
 *     huge or infinite given NVFP4 row scales.
 *   - Thread-safe: no global state.
 *   - Packed nibble order: the even column in the low nibble, the following
 *     odd column in the high nibble ([mxfp4 page] and [nvfp4 page],
 *     introductions).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 2

/* Floating element types of inputs and dequantized outputs ([mxfp4 page]
 * and [nvfp4 page] take any floating-point tensor). */
typedef enum mxq_dtype {
  MXQ_F32 = 0,
  MXQ_BF16 = 1,
  MXQ_F16 = 2
} mxq_dtype;

/* Cache value formats ([cache page], quantize_cache: fp8 for SWA KV, mxfp4
 * with an E8M0 scale for index Q/K, nvfp4 with an E4M3 scale for compressed
 * KV). */
typedef enum mxq_format {
  MXQ_FMT_FP8 = 0,
  MXQ_FMT_MXFP4 = 1,
  MXQ_FMT_NVFP4 = 2
} mxq_format;

/* How mxq_quantize_nvfp4 obtains the float32 scale g of each row. */
typedef enum mxq_nv_mode {
  /* g = amax(row) / (6 * 448) for every row ([nvfp4 page] quantize_nvfp4,
   * default rule: one global scale per row). */
  MXQ_NV_ROW_AMAX = 0,
  /* g = given[r * given_stride]: caller-supplied scales ([nvfp4 page]
   * quantize_nvfp4 with global_scale); given_stride 1 = one per row, 0 = one
   * for the whole tensor. */
  MXQ_NV_GIVEN = 1,
  /* g = amax(whole tensor) / (6 * 448), written to every row_scale entry
   * ([nvfp4 page] quantize_nvfp4_modelopt: one tensor scale). Needs
   * `scratch`: 4 bytes of device memory that receive the tensor amax. */
  MXQ_NV_TENSOR_AMAX = 2
} mxq_nv_mode;

typedef enum mxq_status {
  MXQ_OK = 0,
  MXQ_E_NULL = 1,    /* a required pointer is NULL                           */
  MXQ_E_SHAPE = 2,   /* negative size, or K not a whole number of blocks     */
  MXQ_E_DTYPE = 3,   /* unknown mxq_dtype                                    */
  MXQ_E_FORMAT = 4,  /* unknown mxq_format                                   */
  MXQ_E_BLOCK = 5,   /* block_size outside what the call accepts             */
  MXQ_E_SIZE = 6,    /* rows * K overflows int64                             */
  MXQ_E_LAUNCH = 7,  /* the HIP runtime rejected a kernel launch             */
  MXQ_E_MODE = 8,    /* unknown mxq_nv_mode                                  */
  MXQ_E_ALIGN = 9,   /* a pointer is not 16-byte aligned where required      */
  MXQ_E_SCRATCH = 10 /* the call needs more than its static device scratch   */
} mxq_status;

/*
 * MXFP4 quantize ([mxfp4 page] quantize_mxfp4).
 *   x       [rows, K] of xdt; K % 32 == 0, else MXQ_E_SHAPE.
 *   packed  [rows, K/2] int8: two e2m1 codes per byte.
 *   scales  [rows, K/32] float8_e8m0fnu bytes: for each 32-column block the
 *           scale 2^(floor(log2(amax)) - 2), floor exact, clamped below at
 *           2^-127 (byte 0; also for an all-zero block).  Elements are divided
 *           by the stored scale and rounded to the nearest e2m1 value (ties to
 *           the smaller magnitude); the sign nibble bit is the input's sign.
 */
mxq_status mxq_quantize_mxfp4(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, int8_t* packed, uint8_t* scales,
                              hipStream_t stream);

/*
 * MXFP4 dequantize ([mxfp4 page] dequantize_mxfp4).
 *   packed [rows, K/2] int8, scales [rows, K/32] e8m0 bytes (K % 32 == 0).
 *   y      [rows, K] of ydt: e2m1(code) * 2^(scale - 127), computed exactly in
 *          float32 and rounded once to ydt (code 8 decodes to +0.0; scale byte
 *          0xFF gives NaN).
 */
mxq_status mxq_dequantize_mxfp4(const int8_t* packed, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y,
                                mxq_dtype ydt, hipStream_t stream);

/*
 * NVFP4 quantize ([nvfp4 page] quantize_nvfp4, quantize_nvfp4_modelopt;
 * K % 16 == 0 else MXQ_E_SHAPE, the rule of _check_last_dim).
 *   Per row: g as selected by `mode` (float32).  Per 16-column block with
 *   amax a: block scale = e4m3(clamp((a / 6) / g, 2^-9, 448)); each element is
 *   divided by (block scale * g) and rounded to the nearest e2m1 value (ties to
 *   the smaller magnitude).  All arithmetic is float32, correctly rounded,
 *   evaluated in that order.
 *   given, given_stride   used by MXQ_NV_GIVEN only (device pointer).
 *   scratch               MXQ_NV_TENSOR_AMAX only: 4 bytes of device memory,
 *                         overwritten with the tensor amax.
 *   packed     [rows, K/2] uint8 (same bits as int8).
 *   scales     [rows, K/16] float8_e4m3fn bytes.
 *   row_scale  [rows] float32: the g used for each row.
 *   The ModelOpt NVFP4 layout: 0.5625 bytes per parameter plus 4 bytes per
 *   row ([nvfp4 page] introduction).
 */
mxq_status mxq_quantize_nvfp4(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, mxq_nv_mode mode, const float* given,
                              int64_t given_stride, float* scratch,
                              uint8_t* packed, uint8_t* scales,
                              float* row_scale, hipStream_t stream);

/*
 * NVFP4 dequantize ([nvfp4 page] dequantize_nvfp4).
 *   packed [rows, K/2] uint8 or int8 bits, scales [rows, K/16] e4m3 bytes,
 *   row_scale [rows] float32.
 *   y [rows, K] of ydt: (e2m1(code) * e4m3(scale)) * row_scale in float32,
 *   left to right, then one rounding to ydt.
 */
mxq_status mxq_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t rows,
                                int64_t K, void* y, mxq_dtype ydt,
                                hipStream_t stream);

/*
 * Cache quantize/dequantize round trip ([cache page] quantize_cache and
 * _CacheQuantization.forward): y gets x's shape [rows, C] and dtype.
 *   Groups are block_size consecutive channels (block_size >= 1, else
 *   MXQ_E_BLOCK); a last partial group behaves as if zero-padded.  Per group
 *   with amax a:
 *     MXQ_FMT_FP8:   s = pow2ceil(max(a / 448, 2^-126)); y = e4m3(x / s) * s
 *                    (e4m3 round to nearest even; the sign of zero is kept);
 *     MXQ_FMT_MXFP4: s = pow2ceil(max(a / 6, 2^-126)); y = e2m1(x / s) * s;
 *     MXQ_FMT_NVFP4: s = e4m3(clamp(a / 6, 2^-9, 448));  y = e2m1(x / s) * s;
 *   pow2ceil is the [cache page] _power_of_two_ceiling; e2m1 rounds to the
 *   nearest value with ties to the smaller magnitude and decodes code 8 to
 *   +0.0.  The products are exact in float32; y is rounded once to dt.
 *   x and y must not overlap.
 */
mxq_status mxq_quantize_cache(const void* x, void* y, mxq_dtype dt,
                              int64_t rows, int64_t C, mxq_format fmt,
                              int32_t block_size, hipStream_t stream);

/*
 * MXFP8 quantize ([modelopt] TensorQuantizer._real_quantize, the MX branch
 * with e4m3 elements, which requires block size 32).  The pages name the
 * MXFP8 tensor class without its arithmetic; the block scale is the fp8
 * power-of-two rule of [cache page] quantize_cache / _power_of_two_ceiling.
 *   x       [rows, K] of xdt; K % 32 == 0, else MXQ_E_SHAPE.
 *   codes   [rows, K] float8_e4m3fn bytes: e4m3(x / s), round to nearest
 *           even, sign bit of x kept (also on zeros); |x / s| <= 448 always.
 *   scales  [rows, K/32] float8_e8m0fnu bytes of s = pow2ceil(max(amax / 448,
 *           2^-126)) per 32-column block (bytes 1 .. 247 for finite input).
 *   x and codes 16-byte aligned (MXQ_E_ALIGN otherwise).
 */
mxq_status mxq_quantize_mxfp8(const void* x, mxq_dtype xdt, int64_t rows,
                              int64_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);

/*
 * MXFP8 dequantize (the inverse of mxq_quantize_mxfp8).
 *   codes [rows, K] e4m3 bytes, scales [rows, K/32] e8m0 bytes (K % 32 == 0).
 *   y     [rows, K] of ydt: e4m3(code) * 2^(scale - 127), exact in float32
 *         (or infinite when it overflows), rounded once to ydt; code bytes
 *         0x7F / 0xFF and scale byte 0xFF give NaN.
 *   codes and y 16-byte aligned.
 */
mxq_status mxq_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales,
                                int64_t rows, int64_t K, void* y,
                                mxq_dtype ydt, hipStream_t stream);

/*
 * Static two-level FP4 fake quantization ([modelopt]
 * StaticBlockScaleQuantizer._block_scale_from_amax with FP8 block scales,
 * _amax_to_scale, _clamp_scale, _FP8_E4M3_MIN_POSITIVE, and _fake_quantize
 * with one amax as both the pre and the post scale).
 *   x            [rows, K] of dt; y receives the round trip, same shape and dtype.
 *   block_size   B: a power of two in [8, 1024] (else MXQ_E_BLOCK); K % B == 0
 *                (else MXQ_E_SHAPE).
 *   block_amax   [rows, K/B] float32 device array: the calibrated amax of each
 *                block of B consecutive columns (finite, >= 0).
 *   global_amax  one float32 in device memory (finite, >= 0).
 *   float32 arithmetic, in this order:
 *     P = G / 6 (1e-8 when <= 1e-8);  m = float32(2^-9 / 448) * P;
 *     s = a / 6 (m when <= m);  t = 448 / P;  s' = e4m3(s * t) / t
 *       (e4m3 round to nearest even, saturating at 448);
 *     y = RN_dt(e2m1(x / s') * s')  (e2m1 ties to the smaller magnitude;
 *       code 8 decodes to +0.0).
 *   x and y 16-byte aligned.
 */
mxq_status mxq_fake_quantize_fp4_static(const void* x, mxq_dtype dt, int64_t rows,
                                        int64_t K, int32_t block_size,
                                        const float* block_amax,
                                        const float* global_amax, void* y,
                                        hipStream_t stream);

/*
 * Paged NVFP4 KV cache -> one contiguous tensor ([longlive] dequantize_kv_cache).
 *   The cache is a list of num_blocks blocks, each a separate device
 *   allocation reached through three DEVICE arrays of num_blocks DEVICE
 *   pointers:
 *     values[b]  uint8 [block_tokens * heads, head_dim / 2]: packed e2m1 codes,
 *                row t * heads + h holding token t, head h;
 *     scales[b]  e4m3 bytes [block_tokens * heads, head_dim / 16], row-major
 *                (the page's third-party class keeps them swizzled; that
 *                layout is not supported);
 *     amax[b]    one float32: the block's global scale is amax / (6 * 448).
 *   Each block's arrays must be 16-byte aligned.  head_dim % 16 == 0 (else
 *   MXQ_E_SHAPE).
 *   y  [num_blocks * block_tokens, heads, head_dim] of ydt (16-byte aligned):
 *      token b * block_tokens + t of y is token t of block b; values decode as
 *      mxq_dequantize_nvfp4 does ((e2m1 * e4m3) * global in float32, one
 *      rounding to ydt).
 */
mxq_status mxq_dequantize_kv_pages_nvfp4(const uint8_t* const* values,
                                         const uint8_t* const* scales,
                                         const float* const* amax, int64_t num_blocks,
                                         int64_t block_tokens, int64_t heads,
                                         int64_t head_dim, void* y, mxq_dtype ydt,
                                         hipStream_t stream);

/*
 * Per-head NVFP4 quantization of a K or V tensor ([longlive] quantize_kv,
 * k_smooth), with the NVFP4 rule of [nvfp4 page] quantize_nvfp4_modelopt
 * applied to each head's slice.
 *   k          [tokens, heads, head_dim] of dt (16-byte aligned); head_dim a
 *              power of two in [16, 512], heads <= 4096 (else MXQ_E_SHAPE).
 *   smooth     1: each row (token, head) first has its mean removed
 *              (k_smooth): mean = binary32 pairwise sum over the row times
 *              1 / head_dim, rounded to dt; value - mean evaluated in binary32
 *              and rounded to dt.  0: no smoothing (values).  Else MXQ_E_MODE.
 *   head_amax  [heads * 32] float32 device scratch (each head's maximum is
 *              gathered in 32 slots, slot-major); after the call head_amax[h]
 *              holds head h's amax (of the smoothed values).
 *   packed     uint8 [tokens, heads, head_dim / 2] (16-byte aligned),
 *   scales     e4m3 bytes [tokens, heads, head_dim / 16],
 *   row_scale  float32 [tokens, heads]: the head's g = amax / (6 * 448) on each
 *              of its rows, so that mxq_dequantize_nvfp4 with rows =
 *              tokens * heads decodes the result.
 *   Block scales and codes as mxq_quantize_nvfp4 with that g.  The page's
 *   mean-squared-error scale rule belongs to a third-party library and is not
 *   offered.  Two passes over k (the per-head amax first).
 */
mxq_status mxq_quantize_kv_nvfp4(const void* k, mxq_dtype dt, int64_t tokens, int64_t heads,
                                 int64_t head_dim, int32_t smooth, float* head_amax,
                                 uint8_t* packed, uint8_t* scales, float* row_scale,
                                 hipStream_t stream);

/*
 * mxq_quantize_kv_nvfp4 without the head_amax workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, validation,
 * kernels and results as mxq_quantize_kv_nvfp4, minus head_amax: the per-head
 * maxima are gathered in a static device array that the library holds on
 * each GPU it runs on until the process ends (heads * 32 float32 words,
 * 128 KiB at the limit).
 *   heads > MXQ_NOALLOC_KV_MAX_HEADS returns MXQ_E_SCRATCH (before any launch).
 *   The call allocates nothing; the first call on a device looks up the
 *   array's device address (hipGetSymbolAddress) and keeps it.
 *   Every call on one GPU uses the same array: calls that overlap in time on
 *   one GPU (different streams) race and give unspecified results; calls in
 *   stream order are independent (each clears the words it uses).
 */
#define MXQ_NOALLOC_KV_MAX_HEADS 1024
mxq_status mxq_quantize_kv_nvfp4_noalloc(const void* k, mxq_dtype dt, int64_t tokens,
                                         int64_t heads, int64_t head_dim, int32_t smooth,
                                         uint8_t* packed, uint8_t* scales, float* row_scale,
                                         hipStream_t stream);

/*
 * Grouped GEMM over packed fp4 expert weights, dequantized on the fly
 * ([mxfp4 page] MXFP4GroupedMM, [nvfp4 page] NVFP4GroupedMM, forward and
 * backward).
 *   x       [tokens, D_in] bfloat16 activations (MXQ_BF16 only, else
 *           MXQ_E_DTYPE), rows grouped contiguously by expert.
 *   offs    [experts] int32 device array of cumulative token counts: expert e
 *           owns rows [offs[e-1], offs[e]) (offs[-1] = 0).  It must be
 *           non-decreasing with offs[experts-1] <= tokens; each group is
 *           clamped to [0, tokens], so malformed offs cannot make an access
 *           out of bounds (the results are then unspecified).
 *   weights W [experts, N, K] packed along K as the quantize calls write them:
 *           MXFP4: packed int8 [E, N, K/2] + e8m0 scales [E, N, K/32];
 *           NVFP4: packed uint8 [E, N, K/2] + e4m3 scales [E, N, K/16] + float32
 *           row_scale [E, N].  Each weight is dequantized to bfloat16 exactly
 *           as mxq_dequantize_mxfp4 / mxq_dequantize_nvfp4 with MXQ_BF16 do.
 *   transpose 0 (forward):  D_in = K, y [tokens, N], y[t] = x[t] @ W_e^T;
 *             1 (backward): D_in = N, y [tokens, K], y[t] = x[t] @ W_e
 *           (else MXQ_E_MODE).
 *   y       bfloat16; float32 accumulation, one rounding per output.  Rows
 *           outside every expert's group are not written.
 *   N and K must be positive multiples of 128 (MXQ_E_SHAPE otherwise); x,
 *   packed and y 16-byte aligned.  tokens == 0 or experts == 0 launches
 *   nothing.
 */
mxq_status mxq_grouped_mm_mxfp4(const void* x, mxq_dtype xdt, int64_t tokens,
                                const int8_t* packed, const uint8_t* scales,
                                int64_t experts, int64_t N, int64_t K,
                                const int32_t* offs, int32_t transpose, void* y,
                                hipStream_t stream);
mxq_status mxq_grouped_mm_nvfp4(const void* x, mxq_dtype xdt, int64_t tokens,
                                const uint8_t* packed, const uint8_t* scales,
                                const float* row_scale, int64_t experts, int64_t N,
                                int64_t K, const int32_t* offs, int32_t transpose,
                                void* y, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* mxq_status_string(mxq_status s);

/* MXQ_ABI_VERSION of the loaded library. */
int32_t mxq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
