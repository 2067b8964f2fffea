/*
 * mxq_oracle.h -- plain, slow CPU oracle for block-scaled microscaling
 * quantization (MXFP4, NVFP4, MXFP8, static two-level FP4, block-scaled
 * cache QDQ, paged NVFP4 KV cache) and the grouped GEMM over its weights.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and mxq_oracle.c are used by the
 * test-suite, by the smoke check and by the CPU-baseline leg of the bench.
 * The product library never includes, links or calls anything here, and this
 * oracle shares no code, table or helper with the GPU path.
 *
 * All data pointers are host pointers to contiguous row-major arrays.
 * Element dtypes: 0 = float32, 1 = bfloat16 (raw 16-bit patterns),
 * 2 = float16 (raw 16-bit patterns).
 */
#ifndef MXQ_ORACLE_H
#define MXQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- primitives (exported so the tests can pin them one by one) ---- */
double   orc_e2m1_decode(uint32_t code);            /* D(c)                        */
uint32_t orc_e2m1_round_mag(float q);               /* R(q): 0..7                  */
double   orc_round_binary(double v, int p, int emin); /* RN to p-bit significand */
double   orc_e4m3_decode(uint32_t byte);
uint32_t orc_e4m3_encode(float v);                  /* sign kept, saturates at 448 */
double   orc_e8m0_decode(uint32_t byte);
float    orc_pow2_ceil(float v);
int      orc_floor_log2(float a);                   /* a > 0                       */
float    orc_load(const void* x, int dtype, int64_t i);
void     orc_store(void* y, int dtype, int64_t i, float v);

/* ---- the five operations ---- */
void orc_quantize_mxfp4(const void* x, int dtype, int64_t rows, int64_t K,
                        uint8_t* packed, uint8_t* scales);
void orc_dequantize_mxfp4(const uint8_t* packed, const uint8_t* scales,
                          int64_t rows, int64_t K, void* y, int dtype);
/* mode 0: per-row amax, 1: given (given[r * given_stride]), 2: whole-tensor amax */
void orc_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t K,
                        int mode, const float* given, int64_t given_stride,
                        uint8_t* packed, uint8_t* scales, float* row_scale);
void orc_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales,
                          const float* row_scale, int64_t rows, int64_t K,
                          void* y, int dtype);
/* fmt 0: fp8 (e4m3 values, power-of-two scale), 1: mxfp4, 2: nvfp4 */
void orc_quantize_cache(const void* x, void* y, int dtype, int64_t rows,
                        int64_t C, int fmt, int64_t block_size);

/* MXFP8: e4m3 codes [rows, K] and e8m0 scale bytes [rows, K / 32]. */
void orc_quantize_mxfp8(const void* x, int dtype, int64_t rows, int64_t K,
                        uint8_t* codes, uint8_t* scales);
void orc_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales,
                          int64_t rows, int64_t K, void* y, int dtype);

/* Static two-level FP4 fake quantization: block_amax [rows, K / block],
 * global amax G; y has x's shape and dtype.  orc_static_block_scale gives
 * the dequantization-side block scale of one block. */
float orc_static_block_scale(float a, float G);
void orc_fake_quantize_fp4_static(const void* x, int dtype, int64_t rows,
                                  int64_t K, int64_t block,
                                  const float* block_amax, float G, void* y);

/* Paged NVFP4 KV cache -> contiguous [nblocks * block_tokens, H, D]; the
 * three arrays hold one host pointer / value per block. */
void orc_dequantize_kv_pages(const uint8_t* const* values,
                             const uint8_t* const* scales, const float* amax,
                             int64_t nblocks, int64_t block_tokens, int64_t H,
                             int64_t D, void* y, int dtype);
/* k_smooth of one row of D values (dtype values held as float32), in place. */
void orc_k_smooth_row(float* row, int64_t D, int dtype);
/* Per-head NVFP4 of k [S, H, D] (smooth != 0: k_smooth first). */
void orc_quantize_kv_nvfp4(const void* k, int dtype, int64_t S, int64_t H,
                           int64_t D, int smooth, uint8_t* packed,
                           uint8_t* scales, float* row_scale);

/* Grouped GEMM over dequantized expert weights, selected output rows only.
 * x [T, D_in] (dtype xdt), w [E, N, K] (dtype wdt: the dequantized weights in
 * the activation dtype); rows of x are grouped by expert through the
 * cumulative counts offs[E].  trans 0: D_in = K, out[i, n] = sum_k x[r, k] *
 * w[e, n, k]; trans 1: D_in = N, out[i, k] = sum_n x[r, n] * w[e, n, k], for
 * r = rows[i] and e its expert (a row in no group gives zeros).  Products and
 * sums in binary64; absout receives sum |x * w| for each output. */
void orc_grouped_mm(const void* x, int xdt, int64_t T, const void* w, int wdt,
                    int64_t E, int64_t N, int64_t K, const int32_t* offs,
                    int trans, const int64_t* rows, int64_t nrows,
                    double* out, double* absout);

/* Thread count of the OpenMP row loops (results do not depend on it). */
void orc_set_threads(int n);
int orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
