/*
 * mxq_roofline.h -- C ABI of libmxq_roofline: plain streaming kernels that
 * measure the practical HBM ceiling of one MI355X (gfx950), with which the
 * codec kernels of libmxq are compared, and a shader clock probe.  Not part
 * of the codec.  The streaming calls compute nothing the source pages
 * define; they move bytes with the same
 * 16-byte non-temporal vector accesses and the same wave-tile mapping as the
 * codec's streaming kernels (every wave instruction touches one contiguous
 * 1 KiB range; four waves per workgroup, one tile of `unroll` x 64 chunks per
 * wave), and no arithmetic.
 *
 * Conventions: every pointer is a caller-owned DEVICE pointer, 16-byte
 * aligned; `bytes` is a multiple of 16; `unroll` (16-byte chunks per lane and
 * tile) is 1, 2, 4 or 8.  Arguments are checked on the host before anything
 * is launched; calls are asynchronous on `stream` and allocate nothing.
 * bytes == 0 launches nothing.
 */
#ifndef MXQ_ROOFLINE_H
#define MXQ_ROOFLINE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MXQ_REF_OK = 0,
  MXQ_REF_E_NULL = 1,    /* a pointer is NULL while bytes > 0          */
  MXQ_REF_E_SHAPE = 2,   /* bytes negative or not a multiple of 16     */
  MXQ_REF_E_UNROLL = 5,  /* unroll not 1, 2, 4 or 8                    */
  MXQ_REF_E_LAUNCH = 7,  /* the HIP runtime rejected the launch        */
  MXQ_REF_E_ALIGN = 9    /* a pointer is not 16-byte aligned           */
};

/* Copy `bytes` from src to dst (no overlap): reads and writes each byte once. */
int mxq_ref_copy(const void* src, void* dst, int64_t bytes, int32_t unroll,
                 hipStream_t stream);

/* Read `bytes` from src once and fold them into an XOR that is written to
 * sink[0] only when it equals `magic` (pick a value the data cannot produce
 * in practice): a read-only stream that the compiler cannot drop. */
int mxq_ref_read(const void* src, int64_t bytes, int32_t unroll, uint32_t magic,
                 uint32_t* sink, hipStream_t stream);

/* Write the 32-bit `value` over `bytes` of dst: a write-only stream. */
int mxq_ref_fill(void* dst, int64_t bytes, uint32_t value, int32_t unroll,
                 hipStream_t stream);

/* Shader clock probe: `blocks` workgroups of one wave each read the shader
 * cycle counter and the constant 100 MHz counter around a chain of `iters`
 * dependent VALU operations and store, per workgroup, the two differences:
 * out[2 b] = shader cycles, out[2 b + 1] = 100 MHz ticks (out holds 2 * blocks
 * 8-byte-aligned values).  sum(cycles) / sum(ticks) * 100 is the mean shader
 * clock in MHz over the window.  blocks in [1, 65536], iters in [1, 2^24],
 * else MXQ_REF_E_SHAPE. */
int mxq_ref_clock(uint64_t* out, int32_t blocks, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_ROOFLINE_H */
