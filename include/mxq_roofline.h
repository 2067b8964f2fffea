/*
 * mxq_roofline.h -- C ABI of libmxq_roofline: plain streaming kernels that
 * measure the practical HBM ceiling of one MI355X (gfx950), against which the
 * codec kernels of libmxq are judged.  Not part of the codec: these calls
 * compute nothing the source pages define; they move bytes with the same
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

#ifdef __cplusplus
}
#endif
#endif /* MXQ_ROOFLINE_H */
