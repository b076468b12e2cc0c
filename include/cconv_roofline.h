/*
 * cconv_roofline.h -- flat-copy kernels of libcconv_roofline.so, the measured bandwidth
 * roofline the convolution kernels are compared against. The kernel-fun wheel's strip.py
 * module docstring judges its strip kernels against a flat copy on the same GPU; the forward
 * moves 1 read : 1 write of bf16 rows and the backward 2 reads : 1 write, so both mixes
 * exist here.
 *
 * cconv_roofline_copy(kind, a, b, dst, bytes, unroll, threads, nontemporal, stream)
 *   kind 1: dst = a (1 read, 1 write); kind 2: dst = a ^ b bitwise (2 reads, 1 write).
 *   a, b, dst: 16-byte aligned device buffers of `bytes` bytes (b unused for kind 1; dst
 *   must not overlap a or b). bytes must be a multiple of 16.
 *   unroll: 16-byte vectors per thread (1, 2, 4 or 8); threads per block: 256, 512 or 1024;
 *   nontemporal: 1 to use non-temporal loads and stores.
 * Returns 0 on success, 1 on a bad argument (nothing enqueued), 2 on a failed launch.
 *
 * cconv_roofline_copy_persistent(kind, a, b, dst, bytes, blocks, unroll, threads, nontemporal,
 *                                stream)
 *   The same copies with a fixed grid of `blocks` blocks (1 .. 65536) walking the buffer in
 *   grid-stride chunks; each thread keeps `unroll` (2, 4 or 8) 16-byte loads in flight before
 *   its stores. Same arguments and returns otherwise.
 */
#ifndef CCONV_ROOFLINE_H
#define CCONV_ROOFLINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;

int cconv_roofline_copy(int kind, const void* a, const void* b, void* dst, int64_t bytes, int unroll,
                        int threads, int nontemporal, struct ihipStream_t* stream);

int cconv_roofline_copy_persistent(int kind, const void* a, const void* b, void* dst, int64_t bytes, int blocks,
                                   int unroll, int threads, int nontemporal, struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif

#endif /* CCONV_ROOFLINE_H */
