/*
 * fos_ceiling.h -- measured HBM ceilings (libfos_ceiling.so), for reporting only.
 *
 * These entry points are not part of the Four Over Six method.  They launch kernels
 * that move exactly the bytes of a quantize kernel without computing anything, so
 * that the benchmark can place each kernel's bandwidth beside what plain streaming
 * reaches on the same GPU.  Each lane moves 32 bytes with two 16-byte non-temporal
 * accesses; one workgroup of 256 lanes per fos_ceiling_granule() bytes.
 *
 * All pointers are device pointers owned by the caller; calls are asynchronous on
 * `stream` (a hipStream_t, NULL = default stream).  Return value: 0 on success,
 * 1 a NULL pointer, 2 `bytes` not a positive multiple of fos_ceiling_granule() (or
 * 2^24 granules or more), 3 a misaligned pointer, 6 a failed launch.  Nothing is
 * launched unless the return value is 0.
 */
#ifndef FOS_CEILING_H
#define FOS_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes per workgroup (8192): every size below must be a multiple of it. */
size_t fos_ceiling_granule(void);

/* Read `bytes` from x (16-byte aligned).  The words of each chunk are folded with xor
 * and stored to sink[0] only when the result equals `key` (pass a key that the data
 * is unlikely to produce; a match only rewrites sink[0]). */
int fos_ceiling_read(const void* x, size_t bytes, uint32_t key, uint32_t* sink, void* stream);

/* Copy `bytes` from x to y (both 16-byte aligned, not overlapping): read + write. */
int fos_ceiling_copy(const void* x, void* y, size_t bytes, void* stream);

/* The row-wise quantize kernel's traffic without its arithmetic: read `bytes` from x
 * (16-byte aligned) and, per 32-byte chunk g, write 8 bytes to y8 + 8g (8-byte aligned)
 * and 1 byte to y1 + g (bytes / 4 and bytes / 32 bytes of output). */
int fos_ceiling_pattern(const void* x, size_t bytes, void* y8, void* y1, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FOS_CEILING_H */
