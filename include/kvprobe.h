/*
 * kvprobe: a streaming-read probe for measuring the HBM read ceiling of the
 * device the decode-attention kernels run on.  It reads a buffer once with
 * 16-byte loads, as the attention kernels read a KV cache, and is used only
 * to put their achieved bandwidth next to what a plain read reaches for the
 * same number of bytes per launch.  Not part of the attention path.
 */
#ifndef KVPROBE_H
#define KVPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at device address `p` once: `n_workgroups` workgroups of
 * 256 threads, each reading a contiguous share with `unroll` (1, 4, 8 or 16)
 * 16-byte loads in flight per thread, and write one XOR of what each thread
 * read to `sink` (device, n_workgroups * 256 uint32) so that the loads cannot
 * be dropped.  p must be 16-byte aligned and bytes a multiple of 16.  The
 * launch is asynchronous on `stream` (a hipStream_t, NULL = default stream).
 * Returns 0, -1 for an invalid argument, or a positive hipError_t of the
 * launch.
 */
int kvprobe_read(const void* p, int64_t bytes, int32_t n_workgroups, int32_t unroll, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
