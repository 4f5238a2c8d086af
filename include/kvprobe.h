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

/*
 * The same read in one of a sweep of launch shapes.  lds_dma = 0: register
 * loads, n_workgroups workgroups of `threads` threads each reading a
 * contiguous share with `loads` 16-byte loads in flight per thread --
 * (threads, loads) one of (256, 1 / 4 / 8 / 16 / 32), (512, 4 / 8 / 16 / 32),
 * (1024, 4 / 8 / 16).  lds_dma = 1: every thread issues its whole share,
 * `loads` 16-byte global_load_lds into LDS, at workgroup entry, waits once
 * and folds its LDS words -- (threads, loads) one of (256, 8 / 16 / 32),
 * (512, 8 / 16), (1024, 4 / 8); the grid is kvprobe_lds_workgroups(bytes,
 * threads, loads) and n_workgroups is ignored.  sink: device uint32 [grid *
 * threads].  Other arguments and return values as kvprobe_read.
 */
int kvprobe_read_shape(const void* p, int64_t bytes, int32_t n_workgroups, int32_t threads, int32_t loads,
                       int32_t lds_dma, void* sink, void* stream);

/* Workgroups of an LDS-DMA read of `bytes` bytes (each takes threads * loads
 * 16-byte words), or -1 for a non-positive argument. */
int64_t kvprobe_lds_workgroups(int64_t bytes, int32_t threads, int32_t loads);

#ifdef __cplusplus
}
#endif

#endif
