// Streaming-read probe (include/kvprobe.h): the read ceiling that the
// attention kernels' bandwidth is compared with.  Each workgroup reads one
// contiguous share of the buffer with 16-byte loads, U of them in flight per
// thread, and leaves an XOR per thread in the sink.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvprobe.h"

namespace {

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, int64_t n16, int64_t per_wg,
                                                   uint32_t* __restrict__ sink) {
    const int64_t b = (int64_t)blockIdx.x * per_wg;
    const int64_t e = (b + per_wg < n16) ? b + per_wg : n16;
    uint32_t acc = 0;
    for (int64_t i = b + threadIdx.x; i < e; i += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * 256;
            v[u] = j < e ? p[j] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int kvprobe_read(const void* p, int64_t bytes, int32_t n_workgroups, int32_t unroll, uint32_t* sink,
                            void* stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 || ((uintptr_t)p % 16) || n_workgroups <= 0) return -1;
    const int64_t n16 = bytes / 16;
    const int64_t per = (n16 + n_workgroups - 1) / n_workgroups;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* q = static_cast<const uint4*>(p);
    switch (unroll) {
        case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(n_workgroups), dim3(256), 0, s, q, n16, per, sink); break;
        case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(n_workgroups), dim3(256), 0, s, q, n16, per, sink); break;
        case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(n_workgroups), dim3(256), 0, s, q, n16, per, sink); break;
        case 16: hipLaunchKernelGGL(read_kernel<16>, dim3(n_workgroups), dim3(256), 0, s, q, n16, per, sink); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}
