// Streaming-read probe (include/kvprobe.h): the read ceiling that the
// attention kernels' bandwidth is compared with, over a sweep of launch
// shapes.  Register loads: each workgroup reads one contiguous share of the
// buffer with 16-byte loads, U of them in flight per thread, and leaves an
// XOR per thread in the sink.  LDS DMA: each thread issues its whole share
// (N 16-byte global_load_lds) at entry, waits once, and XORs its LDS words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvprobe.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int U, int T>
__global__ __launch_bounds__(T) void read_kernel(const uint4* __restrict__ p, int64_t n16, int64_t per_wg,
                                                 uint32_t* __restrict__ sink) {
    const int64_t b = (int64_t)blockIdx.x * per_wg;
    const int64_t e = (b + per_wg < n16) ? b + per_wg : n16;
    uint32_t acc = 0;
    for (int64_t i = b + threadIdx.x; i < e; i += (int64_t)T * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * T;
            v[u] = j < e ? p[j] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(int64_t)blockIdx.x * T + threadIdx.x] = acc;
}

// Share of a workgroup: N * T 16-byte words; past the end a thread reads the
// last word again (in bounds), so every wait covers loads that were issued.
template <int N, int T>
__global__ __launch_bounds__(T) void read_lds_kernel(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * N * T;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int64_t j = b + (int64_t)u * T + threadIdx.x;
        const int64_t jj = j < n16 ? j : n16 - 1;
        // one wave's 64 words land in consecutive LDS words at this base
        __builtin_amdgcn_global_load_lds((const void*)(p + jj), (lds_void*)(lds + (u * (T / 64) + wave) * 64 * 16),
                                         16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t acc = 0;
#pragma unroll 4
    for (int u = 0; u < N; ++u) {
        const uint4 x = *reinterpret_cast<const uint4*>(lds + ((u * (T / 64) + wave) * 64 + lane) * 16);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    sink[(int64_t)blockIdx.x * T + threadIdx.x] = acc;
}

template <int U, int T>
int launch_reg(const uint4* q, int64_t n16, int32_t nwg, uint32_t* sink, hipStream_t s) {
    const int64_t per = (n16 + nwg - 1) / nwg;
    hipLaunchKernelGGL((read_kernel<U, T>), dim3(nwg), dim3(T), 0, s, q, n16, per, sink);
    return (int)hipGetLastError();
}

template <int N, int T>
int launch_lds(const uint4* q, int64_t n16, uint32_t* sink, hipStream_t s) {
    const size_t lds = (size_t)N * T * 16;
    hipError_t e = hipFuncSetAttribute((const void*)read_lds_kernel<N, T>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    const int64_t nwg = (n16 + (int64_t)N * T - 1) / ((int64_t)N * T);
    hipLaunchKernelGGL((read_lds_kernel<N, T>), dim3((unsigned)nwg), dim3(T), lds, s, q, n16, sink);
    return (int)hipGetLastError();
}

}  // namespace

extern "C" int kvprobe_read(const void* p, int64_t bytes, int32_t n_workgroups, int32_t unroll, uint32_t* sink,
                            void* stream) {
    return kvprobe_read_shape(p, bytes, n_workgroups, 256, unroll, 0, sink, stream);
}

extern "C" int64_t kvprobe_lds_workgroups(int64_t bytes, int32_t threads, int32_t loads) {
    if (bytes <= 0 || threads <= 0 || loads <= 0) return -1;
    const int64_t n16 = (bytes + 15) / 16, share = (int64_t)threads * loads;
    return (n16 + share - 1) / share;
}

extern "C" int kvprobe_read_shape(const void* p, int64_t bytes, int32_t n_workgroups, int32_t threads, int32_t loads,
                                  int32_t lds_dma, void* sink_, void* stream) {
    uint32_t* sink = static_cast<uint32_t*>(sink_);
    if (!p || !sink || bytes <= 0 || bytes % 16 || ((uintptr_t)p % 16)) return -1;
    const int64_t n16 = bytes / 16;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* q = static_cast<const uint4*>(p);
#define KVP_REG(U, T) \
    if (loads == U && threads == T) return launch_reg<U, T>(q, n16, n_workgroups, sink, s);
#define KVP_LDS(N, T) \
    if (loads == N && threads == T) return launch_lds<N, T>(q, n16, sink, s);
    if (!lds_dma) {
        if (n_workgroups <= 0) return -1;
        KVP_REG(1, 256) KVP_REG(4, 256) KVP_REG(8, 256) KVP_REG(16, 256) KVP_REG(32, 256)
        KVP_REG(4, 512) KVP_REG(8, 512) KVP_REG(16, 512) KVP_REG(32, 512)
        KVP_REG(4, 1024) KVP_REG(8, 1024) KVP_REG(16, 1024)
    } else {
        KVP_LDS(8, 256) KVP_LDS(16, 256) KVP_LDS(32, 256)
        KVP_LDS(8, 512) KVP_LDS(16, 512)
        KVP_LDS(4, 1024) KVP_LDS(8, 1024)
    }
#undef KVP_REG
#undef KVP_LDS
    return -1;
}
