// The device memory of kvdec_attend_static: one file-scope array that each
// GPU the library runs on holds until the process ends, laid out as a merge
// ticket area (KVDEC_STATIC_TICKET_BYTES) followed by a plan workspace
// (KVDEC_STATIC_WORKSPACE_BYTES).  Host code never passes the array's name to
// a kernel or a copy: in host code that name is a stand-in, not a device
// address.  The device address is looked up once per device, with that
// device current, and kept here.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace kvdec {
namespace {

constexpr size_t kScratchBytes = (size_t)KVDEC_STATIC_TICKET_BYTES + (size_t)KVDEC_STATIC_WORKSPACE_BYTES;
static_assert(KVDEC_STATIC_TICKET_BYTES % (256 * 16) == 0, "the clear kernel writes 16 bytes per thread per step");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void* ptr = nullptr;   // this device's copy of `scratch`
    bool cleared = false;  // a clear of the ticket area was enqueued outside stream capture
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// Zero the ticket area: one workgroup of 256 threads, 16-byte vector stores.
__global__ __launch_bounds__(256) void clear_tickets(uint4* t) {
    for (int i = threadIdx.x; i < KVDEC_STATIC_TICKET_BYTES / 16; i += 256) t[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

int static_scratch(void* stream, void** base) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch& d = g_dev[dev];
    if (!d.ptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!ptr) return (int)hipErrorInvalidSymbol;
        d.ptr = ptr;
    }
    if (!d.cleared) {
        // A clear recorded into a graph runs only when the graph does, so
        // only an enqueue outside capture counts as done.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap);
        if (e != hipSuccess) return (int)e;
        hipLaunchKernelGGL(clear_tickets, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<uint4*>(d.ptr));
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        if (cap == hipStreamCaptureStatusNone) d.cleared = true;
    }
    *base = d.ptr;
    return (int)hipSuccess;
}

}  // namespace kvdec
