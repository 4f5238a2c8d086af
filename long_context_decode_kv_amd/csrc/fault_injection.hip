// Test build only (libkvdec_fi.so, with api.cpp compiled under
// KVDEC_FAULT_INJECTION): host-side failure injection for the tail
// streamer, and a bounded delay kernel that makes the readers of the tail
// staging ring slow.  No injected failure touches the device: a failing
// copy or launch is simply not enqueued and reports an error code.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace kvdec {
namespace {

int g_fail_copy = -1;    // the n-th host-to-device tail copy from now fails (0-based); -1: none
int g_fail_launch = -1;  // the n-th split-kernel launch from now fails; -1: none
int g_delay = 0;         // s_sleep iterations of the delay kernel before each tail-chunk kernel

// About 127 * 64 cycles per iteration; always ends after `iters` of them.
__global__ void delay_kernel(int iters) {
    for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

bool fi_fail_copy() {
    if (g_fail_copy < 0) return false;
    return g_fail_copy-- == 0;
}

bool fi_fail_launch() {
    if (g_fail_launch < 0) return false;
    return g_fail_launch-- == 0;
}

int fi_delay(void* stream) {
    if (g_delay <= 0) return 0;
    hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), g_delay);
    return (int)hipGetLastError();
}

}  // namespace kvdec

// fail_copy / fail_launch: index (from the next one on) of the tail copy /
// split-kernel launch that fails, or -1; delay_iters: delay before each
// tail-chunk kernel (0: none).  Process-wide; for single-threaded tests.
extern "C" void kvdec_fi_configure(int fail_copy, int fail_launch, int delay_iters) {
    kvdec::g_fail_copy = fail_copy;
    kvdec::g_fail_launch = fail_launch;
    kvdec::g_delay = delay_iters > 0 ? delay_iters : 0;
}
