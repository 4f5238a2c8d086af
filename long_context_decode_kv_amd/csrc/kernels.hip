// The log-sum-exp merge kernel of kvdec_merge and the dispatch from a
// (head_dim, group, K kind, V kind) to its split-kernel instance (compiled in
// the split_*.hip translation units).

#include "split_kernels.h"

namespace kvdec {
namespace {

// kvdec_merge: one workgroup per row, one thread per element of head_dim.
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
    const int64_t row = blockIdx.x;
    for (int d = threadIdx.x; d < a.head_dim; d += blockDim.x) {
        float M = kNegInf;
        for (int p = 0; p < a.n_parts; ++p) M = fmaxf(M, a.m[p][row]);
        float L = 0.f, O = 0.f;
        if (M != kNegInf) {
            for (int p = 0; p < a.n_parts; ++p) {
                const float mp = a.m[p][row];
                if (mp == kNegInf) continue;
                const float f = __expf(mp - M);
                L += a.l[p][row] * f;
                O += a.o[p][row * a.head_dim + d] * f;
            }
        }
        const bool empty = !(L > 0.f);
        if (a.out) a.out[row * a.head_dim + d] = empty ? 0.f : O / L;
        if (a.mo) a.mo[row * a.head_dim + d] = O;
        if (d == 0) {
            if (a.lse) a.lse[row] = empty ? kNegInf : M + __logf(L);
            if (a.mm) {
                a.mm[row] = empty ? kNegInf : M;
                a.ml[row] = L;
            }
        }
    }
}

}  // namespace

SplitLaunchFn pick_split(int head_dim, int g, int n_q, int kt, int vt, bool mfma) {
    // K stored at least as finely as V: f16/f16, int8/int8, 4-bit/4-bit,
    // f16/int8, f16/4-bit, int8/4-bit.
    if (kt == KVDEC_F16 && vt == KVDEC_F16) return pick_split_f16(head_dim, g, n_q, mfma);
    if (kt == KVDEC_Q8_B32 && vt == KVDEC_Q8_B32) return pick_split_q8(head_dim, g, n_q, mfma);
    if (kt == KVDEC_Q4_B32 && vt == KVDEC_Q4_B32) return pick_split_q4(head_dim, g, n_q, mfma);
    if (kt == KVDEC_F16 && vt == KVDEC_Q8_B32) return pick_split_f16_q8(head_dim, g, n_q, mfma);
    if (kt == KVDEC_F16 && vt == KVDEC_Q4_B32) return pick_split_f16_q4(head_dim, g, n_q, mfma);
    if (kt == KVDEC_Q8_B32 && vt == KVDEC_Q4_B32) return pick_split_q8_q4(head_dim, g, n_q, mfma);
    return nullptr;
}

bool split_instance_exists(int head_dim, int group, int n_q, int k_type, int v_type, bool mfma) {
    return pick_split(head_dim, group, n_q, k_type, v_type, mfma) != nullptr;
}

int launch_split(int head_dim, int group, int n_q, int k_type, int v_type, bool mfma, const SplitArgs& a,
                 void* stream) {
    SplitLaunchFn f = pick_split(head_dim, group, n_q, k_type, v_type, mfma);
    if (!f) return (int)hipErrorInvalidValue;
    return f(a, stream);
}

int launch_merge(const MergeArgs& a, void* stream) {
    const int threads = a.head_dim >= 256 ? 256 : (a.head_dim >= 64 ? ((a.head_dim + 63) / 64) * 64 : 64);
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.n_rows), dim3(threads), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace kvdec
