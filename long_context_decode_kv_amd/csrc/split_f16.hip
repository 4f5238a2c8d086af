// Split-kernel instances for K stored as KVDEC_F16 and V as KVDEC_F16.
#include "split_kernels.h"

namespace kvdec {
SplitLaunchFn pick_split_f16(int head_dim, int group, int n_q, bool mfma) {
    return pick_dg<KVDEC_F16, KVDEC_F16>(head_dim, group, n_q, mfma);
}
}  // namespace kvdec
