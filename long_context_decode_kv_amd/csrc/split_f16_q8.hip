// Split-kernel instances for K stored as KVDEC_F16 and V as KVDEC_Q8_B32.
#include "split_kernels.h"

namespace kvdec {
SplitLaunchFn pick_split_f16_q8(int head_dim, int group, int n_q, bool mfma) {
    return pick_dg<KVDEC_F16, KVDEC_Q8_B32>(head_dim, group, n_q, mfma);
}
}  // namespace kvdec
