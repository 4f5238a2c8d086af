// Split-kernel instances for K stored as KVDEC_Q8_B32 and V as KVDEC_Q8_B32.
#include "split_kernels.h"

namespace kvdec {
SplitLaunchFn pick_split_q8(int head_dim, int group, int n_q, bool mfma) {
    return pick_dg<KVDEC_Q8_B32, KVDEC_Q8_B32>(head_dim, group, n_q, mfma);
}
}  // namespace kvdec
