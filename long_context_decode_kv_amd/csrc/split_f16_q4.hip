// Split-kernel instances for K stored as KVDEC_F16 and V as KVDEC_Q4_B32.
#include "split_kernels.h"

namespace kvdec {
SplitLaunchFn pick_split_f16_q4(int head_dim, int group) { return pick_dg<KVDEC_F16, KVDEC_Q4_B32>(head_dim, group); }
}  // namespace kvdec
