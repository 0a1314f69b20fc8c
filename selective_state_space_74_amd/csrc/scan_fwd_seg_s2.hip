// scan_fwd_seg_s2.hip -- instantiations of the two passes of the segmented
// prefill scan with 2 state slot(s) per lane (dstate up to 32); the kernel
// is in scan_fwd_kernel.h.
#include "scan_fwd_kernel.h"

namespace ssm {
namespace fwd {

template <>
void launch_slots_seg<2>(int pass, int lane, bool bf16, bool softplus, int K, dim3 grid,
                          const ScanParams& p, hipStream_t stream) {
  if (pass == 1) launch_mode<Mode::kSeg, 2>(lane, bf16, softplus, K, false, grid, p, stream);
  else launch_mode<Mode::kFix, 2>(lane, bf16, softplus, K, false, grid, p, stream);
}

}  // namespace fwd
}  // namespace ssm
