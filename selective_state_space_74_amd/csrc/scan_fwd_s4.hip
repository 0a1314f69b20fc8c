// scan_fwd_s4.hip -- instantiations of the one-segment prefill scan with 4
// state slot(s) per lane (dstate up to 64); the kernel is in scan_fwd_kernel.h.
#include "scan_fwd_kernel.h"

namespace ssm {
namespace fwd {

template <>
void launch_slots<4>(int pass, int lane, bool bf16, bool softplus, int K, bool defer,
                      dim3 grid, const ScanParams& p, hipStream_t stream) {
  if (pass != 0) launch_slots_seg<4>(pass, lane, bf16, softplus, K, grid, p, stream);
  else launch_mode<Mode::kScan, 4>(lane, bf16, softplus, K, defer, grid, p, stream);
}

}  // namespace fwd
}  // namespace ssm
