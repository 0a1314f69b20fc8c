// scan_fwd_s2.hip -- instantiations of the one-segment prefill scan with 2
// state slot(s) per lane (dstate up to 32); the kernel is in scan_fwd_kernel.h.
#include "scan_fwd_kernel.h"

namespace ssm {
namespace fwd {

template <>
void launch_slots<2>(int pass, int lane, bool bf16, bool softplus, int K, bool defer,
                      dim3 grid, const ScanParams& p, hipStream_t stream) {
  if (pass != 0) launch_slots_seg<2>(pass, lane, bf16, softplus, K, grid, p, stream);
  else launch_mode<Mode::kScan, 2>(lane, bf16, softplus, K, defer, grid, p, stream);
}

}  // namespace fwd
}  // namespace ssm
