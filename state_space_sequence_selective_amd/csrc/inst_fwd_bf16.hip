// Forward kernels with bf16 activations.
#include "scan_fwd.h"
#include "scan_step.h"

namespace mscan {
hipError_t launch_fwd_bf16(const FwdArgs& p, int ds, int spl, hipStream_t st) {
  return launch_fwd_a<Act::BF16>(p, ds, spl, st);
}
hipError_t launch_step_bf16(const FwdArgs& p, int ds, hipStream_t st) {
  return launch_step_a<Act::BF16>(p, ds, st);
}
}  // namespace mscan
