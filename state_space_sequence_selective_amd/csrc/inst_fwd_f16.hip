// Forward kernels with f16 activations.
#include "scan_fwd.h"
#include "scan_step.h"

namespace mscan {
hipError_t launch_fwd_f16(const FwdArgs& p, int ds, int spl, hipStream_t st) {
  return launch_fwd_a<Act::F16>(p, ds, spl, st);
}
hipError_t launch_step_f16(const FwdArgs& p, int ds, hipStream_t st) {
  return launch_step_a<Act::F16>(p, ds, st);
}
}  // namespace mscan
