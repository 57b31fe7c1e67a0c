// Forward kernels with f16 activations.
#include "scan_fwd.h"

namespace mscan {
hipError_t launch_fwd_f16(const FwdArgs& p, int ds, int spl, hipStream_t st) {
  return launch_fwd_a<Act::F16>(p, ds, spl, st);
}
}  // namespace mscan
