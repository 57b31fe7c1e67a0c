// Forward kernels with bf16 activations.
#include "scan_fwd.h"

namespace mscan {
hipError_t launch_fwd_bf16(const FwdArgs& p, int ds, int spl, hipStream_t st) {
  return launch_fwd_a<Act::BF16>(p, ds, spl, st);
}
}  // namespace mscan
