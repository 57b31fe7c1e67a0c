// Backward kernels with bf16 activations.
#include "scan_bwd.h"

namespace mscan {
hipError_t launch_bwd_bf16(const BwdArgs& p, int ds, int L, hipStream_t st) {
  return launch_bwd_a<Act::BF16>(p, ds, L, st);
}
}  // namespace mscan
