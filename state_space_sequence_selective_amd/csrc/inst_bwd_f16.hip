// Backward kernels with f16 activations.
#include "scan_bwd.h"
#include "scan_conv.h"

namespace mscan {
hipError_t launch_bwd_f16(const BwdArgs& p, int ds, int L, hipStream_t st) {
  return launch_bwd_a<Act::F16>(p, ds, L, st);
}
hipError_t launch_carry_f16(const CarryArgs& p, int ds, hipStream_t st) {
  return launch_carry_a<Act::F16>(p, ds, st);
}
hipError_t launch_conv_bwd_f16(const ConvBwdArgs& p, hipStream_t st) {
  return launch_conv_bwd<Act::F16>(p, st);
}
}  // namespace mscan
