// Backward kernels with bf16 activations.
#include "scan_bwd.h"
#include "scan_conv.h"

namespace mscan {
hipError_t launch_bwd_bf16(const BwdArgs& p, int ds, int L, hipStream_t st) {
  return launch_bwd_a<Act::BF16>(p, ds, L, st);
}
hipError_t launch_carry_bf16(const CarryArgs& p, int ds, hipStream_t st) {
  return launch_carry_a<Act::BF16>(p, ds, st);
}
hipError_t launch_conv_bwd_bf16(const ConvBwdArgs& p, hipStream_t st) {
  return launch_conv_bwd<Act::BF16>(p, st);
}
}  // namespace mscan
