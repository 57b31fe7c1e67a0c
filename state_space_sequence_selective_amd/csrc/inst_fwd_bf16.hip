// Forward kernels with bf16 activations.
#include "scan_fwd2.h"
#include "scan_step.h"

namespace mscan {
hipError_t launch_step_bf16(const FwdArgs& p, int ds, hipStream_t st) {
  return launch_step_a<Act::BF16>(p, ds, st);
}
hipError_t launch_fwd2_bf16(const Fwd2Args& p, int ds, bool regen, hipStream_t st) {
  return launch_fwd2_a<Act::BF16>(p, ds, regen, st);
}
hipError_t launch_bc_f32_bf16(const BcArgs& p, hipStream_t st) {
  return launch_bc_f32<Act::BF16>(p, st);
}
}  // namespace mscan
