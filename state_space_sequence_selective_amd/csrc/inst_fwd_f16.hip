// Forward kernels with f16 activations.
#include "scan_fwd2.h"
#include "scan_step.h"

namespace mscan {
hipError_t launch_step_f16(const FwdArgs& p, int ds, hipStream_t st) {
  return launch_step_a<Act::F16>(p, ds, st);
}
hipError_t launch_fwd2_f16(const Fwd2Args& p, int ds, bool regen, hipStream_t st) {
  return launch_fwd2_a<Act::F16>(p, ds, regen, st);
}
hipError_t launch_bc_f32_f16(const BcArgs& p, hipStream_t st) {
  return launch_bc_f32<Act::F16>(p, st);
}
}  // namespace mscan
