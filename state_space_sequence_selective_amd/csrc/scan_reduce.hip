// Fixed-order reduction of the backward's per-group / per-(segment, batch
// row) partials into the caller's accumulated gradients (d_xdbl B/C
// columns, d_a_log, d_D, d_conv_w, d_conv_b).  No atomics: every output
// element is summed by one thread in ascending group / row order, so
// repeated runs give identical bits.
#include "scan_common.h"

namespace mscan {

__global__ void __launch_bounds__(256) mscan_reduce_kernel(const ReduceArgs p) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t BT = p.B * p.T;
  const int64_t W = 2 * p.Ds;
  const int64_t nbc = BT * W;
  if (j < nbc) {
    const int64_t row = j / W, m = j % W;
    p.d_xdbl[row * p.X + p.R + m] += ordered_sum(p.part_bc + row * W + m, p.nG, BT * W);
    return;
  }
  const int64_t jp = j - nbc;
  if (jp >= p.Di * p.PW) return;
  const int64_t i = jp / p.PW, slot = jp % p.PW;
  const float acc = ordered_sum(p.part_par + i * p.PW + slot, p.par_rows, p.Di * p.PW);
  if (slot < p.Ds) {
    p.d_a_log[i * p.Ds + slot] += acc;
  } else if (slot == p.Ds) {
    p.d_D[i] += acc;
  } else if (slot < p.Ds + 1 + p.K) {
    p.d_conv_w[i * p.K + (slot - p.Ds - 1)] += acc;
  } else {
    p.d_conv_b[i] += acc;
  }
}

hipError_t launch_reduce(const ReduceArgs& p, hipStream_t st) {
  const int64_t n = p.B * p.T * 2 * p.Ds + p.Di * p.PW;
  dim3 grid(static_cast<unsigned>((n + 255) / 256));
  hipLaunchKernelGGL(mscan_reduce_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mscan
