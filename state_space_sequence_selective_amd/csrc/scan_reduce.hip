// Fixed-order reduction of the backward's per-group / per-(segment, batch
// row) / per-(batch row, conv tile) partials into the caller's accumulated
// gradients (d_xdbl B/C columns, d_a_log, d_D, d_conv_w, d_conv_b).  No
// atomics: every output element is summed by one thread in ascending
// group / row order, so repeated runs give identical bits.  Also the fold
// of the segmented backward's carry pairs into each segment's starting
// carry, in a fixed order too.
#include "scan_common.h"

namespace mscan {

// four adjacent B/C columns (W = 2 * d_state is a multiple of 4, the
// partials 16-byte aligned) summed over the groups in ascending order
__device__ __forceinline__ float4 ordered_sum4(const float* src, int64_t n, int64_t stride) {
  constexpr int U = 8;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  int64_t r = 0;
  for (; r + U <= n; r += U) {
    float4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = *reinterpret_cast<const float4*>(src + (r + k) * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      acc.x += v[k].x;
      acc.y += v[k].y;
      acc.z += v[k].z;
      acc.w += v[k].w;
    }
  }
  for (; r < n; ++r) {
    const float4 v = *reinterpret_cast<const float4*>(src + r * stride);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  return acc;
}

// The grid puts the conv weight / bias sums (fused entry) first: each is a
// chain of strided loads over the batch rows and conv tiles, so they start at
// once and run beside the bandwidth-bound B/C sums that follow; four
// adjacent lanes share one, each summing a quarter of the rows, and the
// quarters are added in order.  The a_log / D sums over the segments and
// batch rows come last.
constexpr int kConvQuarters = 4;

__global__ void __launch_bounds__(256) mscan_reduce_kernel(const ReduceArgs p) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t CW = p.K + 1;
  constexpr int CQ = kConvQuarters;
  static_assert(CQ == 4, "the quarters are added as ((q0 + q1) + q2) + q3");
  const int64_t nconv = p.K > 0 ? p.Di * CW * CQ : 0;   // whole quads of lanes
  if (j < nconv) {   // conv weight and bias partials
    const int64_t c = j / CQ, i = c / CW, slot = c % CW;
    const int q = static_cast<int>(j % CQ);
    const int64_t per = (p.conv_rows + CQ - 1) / CQ, r0 = q * per;
    const int64_t r1 = r0 + per < p.conv_rows ? r0 + per : p.conv_rows;
    const float v = r1 > r0 ? ordered_sum<16>(p.part_conv + r0 * p.Di * CW + c, r1 - r0, p.Di * CW) : 0.0f;
    const float v1 = __shfl_down(v, 1, CQ), v2 = __shfl_down(v, 2, CQ), v3 = __shfl_down(v, 3, CQ);
    if (q == 0) {
      const float acc = ((v + v1) + v2) + v3;
      if (slot < p.K) p.d_conv_w[i * p.K + slot] += acc;
      else p.d_conv_b[i] += acc;
    }
    return;
  }
  const int64_t jb = j - nconv;   // B/C columns, four per thread
  const int64_t BT = p.B * p.T;
  const int64_t W = 2 * p.Ds;
  const int64_t nbc4 = BT * W / 4;
  if (jb < nbc4) {
    const int64_t row = jb / (W / 4), m = (jb % (W / 4)) * 4;
    const float4 s = ordered_sum4(p.part_bc + row * W + m, p.nG, BT * W);
    float* o = p.d_xdbl + row * p.X + p.R + m;
    o[0] += s.x;
    o[1] += s.y;
    o[2] += s.z;
    o[3] += s.w;
    return;
  }
  const int64_t jp = jb - nbc4;
  if (jp >= p.Di * p.PW) return;
  const int64_t i = jp / p.PW, slot = jp % p.PW;
  const float acc = ordered_sum<16>(p.part_par + i * p.PW + slot, p.par_rows, p.Di * p.PW);
  if (slot < p.Ds) p.d_a_log[i * p.Ds + slot] += acc;
  else p.d_D[i] += acc;
}

// Starting carry of every backward segment from the carry pass's
// sub-segment pairs (Q_q, sum of delta_q), folded from the last sub-segment
// down as  c <- exp2(A log2(e) sum of delta_q) c + Q_q;  the value after
// sub-segment s*F is what segment s-1 starts its reverse sweep from, and
// the last segment starts from zero.  One thread per (batch row, channel,
// state), states fastest; QU sub-segments' loads are issued before their
// FMAs (indexes past the range clamped, their values unused).
__global__ void __launch_bounds__(256) mscan_carry_fold_kernel(const CarryFoldArgs p) {
  constexpr int QU = 8;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t DD = p.Di * p.Ds;
  if (j >= p.B * DD) return;
  const int64_t b = j / DD, in = j % DD, i = in / p.Ds;
  const float a2 = -expf(p.a_log[in]) * kLog2e;
  const int64_t SF = static_cast<int64_t>(p.S) * p.F;
  p.seg_c[(b * p.S + p.S - 1) * DD + in] = 0.0f;
  float c = 0.0f;
  for (int64_t q0 = SF - 1; q0 >= p.F; q0 -= QU) {
    float sd[QU], qv[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t r = b * SF + (q0 - u >= p.F ? q0 - u : p.F);
      sd[u] = p.seg_sd[r * p.Di + i];
      qv[u] = p.seg_q[r * DD + in];
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t q = q0 - u;
      if (q >= p.F) {
        c = fmaf(exp2_fast(a2 * sd[u]), c, qv[u]);
        if (q % p.F == 0) p.seg_c[(b * p.S + q / p.F - 1) * DD + in] = c;
      }
    }
  }
}

hipError_t launch_carry_fold(const CarryFoldArgs& p, hipStream_t st) {
  const int64_t n = p.B * p.Di * p.Ds;
  hipLaunchKernelGGL(mscan_carry_fold_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& p, hipStream_t st) {
  const int64_t n = p.B * p.T * 2 * p.Ds / 4 + p.Di * p.PW + (p.K > 0 ? p.Di * (p.K + 1) * kConvQuarters : 0);
  dim3 grid(static_cast<unsigned>((n + 255) / 256));
  hipLaunchKernelGGL(mscan_reduce_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mscan
