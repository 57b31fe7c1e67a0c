// Adjoint of the fused entry's causal conv + SiLU (gfx950), after the scan
// backward has written d_u.
//
// Step F4a of the per-layer forward (mamba-rs 0.3.1
// src/mamba_ssm/gpu/forward_mixed.rs) is u_t = silu(p_t) with
//   p_t = conv_b[i] + sum_k conv_w[i,k] x_{t-K+1+k}
// over the carried conv state for t-K+1+k < 0.  Its adjoint, per channel:
//   dp_t         = (d_u_t + d_u_extra_t) silu'(p_t)      (p_t recomputed)
//   d_x_s        = sum_k conv_w[i,k] dp_{s+K-1-k}        (dp past T-1 is 0)
//   d_conv_w[k] += sum_t dp_t x_{t-K+1+k},   d_conv_b += sum_t dp_t
// (no gradient flows into the incoming conv state).  d_x at step s needs dp
// up to K-1 steps later, across tile and segment borders, which is why this
// runs as a pass of its own: every d_u is final when it starts.
//
// Mapping.  Thread = channel (consecutive channels, so every access is
// contiguous across a wave), workgroup = 256 channels of one batch row and
// one tile of kConvBwdTT steps, walked forward in time with the latest
// inputs and dp in registers; the tile's last d_x take dp of the steps
// after it, recomputed.  Taps are zero-padded at the front to four
// so the step has no branch on K.  Weight and bias partials go out per
// (batch row, tile) and are summed in a fixed order by mscan_reduce_kernel.
#pragma once
#include "scan_common.h"

namespace mscan {

constexpr int kConvBwdTT = 64;   // steps per tile

struct ConvBwdArgs {
  const void* x;            // [B,T,Di] conv input
  const float* conv_w;      // [Di,K]
  const float* conv_b;      // [Di] or null
  const float* conv_state0; // [B,Di,K] or null
  const float* du;          // [B,T,Di] f32, from the scan backward
  const void* d_u_extra;    // [B,T,Di] or null
  void* d_x;                // [B,T,Di]
  float* part;              // [B * ntiles, Di, K + 1]: d_conv_w | d_conv_b per (batch row, tile)
  int64_t B, T, Di;
  int K;
};

__host__ __device__ inline int64_t conv_bwd_tiles(int64_t T) { return (T + kConvBwdTT - 1) / kConvBwdTT; }

template <Act A>
__global__ void __launch_bounds__(256) conv_bwd_kernel(const ConvBwdArgs p) {
  constexpr int KM = 4;
  using io = IO<A>;
  const int64_t T = p.T, Di = p.Di;
  const int K = p.K;
  const int64_t ncb = (Di + 255) / 256;
  const int64_t ntiles = conv_bwd_tiles(T);
  const int64_t cb_ = blockIdx.x % ncb, rest = blockIdx.x / ncb;   // rest = b * ntiles + tile
  const int64_t i = cb_ * 256 + threadIdx.x;
  if (i >= Di) return;
  const int64_t b = rest / ntiles;
  const int64_t t0 = (rest % ntiles) * kConvBwdTT;
  const int64_t t1 = t0 + kConvBwdTT < T ? t0 + kConvBwdTT : T;
  const int64_t row0 = b * T;

  float w[KM], win[KM - 1], dpw[KM];   // w padded at the front; win[m] = x_{t-(KM-1)+m}; dpw[k] = dp_{t-k}
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int j = k - (KM - K);
    w[k] = j >= 0 ? p.conv_w[i * K + j] : 0.0f;
    dpw[k] = 0.0f;
  }
  const float bias = p.conv_b ? p.conv_b[i] : 0.0f;
#pragma unroll
  for (int m = 0; m < KM - 1; ++m) {
    const int64_t s = t0 - (KM - 1) + m;
    float xv = 0.0f;
    if (s >= 0) xv = io::ld(p.x, (row0 + s) * Di + i);
    else if (p.conv_state0 && s >= -static_cast<int64_t>(K)) xv = p.conv_state0[(b * Di + i) * K + (K + s)];
    win[m] = xv;
  }
  float acc[KM] = {0.0f, 0.0f, 0.0f, 0.0f}, acc_b = 0.0f;
  // d_x_s is emitted at step s + KM-1 (whatever K: with the taps padded at
  // the front, dp_{s+K-1-k} of tap k is dpw[KM-K+k] then), so the walk runs
  // KM-1 steps past the tile
  const int64_t t_stop = t1 + (KM - 1);             // the last d_x emitted is step t1 - 1
  const int64_t t_data = t_stop < T ? t_stop : T;   // steps with data
  constexpr int U = 8;                               // steps whose inputs are loaded together
  for (int64_t ts = t0; ts < t_stop; ts += U) {
    float xs[U], gs[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {   // clamped to the data, so every load is unconditional
      const int64_t e = (row0 + (ts + j < t_data ? ts + j : t_data - 1)) * Di + i;
      xs[j] = io::ld(p.x, e);
      gs[j] = p.du[e] + (p.d_u_extra ? io::ld(p.d_u_extra, e) : 0.0f);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t t = ts + j;
      if (t >= t_stop) break;
      float g = 0.0f;
      if (t < t_data) {
        const float xt = xs[j];
        // padded taps are skipped by a select, not multiplied by zero: a
        // non-finite input they would see must not reach the sum
        float pre = fmaf(w[KM - 1], xt, bias);
#pragma unroll
        for (int m = 0; m < KM - 1; ++m) pre = m >= KM - K ? fmaf(w[m], win[m], pre) : pre;
        const float sg = sigmoid(pre);
        g = gs[j] * (sg * (1.0f + pre * (1.0f - sg)));
        if (t < t1) {
#pragma unroll
          for (int m = 0; m < KM - 1; ++m) acc[m] = fmaf(g, win[m], acc[m]);
          acc[KM - 1] = fmaf(g, xt, acc[KM - 1]);
          acc_b += g;
        }
#pragma unroll
        for (int m = 0; m < KM - 2; ++m) win[m] = win[m + 1];
        win[KM - 2] = xt;
      }
#pragma unroll
      for (int k = KM - 1; k > 0; --k) dpw[k] = dpw[k - 1];
      dpw[0] = g;
      // d_x_s, s = t - (KM-1): sum_k conv_w[i,k] dp_{s+K-1-k} = sum over
      // the padded taps k' of w[k'] dpw[k']
      const int64_t s = t - (KM - 1);
      if (s >= t0 && s < t1) {
        float gx = 0.0f;
#pragma unroll
        for (int k = 0; k < KM; ++k) gx = k >= KM - K ? fmaf(w[k], dpw[k], gx) : gx;
        io::st(p.d_x, (row0 + s) * Di + i, gx);
      }
    }
  }
  float* part = p.part + (rest * Di + i) * (K + 1);
  for (int k = 0; k < K; ++k) part[k] = acc[KM - K + k];
  part[K] = acc_b;
}

template <Act A>
hipError_t launch_conv_bwd(const ConvBwdArgs& p, hipStream_t st) {
  const int64_t n = (p.Di + 255) / 256 * p.B * conv_bwd_tiles(p.T);
  hipLaunchKernelGGL(conv_bwd_kernel<A>, dim3(static_cast<unsigned>(n)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mscan
