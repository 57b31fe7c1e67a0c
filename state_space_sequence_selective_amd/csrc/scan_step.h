// Forward for short sequences (recurrent steps, T <= kStepMaxT; kStepMaxT is
// at most the checkpoint interval, so there is one checkpoint), gfx950.
//
// The forward_mixed page runs one thread per channel, sequential in time, for
// its burn-in / step path.  That layout suits the regime where there is too
// little time for the tiled kernel's staging to pay: thread (b, i) keeps all
// d_state states of channel i in registers, reads its own contiguous 64-byte
// slice of h0 / conv_state0, and walks the T steps doing the per-channel work
// (conv + SiLU, softplus, gate) once.  Lanes are consecutive channels, so the
// activation reads and writes, the state reads / writes and the checkpoint
// writes are all contiguous across a wave.  The B_t / C_t row is the same for
// every channel of a batch row and is served from the caches.
#pragma once
#include "scan_common.h"

namespace mscan {

template <Act A, int DS, bool FUSED>
__global__ void __launch_bounds__(256) scan_step_kernel(const FwdArgs p) {
  constexpr int KMAX = FUSED ? 4 : 1;
  using io = IO<A>;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= p.B * p.Di) return;
  const int64_t Di = p.Di, T = p.T;
  const int64_t b = j / Di, i = j % Di;
  const int K = FUSED ? p.K : 0;
  const bool gate = p.z != nullptr;

  float a2[DS], h[DS];
#pragma unroll
  for (int n = 0; n < DS; ++n) {
    a2[n] = -expf(p.a_log[i * DS + n]) * kLog2e;
    h[n] = p.h0 ? p.h0[j * DS + n] : 0.0f;
  }
  if (p.ckpt) {   // the state entering step 0 (T <= L: the only checkpoint)
#pragma unroll
    for (int n = 0; n < DS; ++n) p.ckpt[((b * p.nC) * DS + n) * Di + i] = h[n];
  }
  const float Dv = p.D ? p.D[i] : 0.0f;
  // conv window of the inputs before the current step: win[KMAX-1-m] holds
  // the input m+1 steps back.  Before step 0 those are the incoming state,
  // whose entry K-1 is the most recent input (oldest first).
  float cw[KMAX], win[KMAX];
  float cb = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    cw[k] = (FUSED && k < K) ? p.conv_w[i * K + k] : 0.0f;
    const int si = k - (KMAX - K);   // state entry for window slot k
    win[k] = (FUSED && si >= 0 && p.conv_state0) ? p.conv_state0[j * K + si] : 0.0f;
  }
  if (FUSED && p.conv_b) cb = p.conv_b[i];

  for (int64_t t = 0; t < T; ++t) {
    const int64_t e = (b * T + t) * Di + i;
    float u;
    if (FUSED) {
      // shift the window by one step: win[KMAX-1-m] is now m steps back, and
      // x_t goes into the last slot after the taps
#pragma unroll
      for (int k = 0; k < KMAX - 1; ++k) win[k] = win[k + 1];
      const float xt = io::ld(p.x, e);
      float pre = cb;
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (k < K) {
          // tap k multiplies the input at step t - (K-1) + k
          const float v = (k == K - 1) ? xt : win[KMAX - K + k];
          pre = fmaf(cw[k], v, pre);
        }
      }
      win[KMAX - 1] = xt;
      u = pre * sigmoid(pre);
      if (p.u_out) io::st(p.u_out, e, u);
    } else {
      u = io::ld(p.x, e);
    }
    const float dl = softplus(io::ld(p.delta_raw, e));
    const float du = dl * u;
    const int64_t row = (b * T + t) * p.X + p.R;
    float y = Dv * u;
#pragma unroll
    for (int n = 0; n < DS; ++n) {
      const float dA = exp2_fast(dl * a2[n]);
      h[n] = fmaf(dA, h[n], du * io::ld(p.xdbl, row + n));
      y = fmaf(io::ld(p.xdbl, row + DS + n), h[n], y);
    }
    float out = y;
    if (gate) {
      const float zv = io::ld(p.z, e);
      out = y * zv * sigmoid(zv);
    }
    io::st(p.out, e, out);
    if (p.y_save) io::st(p.y_save, e, y);
  }

  if (p.h_last) {
#pragma unroll
    for (int n = 0; n < DS; ++n) p.h_last[j * DS + n] = h[n];
  }
  if (FUSED && p.conv_state_last) {
    for (int k = 0; k < K; ++k) {
      const int64_t s = T - K + k;
      float xv;
      if (s >= 0) xv = io::ld(p.x, (b * T + s) * Di + i);
      else xv = p.conv_state0 ? p.conv_state0[j * K + (K + s)] : 0.0f;
      p.conv_state_last[j * K + k] = xv;
    }
  }
}

template <Act A>
hipError_t launch_step_a(const FwdArgs& p, int ds, hipStream_t st) {
  dim3 grid(static_cast<unsigned>((p.B * p.Di + 255) / 256));
#define MSCAN_CASE(DS_)                                                                         \
  if (ds == DS_) {                                                                              \
    if (p.K > 0) hipLaunchKernelGGL((scan_step_kernel<A, DS_, true>), grid, dim3(256), 0, st, p); \
    else hipLaunchKernelGGL((scan_step_kernel<A, DS_, false>), grid, dim3(256), 0, st, p);       \
    return hipGetLastError();                                                                   \
  }
  MSCAN_CASE(4) MSCAN_CASE(8) MSCAN_CASE(16) MSCAN_CASE(32)
#undef MSCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace mscan
