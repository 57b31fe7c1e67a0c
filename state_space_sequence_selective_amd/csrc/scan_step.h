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

// One step's inputs, fetched a step ahead and converted only where they are
// used: x / delta_raw / z as their element bits, and the B_t / C_t row as
// whole 32-bit words (two elements each when the activations are 16-bit).
// Unpacking 16-bit values at the load would make the compiler wait for the
// load right there.
template <Act A, int DS>
struct StepIn {
  static constexpr int NW = A == Act::F32 ? 2 * DS : DS;   // words in the B | C row
  uint32_t x, dr, z;
  uint32_t w[NW];

  __device__ __forceinline__ float bc(int n) const {   // element n of B | C
    if constexpr (A == Act::F32) {
      return __uint_as_float(w[n]);
    } else {
      const uint32_t h = (n & 1) ? w[n >> 1] >> 16 : w[n >> 1] & 0xffffu;
      return IO<A>::cvt(h);
    }
  }
};

template <Act A, int DS, bool FUSED>
__global__ void __launch_bounds__(256) scan_step_kernel(const FwdArgs p) {
  constexpr int KMAX = FUSED ? 4 : 1;
  constexpr int ES = A == Act::F32 ? 4 : 2;
  using io = IO<A>;
  using In = StepIn<A, DS>;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= p.B * p.Di) return;
  const int64_t Di = p.Di, T = p.T;
  const int64_t b = j / Di, i = j % Di;
  const int K = FUSED ? p.K : 0;
  const bool gate = p.z != nullptr;

  // Optional inputs are read unconditionally, from a stand-in address that is
  // always valid when the pointer is NULL (the value is then replaced): a
  // load under a branch makes the compiler wait for it before the branches
  // join, one memory round trip per optional input.
  const void* zsrc = gate ? p.z : p.x;   // same shape; unused without the gate
  const int64_t lz = gate ? p.ldz : Di;   // its row stride
  auto fetch = [&](int64_t t) {
    In s;
    const int64_t e = (b * T + t) * Di + i;
    s.x = io::ldraw(p.x, e);
    s.dr = io::ldraw(p.delta_raw, e);
    s.z = io::ldraw(zsrc, (b * T + t) * lz + i);
    // the row is contiguous; its start need not be 4-byte aligned, which
    // global loads allow
    const char* row = static_cast<const char*>(p.xdbl) + ((b * T + t) * p.X + p.R) * ES;
    __builtin_memcpy(s.w, row, sizeof(s.w));
    return s;
  };

  // every load of the call's first step is issued before anything is stored
  In cur = fetch(0);
  // stand-ins: h0 -> a_log (index i*DS+n), D -> a_log[i*DS],
  // conv_state0 -> conv_w (index i*K+k), conv_b -> conv_w[i*K]
  const bool has_h0 = p.h0 != nullptr, has_D = p.D != nullptr;
  const float* h0src = has_h0 ? p.h0 + j * DS : p.a_log + i * DS;
  float a2[DS], h[DS];
#pragma unroll
  for (int n = 0; n < DS; ++n) {
    a2[n] = p.a_log[i * DS + n];
    h[n] = h0src[n];
  }
  float Dv = (has_D ? p.D : p.a_log)[has_D ? i : i * DS];
  // conv window of the inputs before the current step: win[KMAX-1-m] holds
  // the input m+1 steps back.  Before step 0 those are the incoming state,
  // whose entry K-1 is the most recent input (oldest first).
  float cw[KMAX], win[KMAX];
  float cb = 0.0f;
  bool has_cs = false, has_cb = false;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    cw[k] = 0.0f;
    win[k] = 0.0f;
  }
  if (FUSED) {
    has_cs = p.conv_state0 != nullptr;
    has_cb = p.conv_b != nullptr;
    const float* cssrc = has_cs ? p.conv_state0 + j * K : p.conv_w + i * K;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int si = k - (KMAX - K);   // state entry for window slot k
      if (k < K) cw[k] = p.conv_w[i * K + k];
      if (si >= 0) win[k] = cssrc[si];
    }
    cb = (has_cb ? p.conv_b : p.conv_w)[has_cb ? i : i * K];
  }
  // replace what the stand-ins returned
#pragma unroll
  for (int n = 0; n < DS; ++n) h[n] = has_h0 ? h[n] : 0.0f;
  Dv = has_D ? Dv : 0.0f;
  if (FUSED) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) win[k] = has_cs ? win[k] : 0.0f;
    cb = has_cb ? cb : 0.0f;
  }
#pragma unroll
  for (int n = 0; n < DS; ++n) a2[n] = -expf(a2[n]) * kLog2e;
  if (p.ckpt) {   // the state entering step 0 (T <= L: the only checkpoint)
#pragma unroll
    for (int n = 0; n < DS; ++n) p.ckpt[((b * p.nC) * DS + n) * Di + i] = h[n];
  }

  auto step = [&](int64_t t, const In& s) {
    const int64_t e = (b * T + t) * Di + i;
    const float xt = io::cvt(s.x);
    float u;
    if (FUSED) {
      // tap k multiplies the input at step t - (K-1) + k; x_t is the newest
      float pre = cb;
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (k < K) pre = fmaf(cw[k], k == K - 1 ? xt : win[KMAX - K + k + 1], pre);
      }
      // shift the window by one step: win[KMAX-1] is now x_t
#pragma unroll
      for (int k = 0; k < KMAX - 1; ++k) win[k] = win[k + 1];
      win[KMAX - 1] = xt;
      u = pre * sigmoid(pre);
      if (p.u_out) io::st(p.u_out, e, u);
    } else {
      u = xt;
    }
    const float dl = softplus(io::cvt(s.dr));
    const float du = dl * u;
    float y = Dv * u;
#pragma unroll
    for (int n = 0; n < DS; ++n) {
      const float dA = exp2_fast(dl * a2[n]);
      h[n] = fmaf(dA, h[n], du * s.bc(n));
      y = fmaf(s.bc(DS + n), h[n], y);
    }
    float out = y;
    if (gate) {
      const float zv = io::cvt(s.z);
      out = y * zv * sigmoid(zv);
    }
    io::st(p.out, e, out);
    if (p.y_save) io::st(p.y_save, e, y);
  };

  // unrolled over the at most kStepMaxT steps: step t+1's loads (a clamped,
  // always valid row) are in flight while step t runs, and no value is
  // carried around a loop
#pragma unroll
  for (int t = 0; t < kStepMaxT; ++t) {
    const In nxt = fetch(t + 1 < T ? t + 1 : T - 1);
    step(t, cur);
    if (t + 1 >= T) break;
    cur = nxt;
  }

  if (p.h_last) {
#pragma unroll
    for (int n = 0; n < DS; ++n) p.h_last[j * DS + n] = h[n];
  }
  if (FUSED && p.conv_state_last) {
    // the last K inputs (from the incoming state where T < K) are the
    // window's newest K slots
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) p.conv_state_last[j * K + k] = win[KMAX - K + k];
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
  MSCAN_CASE(4) MSCAN_CASE(8) MSCAN_CASE(16) MSCAN_CASE(32) MSCAN_CASE(64)
#undef MSCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace mscan
