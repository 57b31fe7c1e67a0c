// Mamba-3 SISO state-space core (gfx950): forward and backward in 64-step
// chunks, and the C entry points of include/mamba3.h.
//
// The block follows the chunked state-space part of the per-layer backward
// on the mamba-rs 0.4.0 page src/mamba3_siso/gpu/backward_mixed.rs (B6, B5
// and B4b: m3_extract_da_cs_sum, m3_dqkv_typed, m3_dqktheta_typed,
// m3_ddt_dtrap, m3_angle_dt_bwd_seq, m3_final_grads, bc_bias_add_bwd, the
// bias column sums).  The update it is the chunked form of (a reading of
// that page's names: trap, gamma, scale, k_scaled, qk_dot, angle_cumsum,
// a_floor) is stated in include/mamba3.h.
//
// Chunked form.  Within a chunk (local steps t, s < 64, cum_t = sum of
// dt_r A_r over the chunk's steps r <= t, tot = cum of its last step) the
// trapezoidal update is an Euler-form update of a shifted state
//   St_t = S_t + (1 - lam_{t+1}) dt_{t+1} V_t K_t^T
// whose input weight is scale_t = lam_t dt_t + (1 - lam_{t+1}) dt_{t+1}:
//   y_t   = sum_{s<=t} e^{cum_t - cum_s} scale_s (Q_t . K_s) V_s
//           + e^{cum_t} St_in Q_t + (gamma_t - scale_t)(Q_t . K_t) V_t + D V_t
//   St_out = e^{tot} St_in + sum_s e^{tot - cum_s} scale_s V_s K_s^T
// (gamma_t = lam_t dt_t; the last term of y removes the part of scale_t
// that belongs to the next step).  The passes:
//   forward : m3_prep (per-step scalars) -> angle sums (chunked scan) ->
//             m3_rotate (turned Q, K) -> m3_chunk_state (each chunk's own
//             St_out) -> m3_state_pass (St_in of every chunk, in order) ->
//             m3_chunk_out (y)
//   backward: the first three again -> m3_chunk_state on (dY, Q) and a
//             reverse m3_state_pass (the gradient of every chunk's St_out)
//             -> m3_chunk_bwd (d_x, the gradients of the turned Q and K and
//             of each step's cum, scale, gamma) -> m3_rot_bwd -> angle-sum adjoint
//             -> m3_scalar_bwd -> fixed-order sums (groups, biases, D,
//             angles).  No atomics: every output is the same bits run to run.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "mamba3.h"
#include "scan_common.h"

namespace mscan {
void set_last_error(const std::string& msg);   // abi.hip
}

namespace m3 {

using mscan::Act;
using mscan::IO;

constexpr int kL = 64;    // steps per chunk
constexpr int kP = 64;    // channels per head
constexpr int kThreads = 256;

struct Dims {
  int64_t B, T, H, P, N, G, NA, nc;
  float a_floor;
};

__device__ __forceinline__ float expf_fast(float x) { return mscan::exp2_fast(x * mscan::kLog2e); }

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// inclusive suffix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_suffix_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_down(v, d, 64);
    if (lane + d < 64) v += o;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// ------------------------------------------------------------------ prep
// Per (b, h, t): dt, dt*A, gamma = lam*dt, scale = gamma + (1 - lam_{t+1}) dt_{t+1}
// (the next step's part is 0 past the end), all [B, H, T] f32.
struct PrepArgs {
  const float *dd_dt, *dd_a, *trap, *dt_bias;
  float *dt, *da, *gam, *sc;
  Dims d;
};

__global__ void __launch_bounds__(256) m3_prep_kernel(const PrepArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T) return;
  const int64_t t = i % d.T, bh = i / d.T, h = bh % d.H, b = bh / d.H;
  const int64_t in = (b * d.T + t) * d.H + h;
  const float bias = p.dt_bias[h];
  const float dt = mscan::softplus(p.dd_dt[in] + bias);
  const float A = -fmaxf(mscan::softplus(p.dd_a[in]), d.a_floor);
  const float lam = mscan::sigmoid(p.trap[in]);
  float nxt = 0.0f;
  if (t + 1 < d.T) {
    const float dt1 = mscan::softplus(p.dd_dt[in + d.H] + bias);
    nxt = (1.0f - mscan::sigmoid(p.trap[in + d.H])) * dt1;
  }
  p.dt[i] = dt;
  p.da[i] = dt * A;
  p.gam[i] = lam * dt;
  p.sc[i] = fmaf(lam, dt, nxt);
}

// ---------------------------------------------------------------- angles
// theta[b, h, t, a] = sum_{s<=t} dt[b, h, s] * angles_raw[b, s, a], and in
// the backward g[b, h, t, a] = sum_{s>=t} dtheta[b, h, s, a], as two-level
// scans over the 64-step chunks: each thread scans one (b, h, chunk, angle)
// and leaves the chunk's total; a pass per (b, h, angle) turns the totals
// into the sum of the chunks before (after) each one, which the kernels
// reading theta (the rotation and its adjoint) or g (the contribution pass)
// add to the chunk-local sums.
struct ScanArgs {
  const float *dt, *ang, *src;
  float *out, *ctot;
  Dims d;
};

template <bool REV>
__global__ void __launch_bounds__(256) m3_scan_local_kernel(const ScanArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.nc * d.NA) return;
  const int64_t a = i % d.NA, c = (i / d.NA) % d.nc, bh = i / (d.NA * d.nc), b = bh / d.H;
  const int64_t t0 = c * kL, t1 = t0 + kL < d.T ? t0 + kL : d.T;
  // U steps' loads are issued before their sums and stores (indexes past the
  // chunk clamped, their values unused): the stores may alias the loads (the
  // reverse scan runs in place), so the compiler would not move later loads
  // ahead of them and every step would wait for its own load
  constexpr int U = 16;
  float acc = 0.0f;
  if (!REV) {
    for (int64_t tb = t0; tb < t1; tb += U) {
      float vd[U], va[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = tb + u < t1 ? tb + u : t1 - 1;
        vd[u] = p.dt[bh * d.T + t];
        va[u] = p.ang[(b * d.T + t) * d.NA + a];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tb + u < t1) {
          acc = fmaf(vd[u], va[u], acc);
          p.out[(bh * d.T + tb + u) * d.NA + a] = acc;
        }
    }
  } else {
    for (int64_t tb = t1 - 1; tb >= t0; tb -= U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = p.src[(bh * d.T + (tb - u >= t0 ? tb - u : t0)) * d.NA + a];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tb - u >= t0) {
          acc += v[u];
          p.out[(bh * d.T + tb - u) * d.NA + a] = acc;
        }
    }
  }
  p.ctot[(bh * d.nc + c) * d.NA + a] = acc;
}

template <bool REV>
__global__ void __launch_bounds__(256) m3_scan_carry_kernel(const ScanArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.NA) return;
  const int64_t a = i % d.NA, bh = i / d.NA;
  // in place: U chunks' totals read before they are overwritten (as above)
  constexpr int U = 16;
  float run = 0.0f;
  for (int64_t k0 = 0; k0 < d.nc; k0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u < d.nc ? k0 + u : d.nc - 1;
      v[u] = p.ctot[(bh * d.nc + (REV ? d.nc - 1 - k : k)) * d.NA + a];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < d.nc) {
        p.ctot[(bh * d.nc + (REV ? d.nc - 1 - (k0 + u) : k0 + u)) * d.NA + a] = run;
        run += v[u];
      }
  }
}

// theta[b, h, t, a]: the chunk-local sum plus the sum of the chunks before
// (the scan's exclusive chunk totals), added where theta is read
__device__ __forceinline__ float theta_at(const float* theta, const float* ctot, const Dims& d, int64_t bh,
                                          int64_t t, int64_t a) {
  return theta[(bh * d.T + t) * d.NA + a] + ctot[(bh * d.nc + t / kL) * d.NA + a];
}

// From g = the chunk-local suffix sum plus the chunks after, per (b, h, t,
// angle): the angle gradient's per-head part g dt_t to `cang` [B, H, T, NA],
// and g angles_raw_t[a] in place of g; then per (b, h, t) the sum of the
// latter over the angles (the dt gradient through the angles) to `ddt_ang`.
struct ThetaBwdArgs {
  float* gl;
  const float *ctot, *dt, *ang;
  float *cang, *ddt_ang;
  Dims d;
};

__global__ void __launch_bounds__(256) m3_theta_contrib_kernel(const ThetaBwdArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T * d.NA) return;
  const int64_t a = i % d.NA, bht = i / d.NA, t = bht % d.T, bh = bht / d.T, b = bh / d.H;
  const float g = p.gl[i] + p.ctot[(bh * d.nc + t / kL) * d.NA + a];
  p.cang[i] = g * p.dt[bht];
  p.gl[i] = g * p.ang[(b * d.T + t) * d.NA + a];
}

__global__ void __launch_bounds__(256) m3_theta_dt_kernel(const ThetaBwdArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T) return;
  const float* g = p.gl + i * d.NA;
  constexpr int U = 16;   // loads issued before their adds; the adds keep the angle order
  float acc = 0.0f;
  for (int64_t a0 = 0; a0 < d.NA; a0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = g[a0 + u < d.NA ? a0 + u : d.NA - 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (a0 + u < d.NA) acc += v[u];
  }
  p.ddt_ang[i] = acc;
}

// Both of the above in one pass when NA is a power of two: the grid is (row
// tiles, B * H), so a (b, h, t) row's NA angles are NA aligned lanes of one
// wave, whose sum of g angles_raw_t[a] is a butterfly over those lanes (every
// lane of the row ends with the same bits; the first stores it).  g angles_raw
// itself is then not stored: nothing reads it after this sum.  A thread takes
// kThetaU elements 256 apart, all loads issued first, so that the
// butterflies of its rows overlap.
constexpr int kThetaU = 4;

__global__ void __launch_bounds__(256) m3_theta_grad_kernel(const ThetaBwdArgs p) {
  const Dims d = p.d;
  const uint32_t NA = static_cast<uint32_t>(d.NA), H = static_cast<uint32_t>(d.H), bh32 = blockIdx.y;
  const uint32_t n = static_cast<uint32_t>(d.T) * NA, sh = __builtin_ctz(NA);
  const int64_t bh = bh32, b = bh32 / H;
  // this (b, h)'s blocks; offsets within them are 32-bit (T * NA < 2^31)
  const float* gl = p.gl + bh * n;              // [T, NA]
  const float* ctot = p.ctot + bh * d.nc * NA;  // [nc, NA]
  const float* dtv = p.dt + bh * d.T;           // [T]
  const float* ang = p.ang + b * n;             // [T, NA] of batch row b
  float* cang = p.cang + bh * n;
  float vg[kThetaU], vc[kThetaU], vd[kThetaU], va[kThetaU];
#pragma unroll
  for (int u = 0; u < kThetaU; ++u) {
    // lanes past the last row (whole rows of them) re-read element 0, unused
    const uint32_t li = (blockIdx.x * kThetaU + u) * 256u + threadIdx.x;
    const uint32_t e = li < n ? li : 0, t = e >> sh;
    vg[u] = gl[e];
    vc[u] = ctot[((t / kL) << sh) + (e & (NA - 1))];
    vd[u] = dtv[t];
    va[u] = ang[e];
  }
  float v[kThetaU];
#pragma unroll
  for (int u = 0; u < kThetaU; ++u) {
    const uint32_t li = (blockIdx.x * kThetaU + u) * 256u + threadIdx.x;
    const float g = vg[u] + vc[u];
    if (li < n) cang[li] = g * vd[u];
    v[u] = li < n ? g * va[u] : 0.0f;
  }
  for (uint32_t off = NA >> 1; off > 0; off >>= 1) {
#pragma unroll
    for (int u = 0; u < kThetaU; ++u) v[u] += __shfl_xor(v[u], static_cast<int>(off), 64);
  }
#pragma unroll
  for (int u = 0; u < kThetaU; ++u) {
    const uint32_t li = (blockIdx.x * kThetaU + u) * 256u + threadIdx.x;
    if (li < n && (li & (NA - 1)) == 0) p.ddt_ang[bh * d.T + (li >> sh)] = v[u];
  }
}

// ---------------------------------------------------------------- rotate
// Qr / Kr [B, H, T, N] (activation dtype) = the biased C / B of the head's
// group, pairs (a, a + NA) turned by theta[a].  Thread per (b, h, t, j),
// j < N - NA: j < NA does the pair (j, j + NA), later j the dim j + NA.
struct RotArgs {
  const void *b_in, *c_in;
  const float *b_bias, *c_bias, *theta, *ctot;   // theta chunk-local, ctot the chunks before
  void *Kr, *Qr;
  Dims d;
};

template <Act A>
__global__ void __launch_bounds__(256) m3_rotate_kernel(const RotArgs p) {
  using io = IO<A>;
  const Dims d = p.d;
  const int64_t W = d.N - d.NA;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T * W) return;
  const int64_t j = i % W, bht = i / W, t = bht % d.T, bh = bht / d.T, h = bh % d.H, b = bh / d.H;
  const int64_t g = h / (d.H / d.G);
  const int64_t src = ((b * d.T + t) * d.G + g) * d.N;
  const int64_t dst = bht * d.N;
  if (j < d.NA) {
    const int64_t n1 = j, n2 = j + d.NA;
    const float th = theta_at(p.theta, p.ctot, d, bh, t, j);
    float s, c;
    __sincosf(th, &s, &c);
    const float k1 = io::ld(p.b_in, src + n1) + p.b_bias[h * d.N + n1];
    const float k2 = io::ld(p.b_in, src + n2) + p.b_bias[h * d.N + n2];
    const float q1 = io::ld(p.c_in, src + n1) + p.c_bias[h * d.N + n1];
    const float q2 = io::ld(p.c_in, src + n2) + p.c_bias[h * d.N + n2];
    io::st(p.Kr, dst + n1, k1 * c - k2 * s);
    io::st(p.Kr, dst + n2, k1 * s + k2 * c);
    io::st(p.Qr, dst + n1, q1 * c - q2 * s);
    io::st(p.Qr, dst + n2, q1 * s + q2 * c);
  } else {
    const int64_t n = j + d.NA;
    io::st(p.Kr, dst + n, io::ld(p.b_in, src + n) + p.b_bias[h * d.N + n]);
    io::st(p.Qr, dst + n, io::ld(p.c_in, src + n) + p.c_bias[h * d.N + n]);
  }
}

// The same for 16-bit activations and n_angles a multiple of 8.  The grid
// is (row tiles, B * H, 2): z = 0 turns pairs, NA / 8 threads per (b, h, t)
// row, each 8 pairs (dims a0 .. a0+7 with a0 + NA .. a0 + NA + 7), so each
// angle's sine and cosine is computed once; z = 1 copies the unturned dims
// past 2 NA, (N - 2 NA) / 8 threads per row, 8 dims each.  Every wave takes
// one branch, and (b, h) comes from the workgroup, so a thread's only
// division is the one that splits its row from its dims (32-bit).
template <Act A>
__global__ void __launch_bounds__(256) m3_rotate8_kernel(const RotArgs p) {
  using io = IO<A>;
  const Dims d = p.d;
  const bool turn = blockIdx.z == 0;   // uniform
  const uint32_t per = static_cast<uint32_t>(turn ? d.NA / 8 : (d.N - 2 * d.NA) / 8);
  const uint32_t li = blockIdx.x * 256u + threadIdx.x;
  if (li >= static_cast<uint32_t>(d.T) * per) return;
  const uint32_t H = static_cast<uint32_t>(d.H), bh32 = blockIdx.y;   // B * H < 2^16
  const uint32_t h = bh32 % H, g = h / (H / static_cast<uint32_t>(d.G));
  const int64_t bh = bh32, b = bh32 / H;
  const uint32_t t = li / per, j = li - t * per;
  const int64_t bht = bh * d.T + t;
  // this row's unturned B / C (16-bit), the head's biases, the output rows
  const uint16_t* bsrc = static_cast<const uint16_t*>(p.b_in) + ((b * d.T + t) * d.G + g) * d.N;
  const uint16_t* csrc = static_cast<const uint16_t*>(p.c_in) + ((b * d.T + t) * d.G + g) * d.N;
  const float* bb = p.b_bias + static_cast<int64_t>(h) * d.N;
  const float* cb = p.c_bias + static_cast<int64_t>(h) * d.N;
  uint16_t* kdst = static_cast<uint16_t*>(p.Kr) + bht * d.N;
  uint16_t* qdst = static_cast<uint16_t*>(p.Qr) + bht * d.N;
  auto ld8 = [](const uint16_t* q) { return *reinterpret_cast<const uint4*>(q); };
  auto ldf8 = [](const float* q, float4& lo, float4& hi) {
    lo = *reinterpret_cast<const float4*>(q);
    hi = *reinterpret_cast<const float4*>(q + 4);
  };
  // 8 raw 16-bit values (lower address in the low half) plus 8 biases
  auto unpack = [](const uint4& raw, const float4& lo, const float4& hi, float* v) {
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
    const float bv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = io::cvt(wv[k] & 0xffffu) + bv[2 * k];
      v[2 * k + 1] = io::cvt(wv[k] >> 16) + bv[2 * k + 1];
    }
  };
  auto put = [](uint16_t* q, const float* v) {   // 8 values as one 16-byte store
    uint16_t hv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (A == Act::BF16) hv[k] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[k]));
      else hv[k] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[k]));
    }
    uint4 o;
    o.x = hv[0] | (uint32_t(hv[1]) << 16);
    o.y = hv[2] | (uint32_t(hv[3]) << 16);
    o.z = hv[4] | (uint32_t(hv[5]) << 16);
    o.w = hv[6] | (uint32_t(hv[7]) << 16);
    *reinterpret_cast<uint4*>(q) = o;
  };
  float k1[8], q1[8];
  if (turn) {
    const int64_t d1 = 8 * static_cast<int64_t>(j), d2 = d1 + d.NA;   // the pairs' two halves
    // every load first: rows, biases, the chunk-local angles and the chunks before
    const uint4 rk1 = ld8(bsrc + d1), rq1 = ld8(csrc + d1), rk2 = ld8(bsrc + d2), rq2 = ld8(csrc + d2);
    float4 bk1l, bk1h, bq1l, bq1h, bk2l, bk2h, bq2l, bq2h, thl, thh, tcl, tch;
    ldf8(bb + d1, bk1l, bk1h);
    ldf8(cb + d1, bq1l, bq1h);
    ldf8(bb + d2, bk2l, bk2h);
    ldf8(cb + d2, bq2l, bq2h);
    ldf8(p.theta + bht * d.NA + d1, thl, thh);
    ldf8(p.ctot + (bh * d.nc + t / kL) * d.NA + d1, tcl, tch);
    __builtin_amdgcn_sched_barrier(0);
    float k2[8], q2[8], ko1[8], qo1[8], ko2[8], qo2[8];
    unpack(rk1, bk1l, bk1h, k1);
    unpack(rq1, bq1l, bq1h, q1);
    unpack(rk2, bk2l, bk2h, k2);
    unpack(rq2, bq2l, bq2h, q2);
    const float th[8] = {thl.x + tcl.x, thl.y + tcl.y, thl.z + tcl.z, thl.w + tcl.w,
                         thh.x + tch.x, thh.y + tch.y, thh.z + tch.z, thh.w + tch.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float sn, cs;
      __sincosf(th[k], &sn, &cs);
      // first half: x1 c - x2 s; second half: x1 s + x2 c
      ko1[k] = k1[k] * cs - k2[k] * sn;
      qo1[k] = q1[k] * cs - q2[k] * sn;
      ko2[k] = k1[k] * sn + k2[k] * cs;
      qo2[k] = q1[k] * sn + q2[k] * cs;
    }
    put(kdst + d1, ko1);
    put(qdst + d1, qo1);
    put(kdst + d2, ko2);
    put(qdst + d2, qo2);
  } else {
    const int64_t d1 = 2 * d.NA + 8 * static_cast<int64_t>(j);   // unturned dims
    const uint4 rk1 = ld8(bsrc + d1), rq1 = ld8(csrc + d1);
    float4 bk1l, bk1h, bq1l, bq1h;
    ldf8(bb + d1, bk1l, bk1h);
    ldf8(cb + d1, bq1l, bq1h);
    unpack(rk1, bk1l, bk1h, k1);
    unpack(rq1, bq1l, bq1h, q1);
    put(kdst + d1, k1);
    put(qdst + d1, q1);
  }
}

// ------------------------------------------------------- chunk state
// out[b, h, c] [P, N] f32 = sum_s w_s X_s Y_s^T over the chunk's steps:
//   forward  (BWD false): X = V (x), Y = Kr, w_s = e^{tot - cum_s} scale_s;
//   backward (BWD true) : X = dY,    Y = Qr, w_s = e^{cum_s};
// and each chunk's tot to `tot`.
struct ChunkStateArgs {
  const void *X, *Y;
  const float *da, *sc;
  float *out, *tot;
  Dims d;
};

// chunk step scalars for a 64-step chunk: lane s of wave 0 holds step c*64+s
struct ChunkScalars {
  float cum, tot;
  bool valid;
};

__device__ __forceinline__ ChunkScalars chunk_cum(const float* da_bh, int64_t t0, int64_t T, int lane) {
  ChunkScalars r;
  r.valid = t0 + lane < T;
  const float v = r.valid ? da_bh[t0 + lane] : 0.0f;
  r.cum = wave_incl_scan(v, lane);
  r.tot = __shfl(r.cum, 63, 64);
  return r;
}

template <Act A, int N, bool BWD>
__global__ void __launch_bounds__(kThreads) m3_chunk_state_kernel(const ChunkStateArgs p) {
  using io = IO<A>;
  constexpr int NQ = N / 16;                 // output dims per thread
  constexpr int XS = kP + 4, YS = N + 4;     // padded LDS rows
  __shared__ __attribute__((aligned(16))) float sX[kL * XS];
  __shared__ __attribute__((aligned(16))) float sY[kL * YS];
  __shared__ float sW[kL];
  const Dims d = p.d;
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  if (tid < 64) {
    const ChunkScalars s = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    float w = 0.0f;
    if (s.valid) w = BWD ? expf_fast(s.cum) : expf_fast(s.tot - s.cum) * p.sc[bh * d.T + t0 + tid];
    sW[tid] = w;
    if (tid == 0) p.tot[bh * d.nc + c] = s.tot;
  }
  __syncthreads();
  // X rows: 64 steps x 64 channels of this head; 16 values per thread
  {
    const int s = tid >> 2, p0 = (tid & 3) * 16;
    const bool ok = t0 + s < d.T;
    const int64_t base = ((b * d.T + t0 + s) * d.H + h) * kP + p0;
    const float w = sW[s];
#pragma unroll
    for (int k = 0; k < 16; ++k) sX[s * XS + p0 + k] = ok ? w * io::ld(p.X, base + k) : 0.0f;
  }
  // Y rows: 64 steps x N
  for (int e = tid; e < kL * N; e += kThreads) {
    const int s = e / N, n = e % N;
    sY[s * YS + n] = t0 + s < d.T ? io::ld(p.Y, (bh * d.T + t0 + s) * N + n) : 0.0f;
  }
  __syncthreads();
  const int p0 = (tid & 15) * 4, n0 = (tid >> 4) * NQ;
  float acc[4][NQ] = {};
  for (int s = 0; s < kL; ++s) {
    const float4 xv = *reinterpret_cast<const float4*>(&sX[s * XS + p0]);
    const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
    float ya[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) ya[j] = sY[s * YS + n0 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NQ; ++j) acc[i][j] = fmaf(xa[i], ya[j], acc[i][j]);
  }
  float* out = p.out + (bh * d.nc + c) * kP * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NQ; ++j) out[(p0 + i) * N + n0 + j] = acc[i][j];
}

// ------------------------------------------------------- state passing
// Per (b, h) and state element: forward, st[c] <- the state entering chunk c
// (st[c] held chunk c's own St_out); reverse, dst[c] <- the gradient of
// chunk c's St_out (dst[c] held chunk c's own sum_t e^{cum_t} dY_t Q_t^T).
struct PassArgs {
  float* st;
  const float* tot;
  Dims d;
};

template <bool REV>
__global__ void __launch_bounds__(256) m3_state_pass_kernel(const PassArgs p) {
  const Dims d = p.d;
  const int64_t PN = d.P * d.N;
  const int64_t per = PN / 256;   // workgroups per (b, h)
  const int64_t bh = blockIdx.x / per, e = (blockIdx.x % per) * 256 + threadIdx.x;
  float* st = p.st + bh * d.nc * PN + e;
  const float* tot = p.tot + bh * d.nc;
  // in place: U chunks' states read before they are overwritten (the
  // stores may alias the loads, so the compiler would not move later loads
  // ahead of them)
  constexpr int U = 8;
  float S = 0.0f;
  for (int64_t k0 = 0; k0 < d.nc; k0 += U) {
    float v[U], e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u < d.nc ? k0 + u : d.nc - 1;
      const int64_t c = REV ? d.nc - 1 - k : k;
      v[u] = st[c * PN];
      e[u] = tot[c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < d.nc) {
        const int64_t c = REV ? d.nc - 1 - (k0 + u) : k0 + u;
        st[c * PN] = S;
        S = fmaf(expf_fast(e[u]), S, v[u]);
      }
  }
}

// ---------------------------------------------------------- chunk output
struct OutArgs {
  const void *x, *Qr, *Kr;
  const float *da, *sc, *gam, *D, *st;
  void* y;
  Dims d;
};

// LDS rows of N floats are padded by 4 (float4 alignment, fewer bank conflicts)
template <int N>
struct OutLds {
  static constexpr int QS = N + 4, VS = kP + 4;
  float q[kL * QS];
  float k[kL * QS];      // K rows, then the entering state's rows [P][N]
  float v[kL * VS];
  float gmT[kL * VS];    // (G o M)^T: [s][t]
  float cum[kL], sc[kL], gam[kL], qk[kL];
};

template <Act A, int N>
__global__ void __launch_bounds__(kThreads) m3_chunk_out_kernel(const OutArgs p) {
  using io = IO<A>;
  using L = OutLds<N>;
  constexpr int QS = L::QS, VS = L::VS;
  __shared__ __attribute__((aligned(16))) L s;
  const Dims d = p.d;
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  if (tid < 64) {
    const ChunkScalars cs = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    s.cum[tid] = cs.cum;
    s.sc[tid] = cs.valid ? p.sc[bh * d.T + t0 + tid] : 0.0f;
    s.gam[tid] = cs.valid ? p.gam[bh * d.T + t0 + tid] : 0.0f;
  }
  for (int e = tid; e < kL * N; e += kThreads) {
    const int r = e / N, n = e % N;
    const bool ok = t0 + r < d.T;
    const int64_t gi = (bh * d.T + t0 + r) * N + n;
    s.q[r * QS + n] = ok ? io::ld(p.Qr, gi) : 0.0f;
    s.k[r * QS + n] = ok ? io::ld(p.Kr, gi) : 0.0f;
  }
  for (int e = tid; e < kL * kP; e += kThreads) {
    const int r = e / kP, q = e % kP;
    s.v[r * VS + q] = t0 + r < d.T ? io::ld(p.x, ((b * d.T + t0 + r) * d.H + h) * kP + q) : 0.0f;
  }
  __syncthreads();
  const int ti = (tid & 15) * 4, si = (tid >> 4) * 4;
  {  // G = Q K^T on a 4 x 4 tile, masked and stored transposed
    float g[4][4] = {};
    for (int n = 0; n < N; n += 4) {
      float4 qa[4], ka[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qa[i] = *reinterpret_cast<const float4*>(&s.q[(ti + i) * QS + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) ka[j] = *reinterpret_cast<const float4*>(&s.k[(si + j) * QS + n]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          g[i][j] = fmaf(qa[i].x, ka[j].x, fmaf(qa[i].y, ka[j].y, fmaf(qa[i].z, ka[j].z, fmaf(qa[i].w, ka[j].w, g[i][j]))));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = ti + i, r = si + j;
        const float m = r <= t ? expf_fast(s.cum[t] - s.cum[r]) * s.sc[r] : 0.0f;
        s.gmT[r * VS + t] = g[i][j] * m;
        if (r == t) s.qk[t] = g[i][j];
      }
  }
  __syncthreads();
  // the entering state [P][N] into the K rows
  const float* st = p.st + (bh * d.nc + c) * kP * N;
  for (int e = tid; e < kP * N; e += kThreads) s.k[(e / N) * QS + e % N] = st[e];
  __syncthreads();
  const int pi = (tid >> 4) * 4;
  float y[4][4] = {};
  for (int r = 0; r < kL; ++r) {
    const float4 gv = *reinterpret_cast<const float4*>(&s.gmT[r * VS + ti]);
    const float4 vv = *reinterpret_cast<const float4*>(&s.v[r * VS + pi]);
    const float ga[4] = {gv.x, gv.y, gv.z, gv.w}, va[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) y[i][j] = fmaf(ga[i], va[j], y[i][j]);
  }
  float z[4][4] = {};
  for (int n = 0; n < N; n += 4) {
    float4 qa[4], sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qa[i] = *reinterpret_cast<const float4*>(&s.q[(ti + i) * QS + n]);
#pragma unroll
    for (int j = 0; j < 4; ++j) sa[j] = *reinterpret_cast<const float4*>(&s.k[(pi + j) * QS + n]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        z[i][j] = fmaf(qa[i].x, sa[j].x, fmaf(qa[i].y, sa[j].y, fmaf(qa[i].z, sa[j].z, fmaf(qa[i].w, sa[j].w, z[i][j]))));
  }
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = ti + i;
    if (t0 + t >= d.T) continue;
    const float ec = expf_fast(s.cum[t]);
    const float dg = (s.gam[t] - s.sc[t]) * s.qk[t];
    const int64_t row = ((b * d.T + t0 + t) * d.H + h) * kP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float vt = s.v[t * VS + pi + j];
      io::st(p.y, row + pi + j, fmaf(ec, z[i][j], y[i][j]) + (dg + Dh) * vt);
    }
  }
}

// ---------------------------------------------------------- chunk backward
struct BwdArgs {
  const void *x, *dy, *Qr, *Kr;
  const float *da, *sc, *gam, *D, *st, *dst;
  void* d_x;
  float *dQ, *dK;                 // [B, H, T, N] f32, gradients of the turned Q, K
  float *d_da, *d_sc, *d_gam;     // [B, H, T]
  float* dD_part;                 // [B, H, nc]
  Dims d;
};

template <int N>
struct BwdLds {
  static constexpr int QS = N + 4, VS = kP + 4;
  static constexpr int NB = N < 64 ? N : 64;   // state columns per block of the inter-chunk terms
  static constexpr int BS = NB + 4;
  float q[kL * QS];
  float k[kL * QS];
  float v[kL * VS];
  float dy[kL * VS];
  // GM = G o M and DVM = DV o M, [t][s]; later one block of the entering
  // state and of the outgoing state's gradient, [p][n]
  float gm[kL * VS];
  float dvm[kL * VS];
  float part[3][16][kL];          // cross-thread partial sums
  float cum[kL], sc[kL], gam[kL], qk[kL], dvd[kL];
  float red[kThreads];
};

template <Act A, int N>
__global__ void __launch_bounds__(kThreads) m3_chunk_bwd_kernel(const BwdArgs p) {
  using io = IO<A>;
  using L = BwdLds<N>;
  constexpr int QS = L::QS, VS = L::VS, NB = L::NB, BS = L::BS;
  constexpr int NQ = N / 16;
  static_assert(kP * BS <= kL * VS, "a state block fits the GM / DVM area");
  __shared__ __attribute__((aligned(16))) L s;
  const Dims d = p.d;
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  float tot = 0.0f;
  if (tid < 64) {
    const ChunkScalars cs = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    s.cum[tid] = cs.cum;
    s.sc[tid] = cs.valid ? p.sc[bh * d.T + t0 + tid] : 0.0f;
    s.gam[tid] = cs.valid ? p.gam[bh * d.T + t0 + tid] : 0.0f;
    tot = cs.tot;
  }
  for (int e = tid; e < kL * N; e += kThreads) {
    const int r = e / N, n = e % N;
    const bool ok = t0 + r < d.T;
    const int64_t gi = (bh * d.T + t0 + r) * N + n;
    s.q[r * QS + n] = ok ? io::ld(p.Qr, gi) : 0.0f;
    s.k[r * QS + n] = ok ? io::ld(p.Kr, gi) : 0.0f;
  }
  for (int e = tid; e < kL * kP; e += kThreads) {
    const int r = e / kP, q = e % kP;
    const bool ok = t0 + r < d.T;
    const int64_t gi = ((b * d.T + t0 + r) * d.H + h) * kP + q;
    s.v[r * VS + q] = ok ? io::ld(p.x, gi) : 0.0f;
    s.dy[r * VS + q] = ok ? io::ld(p.dy, gi) : 0.0f;
  }
  __syncthreads();

  // ---- intra-chunk pair terms on a 4 x 4 tile: G = Q K^T, DV = dY V^T
  const int ti = (tid & 15) * 4, si = (tid >> 4) * 4;
  {
    float g[4][4] = {}, dv[4][4] = {};
    for (int n = 0; n < N; n += 4) {
      float4 qa[4], ka[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qa[i] = *reinterpret_cast<const float4*>(&s.q[(ti + i) * QS + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) ka[j] = *reinterpret_cast<const float4*>(&s.k[(si + j) * QS + n]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          g[i][j] = fmaf(qa[i].x, ka[j].x, fmaf(qa[i].y, ka[j].y, fmaf(qa[i].z, ka[j].z, fmaf(qa[i].w, ka[j].w, g[i][j]))));
    }
    for (int q = 0; q < kP; q += 4) {
      float4 ya[4], va[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ya[i] = *reinterpret_cast<const float4*>(&s.dy[(ti + i) * VS + q]);
#pragma unroll
      for (int j = 0; j < 4; ++j) va[j] = *reinterpret_cast<const float4*>(&s.v[(si + j) * VS + q]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dv[i][j] = fmaf(ya[i].x, va[j].x, fmaf(ya[i].y, va[j].y, fmaf(ya[i].z, va[j].z, fmaf(ya[i].w, va[j].w, dv[i][j]))));
    }
    // M[t][s] = e^{cum_t - cum_s} scale_s for s <= t; R = G o DV o M.
    // part[0]: row sums of R over the tile's s; part[1]: column sums of R
    // over its t; part[2]: column sums of G o DV o e^{cum_t - cum_s}.
    float rrow[4] = {}, rcol[4] = {}, ecol[4] = {};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = ti + i, r = si + j;
        const float e = r <= t ? expf_fast(s.cum[t] - s.cum[r]) : 0.0f;
        const float m = e * s.sc[r];
        s.gm[t * VS + r] = g[i][j] * m;
        s.dvm[t * VS + r] = dv[i][j] * m;
        const float gd = g[i][j] * dv[i][j];
        rrow[i] = fmaf(gd, m, rrow[i]);
        rcol[j] = fmaf(gd, m, rcol[j]);
        ecol[j] = fmaf(gd, e, ecol[j]);
        if (r == t) {
          s.qk[t] = g[i][j];
          s.dvd[t] = dv[i][j];
        }
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) s.part[0][tid >> 4][ti + i] = rrow[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s.part[1][tid & 15][si + j] = rcol[j];
      s.part[2][tid & 15][si + j] = ecol[j];
    }
  }
  __syncthreads();
  // per-step sums of the pair terms (lane r of wave 0), fixed order
  float dcum = 0.0f, dsc = 0.0f;
  if (tid < 64) {
    float rs = 0.0f, cs = 0.0f, es = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      rs += s.part[0][k][tid];
      cs += s.part[1][k][tid];
      es += s.part[2][k][tid];
    }
    dcum = rs - cs;
    dsc = es - s.qk[tid] * s.dvd[tid];
  }

  // ---- intra-chunk products
  // dV[s][p] += sum_t GM[t][s] dY[t][p]          (tile: s = ti.., p = si..)
  float dvs[4][4] = {};
  for (int t = 0; t < kL; ++t) {
    float ga[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ga[i] = s.gm[t * VS + ti + i];
    const float4 yv = *reinterpret_cast<const float4*>(&s.dy[t * VS + si]);
    const float ya[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dvs[i][j] = fmaf(ga[i], ya[j], dvs[i][j]);
  }
  // dQ[t][n] += sum_s DVM[t][s] K[s][n]; dK[s][n] += sum_t DVM[t][s] Q[t][n]
  // (tiles: 4 steps ti.., NQ state dims from nq)
  const int nq = (tid >> 4) * NQ;
  float dq[4][NQ] = {}, dk[4][NQ] = {};
  for (int r = 0; r < kL; ++r) {
    float kr[NQ], qr[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      kr[j] = s.k[r * QS + nq + j];
      qr[j] = s.q[r * QS + nq + j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = s.dvm[(ti + i) * VS + r];   // DVM[t][r], t = ti + i
      const float bq = s.dvm[r * VS + ti + i];    // DVM[r][s], s = ti + i
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        dq[i][j] = fmaf(a, kr[j], dq[i][j]);
        dk[i][j] = fmaf(bq, qr[j], dk[i][j]);
      }
    }
  }
  __syncthreads();   // GM / DVM are free from here

  // ---- inter-chunk terms, one block of NB state columns at a time:
  //   dQ[t][n] += e^{cum_t} sum_p dY[t][p] Sin[p][n]
  //   dK[s][n] += u_s sum_p V[s][p] dSout[p][n]        u_s = e^{tot - cum_s} scale_s
  //   dV[s][p] += u_s sum_n K[s][n] dSout[p][n]
  //   dcum_t  += e^{cum_t} Q_t . (dY_t Sin);  du_s = K_s . (V_s dSout)
  //   dtot    += <dSout, Sin> e^{tot}
  const float* stin = p.st + (bh * d.nc + c) * kP * N;
  const float* dsout = p.dst + (bh * d.nc + c) * kP * N;
  float* sin_b = s.gm;
  float* dso_b = s.dvm;
  float ecum[4], ucoef[4];
  __shared__ float s_tot;   // wave 0 holds tot; every wave needs it
  if (tid == 0) s_tot = tot;
  __syncthreads();
  const float totv = s_tot;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ecum[i] = expf_fast(s.cum[ti + i]);
    ucoef[i] = expf_fast(totv - s.cum[ti + i]) * s.sc[ti + i];
  }
  float wv[4][4] = {};       // sum_n K[s][n] dSout[p][n]   (s = ti.., p = si..)
  float dcq[4] = {}, dus[4] = {};
  float dtot_part = 0.0f;
  for (int nb = 0; nb < N; nb += NB) {
    for (int e = tid; e < kP * NB; e += kThreads) {
      const int q = e / NB, n = e % NB;
      sin_b[q * BS + n] = stin[q * N + nb + n];
      dso_b[q * BS + n] = dsout[q * N + nb + n];
      dtot_part = fmaf(stin[q * N + nb + n], dsout[q * N + nb + n], dtot_part);
    }
    __syncthreads();
    if (nq >= nb && nq < nb + NB) {
      const int nl = nq - nb;
      float zq[4][NQ] = {}, zk[4][NQ] = {};
      for (int q = 0; q < kP; ++q) {
        float sr[NQ], dr[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          sr[j] = sin_b[q * BS + nl + j];
          dr[j] = dso_b[q * BS + nl + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float yv = s.dy[(ti + i) * VS + q];
          const float vv = s.v[(ti + i) * VS + q];
#pragma unroll
          for (int j = 0; j < NQ; ++j) {
            zq[i][j] = fmaf(yv, sr[j], zq[i][j]);
            zk[i][j] = fmaf(vv, dr[j], zk[i][j]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          const float qz = ecum[i] * zq[i][j];
          dq[i][j] += qz;
          dcq[i] = fmaf(s.q[(ti + i) * QS + nq + j], qz, dcq[i]);
          dk[i][j] = fmaf(ucoef[i], zk[i][j], dk[i][j]);
          dus[i] = fmaf(s.k[(ti + i) * QS + nq + j], zk[i][j], dus[i]);
        }
    }
    for (int n = 0; n < NB; n += 4) {
      float4 ka[4], da4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const float4*>(&s.k[(ti + i) * QS + nb + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) da4[j] = *reinterpret_cast<const float4*>(&dso_b[(si + j) * BS + n]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wv[i][j] = fmaf(ka[i].x, da4[j].x, fmaf(ka[i].y, da4[j].y, fmaf(ka[i].z, da4[j].z, fmaf(ka[i].w, da4[j].w, wv[i][j]))));
    }
    __syncthreads();
  }
  // cross-thread sums of dcq and dus (per step, over the 16 state-dim groups)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s.part[0][tid >> 4][ti + i] = dcq[i];
    s.part[1][tid >> 4][ti + i] = dus[i];
  }
  s.red[tid] = dtot_part;
  __syncthreads();

  // ---- outputs of the tiles
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ti + i;
    if (t0 + r >= d.T) continue;
    const float dg = s.gam[r] - s.sc[r];
    const float dvr = s.dvd[r];
    const int64_t row = ((b * d.T + t0 + r) * d.H + h) * kP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float yv = s.dy[r * VS + si + j];
      const float gv = fmaf(ucoef[i], wv[i][j], dvs[i][j]) + (dg * s.qk[r] + Dh) * yv;
      io::st(p.d_x, row + si + j, gv);
    }
    const int64_t qrow = (bh * d.T + t0 + r) * N + nq;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      p.dQ[qrow + j] = fmaf(dg * dvr, s.k[r * QS + nq + j], dq[i][j]);
      p.dK[qrow + j] = fmaf(dg * dvr, s.q[r * QS + nq + j], dk[i][j]);
    }
  }
  // ---- per-step scalars (wave 0, lane = step)
  if (tid < 64) {
    float cq = 0.0f, us = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      cq += s.part[0][k][tid];
      us += s.part[1][k][tid];
    }
    float dsum = 0.0f;
    for (int k = 0; k < kThreads; k += 64) dsum += s.red[k + tid];
    const float dotSS = wave_sum(dsum);
    const float u = expf_fast(tot - s.cum[tid]) * s.sc[tid];
    const float dcum_t = dcum + cq - u * us;
    const float dsc_t = dsc + expf_fast(tot - s.cum[tid]) * us;
    const float dtot = wave_sum(u * us) + expf_fast(tot) * dotSS;
    const float dda = wave_suffix_scan(dcum_t, tid) + dtot;
    const bool ok = t0 + tid < d.T;
    if (ok) {
      const int64_t i = bh * d.T + t0 + tid;
      p.d_da[i] = dda;
      p.d_sc[i] = dsc_t;
      p.d_gam[i] = s.qk[tid] * s.dvd[tid];
    }
    const float dD = wave_sum(ok ? s.dvd[tid] : 0.0f);
    if (tid == 0) p.dD_part[bh * d.nc + c] = dD;
  }
}

// ------------------------------------------------------- rotation adjoint
// Per (b, h, t, angle): the gradients of the unturned (biased) B / C, in place
// over dK / dQ, and the angle gradient dtheta [B, H, T, NA].
struct RotBwdArgs {
  const void *Qr, *Kr;
  const float *theta, *ctot;   // theta chunk-local, ctot the chunks before
  float *dQ, *dK, *dtheta;
  Dims d;
};

template <Act A>
__global__ void __launch_bounds__(256) m3_rot_bwd_kernel(const RotBwdArgs p) {
  using io = IO<A>;
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T * d.NA) return;   // unturned dims: the gradient passes through
  const int64_t j = i % d.NA, bht = i / d.NA;
  const int64_t base = bht * d.N, n1 = j, n2 = j + d.NA;
  float s, c;
  __sincosf(theta_at(p.theta, p.ctot, d, bht / d.T, bht % d.T, j), &s, &c);
  const float gq1 = p.dQ[base + n1], gq2 = p.dQ[base + n2];
  const float gk1 = p.dK[base + n1], gk2 = p.dK[base + n2];
  const float q1 = io::ld(p.Qr, base + n1), q2 = io::ld(p.Qr, base + n2);
  const float k1 = io::ld(p.Kr, base + n1), k2 = io::ld(p.Kr, base + n2);
  p.dtheta[bht * d.NA + j] = (gq2 * q1 - gq1 * q2) + (gk2 * k1 - gk1 * k2);
  p.dQ[base + n1] = c * gq1 + s * gq2;
  p.dQ[base + n2] = c * gq2 - s * gq1;
  p.dK[base + n1] = c * gk1 + s * gk2;
  p.dK[base + n2] = c * gk2 - s * gk1;
}

// ------------------------------------------------------- scalar adjoint
// Per (b, h, t): from the gradients of dt*A, gamma, scale and the angle
// part of dt, the gradients of dd_dt_raw, dd_a_raw, trap_raw ([B, T, H]).
struct ScalarBwdArgs {
  const float *dd_dt, *dd_a, *trap, *dt_bias;
  const float *d_da, *d_sc, *d_gam, *ddt_ang;
  float *g_dd_dt, *g_dd_a, *g_trap;
  Dims d;
};

__global__ void __launch_bounds__(256) m3_scalar_bwd_kernel(const ScalarBwdArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.H * d.T) return;
  const int64_t t = i % d.T, bh = i / d.T, h = bh % d.H, b = bh / d.H;
  const int64_t in = (b * d.T + t) * d.H + h;
  const float x = p.dd_dt[in] + p.dt_bias[h];
  const float dt = mscan::softplus(x);
  const float sa = mscan::softplus(p.dd_a[in]);
  const float A = -fmaxf(sa, d.a_floor);
  const float lam = mscan::sigmoid(p.trap[in]);
  const float dsc = p.d_sc[i], dsc_prev = t > 0 ? p.d_sc[i - 1] : 0.0f;
  const float dgam = p.d_gam[i], dda = p.d_da[i];
  // scale_t = lam_t dt_t + (1 - lam_{t+1}) dt_{t+1}; gamma_t = lam_t dt_t
  const float g_dt = dda * A + (dgam + dsc) * lam + dsc_prev * (1.0f - lam) + p.ddt_ang[i];
  const float g_A = dda * dt;
  const float g_lam = (dgam + dsc - dsc_prev) * dt;
  p.g_dd_dt[in] = g_dt * mscan::sigmoid(x);
  p.g_dd_a[in] = sa > d.a_floor ? -g_A * mscan::sigmoid(p.dd_a[in]) : 0.0f;
  p.g_trap[in] = g_lam * lam * (1.0f - lam);
}

// ------------------------------------------------------- fixed-order sums
// d_b_in / d_c_in [B, T, G, N] = sum over the group's heads of dK / dQ.
struct GroupArgs {
  const float *dK, *dQ;
  void *d_b, *d_c;
  Dims d;
};

template <Act A>
__global__ void __launch_bounds__(256) m3_group_sum_kernel(const GroupArgs p) {
  using io = IO<A>;
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.T * d.G * d.N) return;
  const int64_t n = i % d.N, btg = i / d.N, g = btg % d.G, bt = btg / d.G, t = bt % d.T, b = bt / d.T;
  const int64_t hpg = d.H / d.G;
  // heads in batches of U, every load of a batch issued before its adds
  // (heads past the group clamped, their values unused); the adds keep the
  // head order
  constexpr int U = 8;
  float sk = 0.0f, sq = 0.0f;
  for (int64_t k0 = 0; k0 < hpg; k0 += U) {
    float vk[U], vq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u < hpg ? k0 + u : hpg - 1;
      const int64_t e = ((b * d.H + g * hpg + k) * d.T + t) * d.N + n;
      vk[u] = p.dK[e];
      vq[u] = p.dQ[e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < hpg) {
        sk += vk[u];
        sq += vq[u];
      }
  }
  io::st(p.d_b, i, sk);
  io::st(p.d_c, i, sq);
}

// Column sums over the (b, t) rows of [B, H, T, W] arrays (W = N for the
// B / C bias gradients; the dt-bias gradient [B, T, H] is read as one head
// of B * T rows and W = H columns):
// partial sums over RB row blocks, then a fixed-order sum += into out[h, w].
constexpr int kRowBlocks = 128;

struct ColArgs {
  const float* src;
  float* part;   // [kRowBlocks, H, W]
  float* out;    // [H, W], +=
  int64_t B, H, T, W;
};

// The four bias sums (B, C, dt, D) are independent, so each pass runs them
// as one launch: grid y = the job.
constexpr int kColJobs = 4;

struct ColJobs {
  ColArgs job[kColJobs];
};

__global__ void __launch_bounds__(256) m3_colpart_kernel(const ColJobs jobs) {
  const ColArgs& p = jobs.job[blockIdx.y];
  const int64_t HW = p.H * p.W;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= kRowBlocks * HW) return;
  const int64_t hw = i % HW, rb = i / HW, h = hw / p.W, w = hw % p.W;
  const int64_t rows = p.B * p.T, per = (rows + kRowBlocks - 1) / kRowBlocks;
  const int64_t r0 = rb * per, r1 = r0 + per < rows ? r0 + per : rows;
  float acc = 0.0f;
  int64_t r = r0;
  // row r = (b, t), stepped without a division per row
  int64_t b = r0 / p.T, t = r0 % p.T;
  constexpr int U = 16;   // rows whose loads are issued before their adds
  for (; r + U <= r1; r += U) {
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      v[k] = p.src[((b * p.H + h) * p.T + t) * p.W + w];
      if (++t == p.T) {
        t = 0;
        ++b;
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  for (; r < r1; ++r) {
    acc += p.src[((b * p.H + h) * p.T + t) * p.W + w];
    if (++t == p.T) {
      t = 0;
      ++b;
    }
  }
  p.part[i] = acc;
}

__global__ void __launch_bounds__(256) m3_colsum_kernel(const ColJobs jobs) {
  const ColArgs& p = jobs.job[blockIdx.y];
  const int64_t HW = p.H * p.W;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= HW) return;
  constexpr int U = 16;   // partials whose loads are issued before their adds (in order)
  static_assert(kRowBlocks % U == 0, "partial batches");
  float acc = 0.0f;
  for (int r0 = 0; r0 < kRowBlocks; r0 += U) {
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = p.part[(r0 + k) * HW + i];
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  p.out[i] += acc;
}

// d_angles_raw [B, T, NA] = sum over heads of cang [B, H, T, NA] (overwrite);
// d_dt_bias and d_D use the column sums above.
struct AngArgs {
  const float* cang;
  float* d_ang;
  Dims d;
};

__global__ void __launch_bounds__(256) m3_angle_sum_kernel(const AngArgs p) {
  const Dims d = p.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d.B * d.T * d.NA) return;
  const int64_t a = i % d.NA, bt = i / d.NA, t = bt % d.T, b = bt / d.T;
  constexpr int U = 8;   // heads' loads issued before their adds; the adds keep the head order
  float acc = 0.0f;
  for (int64_t h0 = 0; h0 < d.H; h0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p.cang[((b * d.H + (h0 + u < d.H ? h0 + u : d.H - 1)) * d.T + t) * d.NA + a];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (h0 + u < d.H) acc += v[u];
  }
  p.d_ang[i] = acc;
}

__global__ void __launch_bounds__(256) m3_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace m3

#include "m3_mfma.h"

namespace m3 {

// ================================================================ host side

unsigned blocks(int64_t n, int per = 256) { return static_cast<unsigned>((n + per - 1) / per); }

template <int N>
hipError_t launch_chunk_kernels_fwd(Act act, const ChunkStateArgs& cs, const OutArgs* o, unsigned grid,
                                    hipStream_t st) {
  switch (act) {
    case Act::F32:
      if (o) hipLaunchKernelGGL((m3_chunk_out_kernel<Act::F32, N>), dim3(grid), dim3(kThreads), 0, st, *o);
      else hipLaunchKernelGGL((m3_chunk_state_kernel<Act::F32, N, false>), dim3(grid), dim3(kThreads), 0, st, cs);
      break;
    case Act::BF16:   // matrix cores
      if (o) hipLaunchKernelGGL((m3_chunk_out_mfma<N>), dim3(grid), dim3(kThreads), 0, st, *o);
      else hipLaunchKernelGGL((m3_chunk_state_mfma<N, false>), dim3(grid), dim3(kThreads), 0, st, cs);
      break;
    case Act::F16:
      if (o) hipLaunchKernelGGL((m3_chunk_out_kernel<Act::F16, N>), dim3(grid), dim3(kThreads), 0, st, *o);
      else hipLaunchKernelGGL((m3_chunk_state_kernel<Act::F16, N, false>), dim3(grid), dim3(kThreads), 0, st, cs);
      break;
  }
  return hipGetLastError();
}

template <int N>
hipError_t launch_chunk_kernels_bwd(Act act, const ChunkStateArgs* cs, const BwdArgs* bw, unsigned grid,
                                    hipStream_t st) {
  switch (act) {
    case Act::F32:
      if (bw) hipLaunchKernelGGL((m3_chunk_bwd_kernel<Act::F32, N>), dim3(grid), dim3(kThreads), 0, st, *bw);
      else hipLaunchKernelGGL((m3_chunk_state_kernel<Act::F32, N, true>), dim3(grid), dim3(kThreads), 0, st, *cs);
      break;
    case Act::BF16:   // matrix cores
      if (bw) hipLaunchKernelGGL((m3_chunk_bwd_mfma<N>), dim3(grid), dim3(kThreadsB), 0, st, *bw);
      else hipLaunchKernelGGL((m3_chunk_state_mfma<N, true>), dim3(grid), dim3(kThreads), 0, st, *cs);
      break;
    case Act::F16:
      if (bw) hipLaunchKernelGGL((m3_chunk_bwd_kernel<Act::F16, N>), dim3(grid), dim3(kThreads), 0, st, *bw);
      else hipLaunchKernelGGL((m3_chunk_state_kernel<Act::F16, N, true>), dim3(grid), dim3(kThreads), 0, st, *cs);
      break;
  }
  return hipGetLastError();
}

hipError_t chunk_fwd(int64_t N, Act act, const ChunkStateArgs& cs, const OutArgs* o, unsigned grid, hipStream_t st) {
  switch (N) {
    case 32: return launch_chunk_kernels_fwd<32>(act, cs, o, grid, st);
    case 64: return launch_chunk_kernels_fwd<64>(act, cs, o, grid, st);
    case 128: return launch_chunk_kernels_fwd<128>(act, cs, o, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t chunk_bwd(int64_t N, Act act, const ChunkStateArgs* cs, const BwdArgs* bw, unsigned grid, hipStream_t st) {
  switch (N) {
    case 32: return launch_chunk_kernels_bwd<32>(act, cs, bw, grid, st);
    case 64: return launch_chunk_kernels_bwd<64>(act, cs, bw, grid, st);
    case 128: return launch_chunk_kernels_bwd<128>(act, cs, bw, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rotate(Act act, const RotArgs& a, unsigned grid, hipStream_t st) {
  const Dims& d = a.d;
  // the 8-wide kernel: (b, h) on the grid's y, a row's dims in 32-bit indexes
  const int64_t per = d.NA / 8 > (d.N - 2 * d.NA) / 8 ? d.NA / 8 : (d.N - 2 * d.NA) / 8;
  if (act != Act::F32 && d.NA % 8 == 0 && d.B * d.H <= 65535 && d.T * per < (int64_t(1) << 31)) {
    const dim3 g8(blocks(d.T * per), static_cast<unsigned>(d.B * d.H), 2);
    if (act == Act::BF16) hipLaunchKernelGGL(m3_rotate8_kernel<Act::BF16>, g8, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(m3_rotate8_kernel<Act::F16>, g8, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  switch (act) {
    case Act::F32: hipLaunchKernelGGL(m3_rotate_kernel<Act::F32>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::BF16: hipLaunchKernelGGL(m3_rotate_kernel<Act::BF16>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::F16: hipLaunchKernelGGL(m3_rotate_kernel<Act::F16>, dim3(grid), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_rot_bwd(Act act, const RotBwdArgs& a, unsigned grid, hipStream_t st) {
  switch (act) {
    case Act::F32: hipLaunchKernelGGL(m3_rot_bwd_kernel<Act::F32>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::BF16: hipLaunchKernelGGL(m3_rot_bwd_kernel<Act::BF16>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::F16: hipLaunchKernelGGL(m3_rot_bwd_kernel<Act::F16>, dim3(grid), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_group_sum(Act act, const GroupArgs& a, unsigned grid, hipStream_t st) {
  switch (act) {
    case Act::F32: hipLaunchKernelGGL(m3_group_sum_kernel<Act::F32>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::BF16: hipLaunchKernelGGL(m3_group_sum_kernel<Act::BF16>, dim3(grid), dim3(256), 0, st, a); break;
    case Act::F16: hipLaunchKernelGGL(m3_group_sum_kernel<Act::F16>, dim3(grid), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

thread_local const char* g_fn = "";

int fail(int code, const std::string& msg) {
  mscan::set_last_error(std::string(g_fn) + ": " + msg);
  return code;
}

int check_dims(const mamba3_dims_t* dd, Dims* out, Act* act) {
  if (!dd) return fail(MAMBA_ERR_INVALID, "dims is NULL");
  if (dd->batch < 1 || dd->seqlen < 1 || dd->heads < 1 || dd->groups < 1)
    return fail(MAMBA_ERR_INVALID, "batch, seqlen, heads and groups must be >= 1");
  if (dd->heads % dd->groups != 0) return fail(MAMBA_ERR_INVALID, "heads must be a multiple of groups");
  if (dd->act < 0 || dd->act > 2) return fail(MAMBA_ERR_INVALID, "act is not a mamba_dtype_t");
  if (dd->headdim != kP) return fail(MAMBA_ERR_UNSUPPORTED, "headdim must be 64");
  if (dd->d_state != 32 && dd->d_state != 64 && dd->d_state != 128)
    return fail(MAMBA_ERR_UNSUPPORTED, "d_state must be 32, 64 or 128");
  if (dd->act == MAMBA_F32 && dd->d_state > 64)
    return fail(MAMBA_ERR_UNSUPPORTED, "f32 activations take d_state 32 or 64");
  if (dd->n_angles < 0 || 2 * dd->n_angles > dd->d_state)
    return fail(MAMBA_ERR_INVALID, "n_angles must be in [0, d_state / 2]");
  if (dd->n_angles > 64) return fail(MAMBA_ERR_UNSUPPORTED, "n_angles must be <= 64");
  if (dd->chunk != 0 && dd->chunk != kL) return fail(MAMBA_ERR_UNSUPPORTED, "chunk must be 0 or 64");
  if (!(dd->a_floor >= 0.0f) || dd->a_floor > 3.0e38f) return fail(MAMBA_ERR_INVALID, "a_floor must be finite and >= 0");
  // every index stays well inside int64; launch sizes inside 2^32 workgroups
  const int64_t rows = dd->batch * dd->seqlen;
  if (dd->seqlen > (int64_t(1) << 31) || dd->batch > 65535 || dd->heads > 65535 || rows > (int64_t(1) << 31))
    return fail(MAMBA_ERR_CAPACITY, "batch * seqlen must be < 2^31 (batch, heads <= 65535)");
  const int64_t nc = (dd->seqlen + kL - 1) / kL;
  const int64_t maxel = rows * dd->heads * dd->d_state;
  if (maxel > (int64_t(1) << 40) || dd->batch * dd->heads * nc > (int64_t(1) << 31))
    return fail(MAMBA_ERR_CAPACITY, "batch * seqlen * heads * d_state exceeds 2^40");
  out->B = dd->batch;
  out->T = dd->seqlen;
  out->H = dd->heads;
  out->P = kP;
  out->N = dd->d_state;
  out->G = dd->groups;
  out->NA = dd->n_angles;
  out->nc = nc;
  out->a_floor = dd->a_floor;
  *act = static_cast<Act>(dd->act);
  return MAMBA_OK;
}

size_t al(size_t v) { return (v + 255) / 256 * 256; }

// workspace: [dt | da | gam | sc : B*H*T f32 each] [tot : B*H*nc] [theta : B*H*T*NA] [atot : B*H*nc*NA]
//            [Qr | Kr : B*H*T*N act]   -- forward and backward
//            [dst : B*H*nc*P*N] [dQ | dK : B*H*T*N f32] [d_da | d_sc | d_gam | ddt_ang : B*H*T]
//            [dtheta | cang : B*H*T*NA] [dD_part : B*H*nc] [colpart : kRowBlocks*H*(2N+2)]   -- backward
struct Ws {
  float *dt, *da, *gam, *sc, *tot, *theta, *atot;
  void *Qr, *Kr;
  float *dst, *dQ, *dK, *d_da, *d_sc, *d_gam, *ddt_ang, *dtheta, *cang, *dD_part, *colpart;
  size_t fwd_bytes, bwd_bytes;
};

Ws layout(const Dims& d, Act act, char* base) {
  Ws w{};
  const size_t f = 4, es = act == Act::F32 ? 4 : 2;
  const size_t bht = d.B * d.H * d.T, bhc = d.B * d.H * d.nc;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  };
  w.dt = reinterpret_cast<float*>(take(bht * f));
  w.da = reinterpret_cast<float*>(take(bht * f));
  w.gam = reinterpret_cast<float*>(take(bht * f));
  w.sc = reinterpret_cast<float*>(take(bht * f));
  w.tot = reinterpret_cast<float*>(take(bhc * f));
  w.theta = reinterpret_cast<float*>(take(bht * d.NA * f + f));
  w.atot = reinterpret_cast<float*>(take(bhc * d.NA * f + f));
  w.Qr = take(bht * d.N * es);
  w.Kr = take(bht * d.N * es);
  w.fwd_bytes = off;
  w.dst = reinterpret_cast<float*>(take(bhc * d.P * d.N * f));
  w.dQ = reinterpret_cast<float*>(take(bht * d.N * f));
  w.dK = reinterpret_cast<float*>(take(bht * d.N * f));
  w.d_da = reinterpret_cast<float*>(take(bht * f));
  w.d_sc = reinterpret_cast<float*>(take(bht * f));
  w.d_gam = reinterpret_cast<float*>(take(bht * f));
  w.ddt_ang = reinterpret_cast<float*>(take(bht * f));
  w.dtheta = reinterpret_cast<float*>(take(bht * d.NA * f + f));
  w.cang = reinterpret_cast<float*>(take(bht * d.NA * f + f));
  w.dD_part = reinterpret_cast<float*>(take(bhc * f));
  w.colpart = reinterpret_cast<float*>(take(size_t(kRowBlocks) * d.H * (2 * d.N + 2) * f));
  w.bwd_bytes = off;
  return w;
}

#define M3_HIP(expr)                                                                          \
  do {                                                                                        \
    const hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(MAMBA_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

int check_ptr(const char* name, const void* p, bool need, int align) {
  if (!p) return need ? fail(MAMBA_ERR_INVALID, std::string(name) + " is NULL") : MAMBA_OK;
  if (reinterpret_cast<uintptr_t>(p) % align)
    return fail(MAMBA_ERR_INVALID, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return MAMBA_OK;
}

#define M3_TRY(expr)                  \
  do {                                \
    const int rc_ = (expr);           \
    if (rc_ != MAMBA_OK) return rc_;  \
  } while (0)

// the forward's first three passes (shared by the backward): per-step
// scalars, angle sums, turned Q and K
int prep(const Dims& d, Act act, const Ws& w, const void* b_in, const void* c_in, const float* dd_dt,
         const float* dd_a, const float* trap, const float* ang, const float* b_bias, const float* c_bias,
         const float* dt_bias, hipStream_t st) {
  const int64_t bht = d.B * d.H * d.T;
  PrepArgs pa{dd_dt, dd_a, trap, dt_bias, w.dt, w.da, w.gam, w.sc, d};
  hipLaunchKernelGGL(m3_prep_kernel, dim3(blocks(bht)), dim3(256), 0, st, pa);
  M3_HIP(hipGetLastError());
  if (d.NA > 0) {
    ScanArgs sa{w.dt, ang, nullptr, w.theta, w.atot, d};
    hipLaunchKernelGGL(m3_scan_local_kernel<false>, dim3(blocks(d.B * d.H * d.nc * d.NA)), dim3(256), 0, st, sa);
    hipLaunchKernelGGL(m3_scan_carry_kernel<false>, dim3(blocks(d.B * d.H * d.NA)), dim3(256), 0, st, sa);
    M3_HIP(hipGetLastError());
  }
  RotArgs ra{b_in, c_in, b_bias, c_bias, w.theta, w.atot, w.Kr, w.Qr, d};
  M3_HIP(launch_rotate(act, ra, blocks(bht * (d.N - d.NA)), st));
  return MAMBA_OK;
}

}  // namespace m3

using namespace m3;

extern "C" {

int mamba3_states_bytes(const mamba3_dims_t* dims, size_t* bytes) {
  g_fn = "mamba3_states_bytes";
  Dims d;
  Act act;
  M3_TRY(check_dims(dims, &d, &act));
  if (!bytes) return fail(MAMBA_ERR_INVALID, "bytes is NULL");
  *bytes = static_cast<size_t>(d.B * d.H * d.nc * d.P * d.N) * sizeof(float);
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba3_workspace_bytes(const mamba3_dims_t* dims, size_t* bytes) {
  g_fn = "mamba3_workspace_bytes";
  Dims d;
  Act act;
  M3_TRY(check_dims(dims, &d, &act));
  if (!bytes) return fail(MAMBA_ERR_INVALID, "bytes is NULL");
  *bytes = layout(d, act, nullptr).bwd_bytes;
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba3_siso_fwd(const mamba3_dims_t* dims, const void* x, const void* b_in, const void* c_in,
                    const float* dd_dt_raw, const float* dd_a_raw, const float* trap_raw, const float* angles_raw,
                    const float* b_bias, const float* c_bias, const float* dt_bias, const float* D, void* y,
                    float* states, void* workspace, size_t workspace_bytes, void* stream) {
  g_fn = "mamba3_siso_fwd";
  Dims d;
  Act act;
  M3_TRY(check_dims(dims, &d, &act));
  M3_TRY(check_ptr("x", x, true, 16));
  M3_TRY(check_ptr("b_in", b_in, true, 16));
  M3_TRY(check_ptr("c_in", c_in, true, 16));
  M3_TRY(check_ptr("dd_dt_raw", dd_dt_raw, true, 4));
  M3_TRY(check_ptr("dd_a_raw", dd_a_raw, true, 4));
  M3_TRY(check_ptr("trap_raw", trap_raw, true, 4));
  M3_TRY(check_ptr("angles_raw", angles_raw, d.NA > 0, 4));
  M3_TRY(check_ptr("b_bias", b_bias, true, 4));
  M3_TRY(check_ptr("c_bias", c_bias, true, 4));
  M3_TRY(check_ptr("dt_bias", dt_bias, true, 4));
  M3_TRY(check_ptr("D", D, false, 4));
  M3_TRY(check_ptr("y", y, true, 16));
  M3_TRY(check_ptr("states", states, true, 16));
  M3_TRY(check_ptr("workspace", workspace, true, 256));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const Ws w = layout(d, act, static_cast<char*>(workspace));
  if (workspace_bytes < w.fwd_bytes)
    return fail(MAMBA_ERR_CAPACITY, "workspace_bytes " + std::to_string(workspace_bytes) + " < " +
                                        std::to_string(w.fwd_bytes) + " needed");
  M3_TRY(prep(d, act, w, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, st));
  const unsigned grid = static_cast<unsigned>(d.B * d.H * d.nc);
  ChunkStateArgs cs{x, w.Kr, w.da, w.sc, states, w.tot, d};
  M3_HIP(chunk_fwd(d.N, act, cs, nullptr, grid, st));
  PassArgs pa{states, w.tot, d};
  hipLaunchKernelGGL(m3_state_pass_kernel<false>, dim3(static_cast<unsigned>(d.B * d.H * (d.P * d.N / 256))),
                     dim3(256), 0, st, pa);
  M3_HIP(hipGetLastError());
  OutArgs oa{x, w.Qr, w.Kr, w.da, w.sc, w.gam, D, states, y, d};
  M3_HIP(chunk_fwd(d.N, act, cs, &oa, grid, st));
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba3_siso_bwd(const mamba3_dims_t* dims, const void* x, const void* b_in, const void* c_in,
                    const float* dd_dt_raw, const float* dd_a_raw, const float* trap_raw, const float* angles_raw,
                    const float* b_bias, const float* c_bias, const float* dt_bias, const float* D,
                    const float* states, const void* dy, void* d_x, void* d_b_in, void* d_c_in, float* d_dd_dt_raw,
                    float* d_dd_a_raw, float* d_trap_raw, float* d_angles_raw, float* d_b_bias, float* d_c_bias,
                    float* d_dt_bias, float* d_D, void* workspace, size_t workspace_bytes, void* stream) {
  g_fn = "mamba3_siso_bwd";
  Dims d;
  Act act;
  M3_TRY(check_dims(dims, &d, &act));
  M3_TRY(check_ptr("x", x, true, 16));
  M3_TRY(check_ptr("b_in", b_in, true, 16));
  M3_TRY(check_ptr("c_in", c_in, true, 16));
  M3_TRY(check_ptr("dd_dt_raw", dd_dt_raw, true, 4));
  M3_TRY(check_ptr("dd_a_raw", dd_a_raw, true, 4));
  M3_TRY(check_ptr("trap_raw", trap_raw, true, 4));
  M3_TRY(check_ptr("angles_raw", angles_raw, d.NA > 0, 4));
  M3_TRY(check_ptr("b_bias", b_bias, true, 4));
  M3_TRY(check_ptr("c_bias", c_bias, true, 4));
  M3_TRY(check_ptr("dt_bias", dt_bias, true, 4));
  M3_TRY(check_ptr("D", D, false, 4));
  M3_TRY(check_ptr("states", states, true, 16));
  M3_TRY(check_ptr("dy", dy, true, 16));
  M3_TRY(check_ptr("d_x", d_x, true, 16));
  M3_TRY(check_ptr("d_b_in", d_b_in, true, 16));
  M3_TRY(check_ptr("d_c_in", d_c_in, true, 16));
  M3_TRY(check_ptr("d_dd_dt_raw", d_dd_dt_raw, true, 4));
  M3_TRY(check_ptr("d_dd_a_raw", d_dd_a_raw, true, 4));
  M3_TRY(check_ptr("d_trap_raw", d_trap_raw, true, 4));
  M3_TRY(check_ptr("d_angles_raw", d_angles_raw, d.NA > 0, 4));
  M3_TRY(check_ptr("d_b_bias", d_b_bias, true, 4));
  M3_TRY(check_ptr("d_c_bias", d_c_bias, true, 4));
  M3_TRY(check_ptr("d_dt_bias", d_dt_bias, true, 4));
  M3_TRY(check_ptr("d_D", d_D, D != nullptr, 4));
  M3_TRY(check_ptr("workspace", workspace, true, 256));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const Ws w = layout(d, act, static_cast<char*>(workspace));
  if (workspace_bytes < w.bwd_bytes)
    return fail(MAMBA_ERR_CAPACITY, "workspace_bytes " + std::to_string(workspace_bytes) + " < " +
                                        std::to_string(w.bwd_bytes) + " needed");
  M3_TRY(prep(d, act, w, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, st));
  const int64_t bht = d.B * d.H * d.T;
  const unsigned grid = static_cast<unsigned>(d.B * d.H * d.nc);
  // each chunk's own sum_t e^{cum_t} dY_t Q_t^T, then the reverse pass
  ChunkStateArgs cs{dy, w.Qr, w.da, w.sc, w.dst, w.tot, d};
  M3_HIP(chunk_bwd(d.N, act, &cs, nullptr, grid, st));
  PassArgs pa{w.dst, w.tot, d};
  hipLaunchKernelGGL(m3_state_pass_kernel<true>, dim3(static_cast<unsigned>(d.B * d.H * (d.P * d.N / 256))),
                     dim3(256), 0, st, pa);
  M3_HIP(hipGetLastError());
  BwdArgs ba{x, dy, w.Qr, w.Kr, w.da, w.sc, w.gam, D, states, w.dst, d_x, w.dQ, w.dK, w.d_da, w.d_sc, w.d_gam,
             w.dD_part, d};
  M3_HIP(chunk_bwd(d.N, act, nullptr, &ba, grid, st));
  if (d.NA > 0) {
    // theta is read as its chunk-local sums plus w.atot, the forward scan's
    // chunk totals, before the reverse scan below reuses w.atot
    RotBwdArgs rb{w.Qr, w.Kr, w.theta, w.atot, w.dQ, w.dK, w.dtheta, d};
    M3_HIP(launch_rot_bwd(act, rb, blocks(bht * d.NA), st));
    // g = suffix sums of dtheta (in place), then the per-step contributions
    ScanArgs sa{nullptr, nullptr, w.dtheta, w.dtheta, w.atot, d};
    hipLaunchKernelGGL(m3_scan_local_kernel<true>, dim3(blocks(d.B * d.H * d.nc * d.NA)), dim3(256), 0, st, sa);
    hipLaunchKernelGGL(m3_scan_carry_kernel<true>, dim3(blocks(d.B * d.H * d.NA)), dim3(256), 0, st, sa);
    ThetaBwdArgs tb{w.dtheta, w.atot, w.dt, angles_raw, w.cang, w.ddt_ang, d};
    if ((d.NA & (d.NA - 1)) == 0 && d.B * d.H <= 65535 && d.T * d.NA < (int64_t(1) << 31)) {
      const dim3 tg(blocks(d.T * d.NA, 256 * kThetaU), static_cast<unsigned>(d.B * d.H));
      hipLaunchKernelGGL(m3_theta_grad_kernel, tg, dim3(256), 0, st, tb);
    } else {
      hipLaunchKernelGGL(m3_theta_contrib_kernel, dim3(blocks(bht * d.NA)), dim3(256), 0, st, tb);
      hipLaunchKernelGGL(m3_theta_dt_kernel, dim3(blocks(bht)), dim3(256), 0, st, tb);
    }
    M3_HIP(hipGetLastError());
    AngArgs aa{w.cang, d_angles_raw, d};
    hipLaunchKernelGGL(m3_angle_sum_kernel, dim3(blocks(d.B * d.T * d.NA)), dim3(256), 0, st, aa);
    M3_HIP(hipGetLastError());
  } else {
    hipLaunchKernelGGL(m3_zero_kernel, dim3(blocks(bht)), dim3(256), 0, st, w.ddt_ang, bht);
    M3_HIP(hipGetLastError());
  }
  ScalarBwdArgs sb{dd_dt_raw, dd_a_raw, trap_raw, dt_bias, w.d_da, w.d_sc, w.d_gam, w.ddt_ang, d_dd_dt_raw,
                   d_dd_a_raw, d_trap_raw, d};
  hipLaunchKernelGGL(m3_scalar_bwd_kernel, dim3(blocks(bht)), dim3(256), 0, st, sb);
  M3_HIP(hipGetLastError());
  GroupArgs ga{w.dK, w.dQ, d_b_in, d_c_in, d};
  M3_HIP(launch_group_sum(act, ga, blocks(d.B * d.T * d.G * d.N), st));
  // bias gradients: column sums over (b, t) of dK / dQ (B / C biases) and of
  // d_dd_dt_raw (dt bias, [B * T rows, H]); the D gradient sums the per-chunk partials
  {
    const int64_t pbc = int64_t(kRowBlocks) * d.H * d.N, pdt = int64_t(kRowBlocks) * d.H;
    ColJobs cj{};
    cj.job[0] = ColArgs{w.dK, w.colpart, d_b_bias, d.B, d.H, d.T, d.N};
    cj.job[1] = ColArgs{w.dQ, w.colpart + pbc, d_c_bias, d.B, d.H, d.T, d.N};
    cj.job[2] = ColArgs{d_dd_dt_raw, w.colpart + 2 * pbc, d_dt_bias, 1, 1, d.B * d.T, d.H};
    cj.job[3] = ColArgs{w.dD_part, w.colpart + 2 * pbc + pdt, d_D, d.B, d.H, d.nc, 1};
    const unsigned nj = D ? 4 : 3;
    hipLaunchKernelGGL(m3_colpart_kernel, dim3(blocks(kRowBlocks * d.H * d.N), nj), dim3(256), 0, st, cj);
    hipLaunchKernelGGL(m3_colsum_kernel, dim3(blocks(d.H * d.N), nj), dim3(256), 0, st, cj);
  }
  M3_HIP(hipGetLastError());
  mscan::set_last_error("");
  return MAMBA_OK;
}

}  // extern "C"
