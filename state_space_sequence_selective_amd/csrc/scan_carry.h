// Aggregate pass of the segmented backward (gfx950).
//
// The adjoint of h runs backwards in time through the same affine map as
// the forward (see the reverse-time recurrence in scan_bwd.h):
//   dh_t = dy_t C_t[n] + carry,   carry <- dh_t dA_t[n],
// so over a segment [a, b) the carry handed to step a-1 is
//   Q + (prod_{t in [a,b)} dA_t) * (carry arriving at step b-1),
// where Q is the segment's own sweep from a zero carry and the product is
// exp(A * sum of delta).  This kernel computes Q and the sum of delta for
// the sub-segments first .. S-1 (the main backward's segments cut into
// equal sub-segments, so that this pass has workgroups enough to fill the
// chip; those of the first segment hand nothing on); the main backward
// folds the pairs of the sub-segments after its own segment into its
// starting carry.
//
// Mapping as in the main backward: a workgroup owns CPW channels of one
// batch row and one segment; thread (g, c) runs states [g*SPL, (g+1)*SPL)
// of channel c.  Per tile of TT steps the raw delta_raw / dout / z rows are
// copied to LDS asynchronously during the previous tile, turned into
// {delta, dy} per (step, channel), and C_t into f32, both in LDS.
#pragma once
#include <type_traits>

#include "scan_common.h"

namespace mscan {

template <Act A, int DS, int SPL, int CPW>
__global__ void __launch_bounds__(CPW * (DS / SPL))
scan_bwd_carry_kernel(const CarryArgs p) {
  constexpr int TT = 16;               // steps per tile
  constexpr int G = DS / SPL;          // state groups
  constexpr int NT = CPW * G;
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(TT % G == 0, "items per thread");
  constexpr int IPT = TT / G;          // (step, channel) items per thread per tile
  constexpr int ES = A == Act::F32 ? 4 : 2;
  constexpr int RB = CPW * ES;
  constexpr int RPI = rows_per_inst<ES, CPW>();
  constexpr int TR = round_up(TT, RPI);
  constexpr int NCV = TT * DS;         // C values per tile
  constexpr int CPT = (NCV + NT - 1) / NT;
  using io = IO<A>;

  __shared__ __attribute__((aligned(16))) char s_raw[3 * TR * RB];   // delta_raw | dout | z
  __shared__ float2 s_q[TT][CPW];      // delta, dy
  __shared__ float s_c[TT][DS];        // C_t as f32
  __shared__ float s_sd[G][CPW];

  const int tid = threadIdx.x;
  const int c = tid % CPW;
  const int g = tid / CPW;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int NW = NT / 64;
  const int64_t ngrp = (p.Di + CPW - 1) / CPW;
  const int64_t nwg = ngrp * p.B;
  const int64_t seg = p.first + blockIdx.x / nwg;
  const int64_t wg = xcd_group_map<line_sharing_groups<ES, CPW>()>(blockIdx.x % nwg, nwg);
  const int64_t b = wg / ngrp;
  const int64_t i0 = (wg % ngrp) * CPW;
  const int64_t i = i0 + c;
  const bool on = i < p.Di;
  const int64_t T = p.T, Di = p.Di, row0 = b * p.T;
  const bool gate = p.z != nullptr;
  lds_char_t* raw_l = (lds_char_t*)s_raw;
  const char* raw_dr = s_raw;
  const char* raw_go = s_raw + TR * RB;
  const char* raw_z = s_raw + 2 * TR * RB;

  float a2[SPL], carry[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    a2[s] = on ? -expf(p.a_log[i * DS + g * SPL + s]) * kLog2e : 0.0f;
    carry[s] = 0.0f;
  }
  float sd_acc = 0.0f;

  const int64_t tps = p.seg_steps / TT;                        // tiles per segment
  const int64_t ntiles = (T + TT - 1) / TT;
  const int64_t kb = seg * tps;
  const int64_t ke = kb + tps < ntiles ? kb + tps : ntiles;

  uint32_t cbits[CPT];
  // Only the sequence's last tile can reach past its end (FULL false): the
  // other tiles skip the end tests in the row clamps and the stage.
  auto prefetch = [&](auto fullc, int64_t kt) {
    constexpr bool FULL = decltype(fullc)::value;
    const int64_t t0 = kt * TT;
    async_rows<ES, CPW>(raw_l, p.delta_raw, row0, t0, T, Di, i0, TR, wave, NW, lane, Di);
    async_rows<ES, CPW>(raw_l + TR * RB, p.dout, row0, t0, T, Di, i0, TR, wave, NW, lane, Di);
    if (gate) async_rows<ES, CPW>(raw_l + 2 * TR * RB, p.z, row0, t0, T, Di, i0, TR, wave, NW, lane, p.ldz);
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int j = tid + q * NT;
      const int tt = (j < NCV ? j : NCV - 1) / DS, n = j % DS;
      const int64_t t = FULL || t0 + tt < T ? t0 + tt : T - 1;   // rows past the end: zeroed in the stage
      cbits[q] = io::ldraw(p.xdbl, (row0 + t) * p.X + p.R + DS + n);
    }
  };

  auto stage = [&](auto fullc, int len) {
    constexpr bool FULL = decltype(fullc)::value;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int j = tid + q * NT;
      if (NCV % NT == 0 || j < NCV) (&s_c[0][0])[j] = FULL || j / DS < len ? io::cvt(cbits[q]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int tt = g + G * k;
      float dl = 0.0f, dy = 0.0f;
      if ((FULL || tt < len) && on) {
        dl = softplus(raw_ld<A>(raw_dr, tt * CPW + c));
        const float go = raw_ld<A>(raw_go, tt * CPW + c);
        if (gate) {
          const float zv = raw_ld<A>(raw_z, tt * CPW + c);
          dy = go * zv * sigmoid(zv);
        } else {
          dy = go;
        }
      }
      s_q[tt][c] = make_float2(dl, dy);
      sd_acc += dl;
    }
  };

  if ((ke - 1) * TT + TT <= T) prefetch(std::true_type{}, ke - 1);
  else prefetch(std::false_type{}, ke - 1);
  for (int64_t kt = ke - 1; kt >= kb; --kt) {
    const int64_t t0 = kt * TT;
    const int len = static_cast<int>(T - t0 < TT ? T - t0 : TT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (len == TT) stage(std::true_type{}, len);
    else stage(std::false_type{}, len);
    __syncthreads();
    if (kt > kb) prefetch(std::true_type{}, kt - 1);   // tiles before the last are whole
    // past the end of the sequence delta = dy = C = 0: the steps are identities
#pragma unroll
    for (int tt = TT - 1; tt >= 0; --tt) {
      const float2 q = s_q[tt][c];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float dA = exp2_fast(q.x * a2[s]);
        const float dh = fmaf(q.y, s_c[tt][g * SPL + s], carry[s]);
        carry[s] = dh * dA;
      }
    }
  }

  const int64_t r = b * p.S + seg;
  if (on) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) p.seg_q[(r * Di + i) * DS + g * SPL + s] = carry[s];
  }
  s_sd[g][c] = sd_acc;
  __syncthreads();
  if (g == 0 && on) {
    float tot = 0.0f;
    for (int w = 0; w < G; ++w) tot += s_sd[w][c];
    p.seg_sd[r * Di + i] = tot;
  }
}

template <Act A, int DS, int SPL>
static hipError_t launch_carry_t(const CarryArgs& p, hipStream_t st) {
  constexpr int CPW = kBwdCpw;
  constexpr int G = DS / SPL;
  const int64_t nwg = (p.Di + CPW - 1) / CPW * p.B;
  dim3 grid(static_cast<unsigned>(nwg * (p.S - p.first)));
  hipLaunchKernelGGL((scan_bwd_carry_kernel<A, DS, SPL, CPW>), grid, dim3(CPW * G), 0, st, p);
  return hipGetLastError();
}

// sub-segments first .. S-1 (first < S)
template <Act A>
hipError_t launch_carry_a(const CarryArgs& p, int ds, hipStream_t st) {
  if (ds == 4) return launch_carry_t<A, 4, 1>(p, st);
  if (ds == 8) return launch_carry_t<A, 8, 2>(p, st);
  if (ds == 16) return launch_carry_t<A, 16, 2>(p, st);
  if (ds == 32) return launch_carry_t<A, 32, 2>(p, st);
  if (ds == 64) return launch_carry_t<A, 64, 4>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace mscan
