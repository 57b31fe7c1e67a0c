// Forward of the selective-scan layer core (gfx950).
//
// Steps (mamba-rs 0.3.1 src/mamba_ssm/gpu/forward_mixed.rs, per-layer
// forward): F4a causal depthwise conv1d + SiLU (fused entry only), F4c
// delta = softplus(delta_raw), F4d the f32 recurrence
//   h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t,  y_t = C_t . h_t + D u_t
// with A = -exp(a_log) (mamba-rs 0.7.3 trainer.rs, recompute_a_neg_all),
// and F4e out = y * silu(z).
//
// Mapping.  A workgroup owns CPW channels of one batch row and walks the
// whole sequence.  Thread (gs, c) holds channel c's states
// [gs*SPL, (gs+1)*SPL) in registers; a wave covers 64 / CPW state groups, so
// B_t / C_t reads are LDS broadcasts.  Time advances in tiles of TT steps:
//   stage   : the tile's raw activations (copied to LDS asynchronously while
//             the previous tile ran) become, per (t, channel) item, delta and
//             delta*u in LDS (one softplus per item, shared by all waves);
//             then the copies for the next tile are issued.
//   scan    : each thread runs the recurrence for its states and leaves its
//             partial C.h per (t, channel) in LDS; a step's LDS operands are
//             read PD steps before the step (one LDS latency per tile, not
//             one per step).
//   output  : the staging threads add the partials of all groups, add D*u,
//             apply the gate and write out (and y, u when asked).
// The state entering every L-th step is written to ckpt for the backward.
//
// Segments.  The grid is S copies of the channel-group grid; copy s walks
// tiles [s * seg_tiles, (s+1) * seg_tiles).  With AGG the kernel is the
// aggregate pass: segments 0 .. S-2 are scanned from a zero state and only
// their end state and sum of delta are kept.  The main pass then starts
// segment s from h0 folded through the pairs of segments 0 .. s-1:
//   h <- exp(A * sum delta) h + H      (exp of a sum = product of the dA).
#pragma once
#include "scan_common.h"

namespace mscan {

template <Act A, int DS, int SPL, int TT, int CPW, bool FUSED, bool AGG>
__global__ void __launch_bounds__(CPW * (DS / SPL))
scan_fwd_kernel(const FwdArgs p) {
  constexpr int G = DS / SPL;          // state groups
  constexpr int NT = CPW * G;          // threads: (state group, channel)
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(TT % G == 0, "tile must hold a whole number of items per thread");
  constexpr int IPT = TT / G;          // (t, channel) items per thread per tile
  constexpr int KMAX = FUSED ? 4 : 1;  // conv taps supported: 1..4 (fused)
  constexpr int ES = A == Act::F32 ? 4 : 2;
  constexpr int RB = CPW * ES;         // bytes per raw row
  constexpr int RPI = rows_per_inst<ES, CPW>();
  constexpr int XR = round_up(TT + KMAX - 1, RPI);   // raw x rows: conv halo, then the tile
  constexpr int TR = round_up(TT, RPI);
  constexpr int NBC = TT * 2 * DS;
  static_assert(NBC % NT == 0, "B/C values of a tile spread evenly over the threads");
  constexpr int BCPT = NBC / NT;
  constexpr int PD = 4;                // scan operand look-ahead, steps
  static_assert(TT % PD == 0, "look-ahead ring");
  using io = IO<A>;

  // raw tiles, double-buffered (even / odd tiles): x (with halo) | delta_raw | z
  constexpr int RAW = (XR + 2 * TR) * RB;
  __shared__ __attribute__((aligned(16))) char s_raw0[RAW];
  __shared__ __attribute__((aligned(16))) char s_raw1[RAW];
  __shared__ float2 s_st[TT][CPW];     // delta, delta*u
  __shared__ float s_bc[TT][DS][2];    // (B_t[n], C_t[n]) per state, f32
  // per-state-group partial C.h per (t, channel), padded against bank conflicts
  constexpr int YPS = TT * CPW + group_pad<CPW>(TT * CPW);
  __shared__ float s_yp[G][YPS];

  const int tid = threadIdx.x;
  const int c = tid % CPW;             // channel within the group
  const int gs = tid / CPW;            // state group
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int NW = (NT + 63) / 64;
  const int64_t ngrp = (p.Di + CPW - 1) / CPW;
  const int64_t nwg = ngrp * p.B;
  const int64_t seg = blockIdx.x / nwg;
  const int64_t wg = xcd_group_map<line_sharing_groups<ES, CPW>()>(blockIdx.x % nwg, nwg);
  const int64_t b = wg / ngrp;
  const int64_t i0 = (wg % ngrp) * CPW;
  const int64_t i = i0 + c;
  const bool on = i < p.Di;
  const int64_t T = p.T, Di = p.Di, row0 = b * p.T;
  const bool gate = p.z != nullptr;
  const int K = FUSED ? p.K : 0;
  const int lshift = p.L == 32 ? 5 : 4;          // checkpoint interval 1 << lshift steps
  const int64_t lmask = (int64_t(1) << lshift) - 1;

  float a2[SPL], h[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int n = gs * SPL + s;
    a2[s] = on ? -expf(p.a_log[i * DS + n]) * kLog2e : 0.0f;
    float hv = (!AGG && on && p.h0) ? p.h0[(b * Di + i) * DS + n] : 0.0f;
    if (!AGG && on) {
      for (int64_t q = 0; q < seg; ++q) {
        const int64_t r = b * p.S + q;
        hv = fmaf(exp2_fast(a2[s] * p.seg_sd[r * Di + i]), hv, p.seg_h[(r * Di + i) * DS + n]);
      }
    }
    h[s] = hv;
  }
  float sd_acc = 0.0f;   // AGG: this thread's share of the segment's sum of delta
  const float Dv = (on && p.D) ? p.D[i] : 0.0f;
  float cw[KMAX];
  float cb = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) cw[k] = (FUSED && on && k < K) ? p.conv_w[i * K + k] : 0.0f;
  if (FUSED) cb = (on && p.conv_b) ? p.conv_b[i] : 0.0f;

  // copies of tile number kt (time t0 = kt * TT) into raw buffer `raw` and
  // its B/C values into bc, as raw bits: they are converted in the stage, so
  // nothing waits for these loads early.  Even tiles use (bc0, s_raw0), odd
  // tiles (bc1, s_raw1); the tile loop below is unrolled by two so that the
  // choice is static (a run-time choice would make the compiler merge the two
  // register sets, and a merge waits for the loads).
  uint32_t bc0[BCPT], bc1[BCPT];
  auto prefetch = [&](int64_t kt, uint32_t (&bc)[BCPT], char* raw) {
    const int64_t t0 = kt * TT;
    lds_char_t* r = (lds_char_t*)raw;
    async_rows<ES, CPW>(r, p.x, row0, t0 - (KMAX - 1), T, Di, i0, XR, wave, NW, lane);
    async_rows<ES, CPW>(r + XR * RB, p.delta_raw, row0, t0, T, Di, i0, TR, wave, NW, lane);
    if (gate) async_rows<ES, CPW>(r + (XR + TR) * RB, p.z, row0, t0, T, Di, i0, TR, wave, NW, lane);
#pragma unroll
    for (int q = 0; q < BCPT; ++q) {
      const int j = tid + q * NT;
      const int tt = j / (2 * DS), m = j % (2 * DS);
      const int64_t t = t0 + tt < T ? t0 + tt : T - 1;   // rows past the end: zeroed in the stage
      bc[q] = io::ldraw(p.xdbl, (row0 + t) * p.X + p.R + m);
    }
  };

  float e_u[IPT], e_sz[IPT];
  // per-item work of one tile: delta, delta*u to LDS; u and silu(z) kept
  auto stage = [&](int64_t kt, const uint32_t (&bc)[BCPT], const char* raw) {
    const int64_t t0 = kt * TT;
    const int len = static_cast<int>(T - t0 < TT ? T - t0 : TT);
    const char* raw_x = raw;
    const char* raw_dr = raw_x + XR * RB;
    const char* raw_z = raw_x + (XR + TR) * RB;
#pragma unroll
    for (int q = 0; q < BCPT; ++q) {
      const int j = tid + q * NT;
      const int tt = j / (2 * DS), m = j % (2 * DS);   // row order: B_0..B_{DS-1}, C_0..C_{DS-1}
      (&s_bc[0][0][0])[tt * 2 * DS + (m < DS ? 2 * m : 2 * (m - DS) + 1)] = tt < len ? io::cvt(bc[q]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int tt = gs + G * k;
      float dl = 0.0f, u = 0.0f, sz = 1.0f;
      if (tt < len && on) {
        if (FUSED) {
          float pre = cb;
#pragma unroll
          for (int k2 = 0; k2 < KMAX; ++k2) {
            if (k2 < K) {
              const int64_t s = t0 + tt - (K - 1) + k2;
              float xv;
              if (s >= 0) xv = raw_ld<A>(raw_x, (tt + (KMAX - 1) - (K - 1) + k2) * CPW + c);
              else xv = p.conv_state0 ? p.conv_state0[(b * Di + i) * K + (K + s)] : 0.0f;
              pre = fmaf(cw[k2], xv, pre);
            }
          }
          u = pre * sigmoid(pre);
        } else {
          u = raw_ld<A>(raw_x, tt * CPW + c);
        }
        dl = softplus(raw_ld<A>(raw_dr, tt * CPW + c));
        if (gate) {
          const float zv = raw_ld<A>(raw_z, tt * CPW + c);
          sz = zv * sigmoid(zv);
        }
      }
      s_st[tt][c] = make_float2(dl, dl * u);
      if (AGG) sd_acc += dl;
      e_u[k] = u;
      e_sz[k] = sz;
    }
  };
  // combine the per-group partials of one tile, gate, store
  auto output = [&](int64_t t0) {
    const int len = static_cast<int>(T - t0 < TT ? T - t0 : TT);
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int tt = gs + G * k;
      if (tt < len && on) {
        float y = Dv * e_u[k];
#pragma unroll
        for (int w = 0; w < G; ++w) y += s_yp[w][tt * CPW + c];
        const int64_t e = (row0 + t0 + tt) * Di + i;
        io::st(p.out, e, gate ? y * e_sz[k] : y);
        if (p.y_save) io::st(p.y_save, e, y);
        if (p.u_out) io::st(p.u_out, e, e_u[k]);
      }
    }
  };

  // Two barriers per tile.  Copies run two tiles ahead:
  //   (scan k) | wait + barrier | issue copies for k+2 | output k, stage k+1 |
  //   LDS barrier | (scan k+1) ...
  // tile(kt, bcS, rawS, bcP, rawP): scan and output of tile kt, stage of tile
  // kt + 1 from (bcS, rawS), copies for tile kt + 2 into (bcP, rawP), the
  // buffers of tile kt, free once stage kt is done.
  const int64_t ntiles = (T + TT - 1) / TT;
  const int64_t kb = seg * p.seg_tiles;                               // this segment's tiles
  const int64_t ke = kb + p.seg_tiles < ntiles ? kb + p.seg_tiles : ntiles;
  auto tile = [&](int64_t kt, const uint32_t (&bcS)[BCPT], const char* rawS, uint32_t (&bcP)[BCPT],
                  char* rawP) {
    const int64_t t0 = kt * TT;

    // ---- scan (steps past the end of the sequence see delta = 0, B = C = 0:
    // identities that leave h unchanged).  Operands of step tt sit in ring
    // slot tt % PD, read PD steps earlier; the scheduling barrier per step
    // keeps the compiler from pulling the reads closer to their use.
    float2 q_st[PD];
    float q_b[PD][SPL], q_c[PD][SPL];
    auto operands = [&](int tt, int sl) {
      q_st[sl] = s_st[tt][c];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        q_b[sl][s] = s_bc[tt][gs * SPL + s][0];
        q_c[sl][s] = s_bc[tt][gs * SPL + s][1];
      }
    };
#pragma unroll
    for (int d = 0; d < PD; ++d) operands(d, d);
    // the steps issue at a raised wave priority, the tile boundary at the
    // normal one, so that waves in their step loop go first on a shared SIMD
    // (measured: T=8192 forward 0.86 -> 0.78 ms)
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      // checkpoint: the state entering step t0 + tt, every L steps (L is 16
      // or 32, so only 16-step boundaries can hold one)
      if (!AGG && tt % 16 == 0 && p.ckpt && on) {
        const int64_t ts = t0 + tt;
        if ((ts & lmask) == 0 && ts < T) {
          const int64_t cidx = ts >> lshift;
#pragma unroll
          for (int s = 0; s < SPL; ++s)
            p.ckpt[((b * p.nC + cidx) * DS + gs * SPL + s) * Di + i] = h[s];
        }
      }
      const int sl = tt % PD;
      const float2 st = q_st[sl];
      float bb[SPL], cc[SPL];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        bb[s] = q_b[sl][s];
        cc[s] = q_c[sl][s];
      }
      if (tt + PD < TT) operands(tt + PD, sl);
      float yp = 0.0f;
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float dA = exp2_fast(st.x * a2[s]);
        h[s] = fmaf(dA, h[s], st.y * bb[s]);
        yp = fmaf(cc[s], h[s], yp);
      }
      if (!AGG) s_yp[gs][tt * CPW + c] = yp;
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // the copies of tile kt + 1 are complete and visible to all waves
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 2 < ke) prefetch(kt + 2, bcP, rawP);
    if (!AGG) output(t0);
    if (kt + 1 < ke) stage(kt + 1, bcS, rawS);
    // LDS-only: the copies for tile kt + 2 stay in flight through scan kt + 1
    lds_barrier();
  };

  prefetch(kb, bc0, s_raw0);
  if (kb + 1 < ke) prefetch(kb + 1, bc1, s_raw1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  stage(kb, bc0, s_raw0);
  __syncthreads();
  for (int64_t kt = kb; kt < ke; kt += 2) {
    tile(kt, bc1, s_raw1, bc0, s_raw0);
    if (kt + 1 < ke) tile(kt + 1, bc0, s_raw0, bc1, s_raw1);
  }

  if (AGG) {
    // the segment's end state from zero, and its sum of delta (the partial
    // sums of the state groups meet in LDS; s_yp is free here)
    if (on) {
      const int64_t r = b * p.S + seg;
#pragma unroll
      for (int s = 0; s < SPL; ++s) p.seg_h[(r * Di + i) * DS + gs * SPL + s] = h[s];
    }
    s_yp[gs][c] = sd_acc;
    __syncthreads();
    if (gs == 0 && on) {
      float tot = 0.0f;
      for (int w = 0; w < G; ++w) tot += s_yp[w][c];
      p.seg_sd[(b * p.S + seg) * Di + i] = tot;
    }
    return;
  }
  if (seg != p.S - 1) return;   // the last segment ends the sequence

  if (p.h_last && on) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) p.h_last[(b * Di + i) * DS + gs * SPL + s] = h[s];
  }
  if (p.conv_state_last && on && gs == 0) {
    for (int k = 0; k < K; ++k) {
      const int64_t s = T - K + k;
      float xv;
      if (s >= 0) xv = io::ld(p.x, (row0 + s) * Di + i);
      else xv = p.conv_state0 ? p.conv_state0[(b * Di + i) * K + (K + s)] : 0.0f;
      p.conv_state_last[(b * Di + i) * K + k] = xv;
    }
  }
}

// ------------------------------------------------------------------ launch
template <Act A, int DS, int SPL, int TT, int CPW>
static hipError_t launch_fwd_t(const FwdArgs& p, hipStream_t st) {
  static_assert(TT % 16 == 0, "checkpoints fall on 16-step boundaries");
  constexpr int G = DS / SPL;
  const int64_t nwg = (p.Di + CPW - 1) / CPW * p.B;
  if constexpr (TT == kFwdTileShort) if (p.S > 1) {   // aggregate pass over segments 0 .. S-2
    dim3 grid(static_cast<unsigned>(nwg * (p.S - 1)));
    if (p.K > 0)
      hipLaunchKernelGGL((scan_fwd_kernel<A, DS, SPL, TT, CPW, true, true>), grid, dim3(CPW * G), 0, st, p);
    else
      hipLaunchKernelGGL((scan_fwd_kernel<A, DS, SPL, TT, CPW, false, true>), grid, dim3(CPW * G), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(nwg * p.S));
  if (p.K > 0)
    hipLaunchKernelGGL((scan_fwd_kernel<A, DS, SPL, TT, CPW, true, false>), grid, dim3(CPW * G), 0, st, p);
  else
    hipLaunchKernelGGL((scan_fwd_kernel<A, DS, SPL, TT, CPW, false, false>), grid, dim3(CPW * G), 0, st, p);
  return hipGetLastError();
}

template <Act A>
hipError_t launch_fwd_a(const FwdArgs& p, int ds, int spl, hipStream_t st) {
  // channel groups of kFwdCpw; long tiles only without segments
#define MSCAN_CASE(DS_, SPL_)                                                       \
  if (ds == DS_ && spl == SPL_) {                                                   \
    if (p.tile == kFwdTileLong && p.S == 1)                                         \
      return launch_fwd_t<A, DS_, SPL_, kFwdTileLong, kFwdCpw>(p, st);              \
    if (p.tile == kFwdTileShort) return launch_fwd_t<A, DS_, SPL_, kFwdTileShort, kFwdCpw>(p, st); \
    return hipErrorInvalidValue;                                                    \
  }
  MSCAN_CASE(4, 1) MSCAN_CASE(8, 1) MSCAN_CASE(16, 1) MSCAN_CASE(32, 2)
#undef MSCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace mscan
