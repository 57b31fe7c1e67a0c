// Backward of the selective-scan layer core (gfx950): the reverse-time
// adjoint of the forward in scan_fwd.h.
//
// What it produces follows the backward scratch of the mamba-rs 0.3.1
// forward_mixed.rs page (GpuMambaMixedTrainScratch): d_y from the gate,
// d_gate (= d_z), d_delta -> d_delta_raw (softplus backward), d_u, d_B and
// d_C reduced over channels, per-sample d_D and d_a_log, and the conv1d
// weight / bias gradients.  Per step t (reverse time) and state n:
//   dh      = dy_t C_t[n] + carry          (dL/dh_t)
//   d_C     += dy_t h_t        d_B += dh delta_t u_t
//   d_u_t   += dh delta_t B_t  d_delta_t += dh (B_t u_t + A dA h_{t-1})
//   d_A     += dh delta_t dA h_{t-1}       carry = dh dA
// with d_u_t += D dy_t, d_D += dy_t u_t and d_a_log = A d_A (A = -exp(a_log)).
//
// Mapping.  A workgroup owns CPW channels of one batch row; thread (gs, c)
// owns channel c's states [gs*SPL, (gs+1)*SPL) and a wave covers 64 / CPW
// state groups.  The sequence is walked backwards in tiles of L steps, L
// being the checkpoint interval.  Per tile:
//   stage     : the tile's raw activations (already in LDS, copied there
//               asynchronously during the previous tile) become, per
//               (t, channel) item, {delta, delta*u, dy, u} in LDS; d_z =
//               dout * y * silu'(z) is written at once from the saved y.
//               Then the copies for the next tile are issued.
//   recompute : from the checkpoint each thread re-runs its states over the
//               tile and keeps h_t and dA_t of every step in registers
//               (SPL*L = 64 of each).  Every G steps each state group sums
//               dy*h over its CPW channels (d_C) in a private LDS block.
//   reverse   : G steps at a time each thread runs the adjoint of its states,
//               its state group sums delta*u*dh over the channels (d_B) the
//               same way, and
//               leaves per-(t, channel) partials of sum_n dh B and
//               sum_n dh A dA h_{t-1} in LDS; the epilogue threads add the
//               partials of all groups and write d_u (fused: as f32 to
//               du_out, for the conv adjoint pass in scan_conv.h) and
//               d_delta_raw.
// Past the end of the sequence the staged values are zero, which makes the
// extra steps of a short last tile identities, so the step loops need no
// bounds tests.  d_B / d_C per channel group and d_a_log / d_D / conv grads
// per segment and batch row go to a workspace; mscan_reduce_kernel sums them
// in a fixed order.
//
// Segments.  The grid is S copies of the channel-group grid; copy s walks
// the tiles [s * seg_tiles, (s+1) * seg_tiles) backwards, starting from the
// carry the later segments hand it: the pairs (Q, sum delta) of segments
// S-1 .. s+1 from scan_bwd_carry_kernel, folded as
//   carry <- exp(A * sum delta) carry + Q.
// The fused entry recomputes u = silu(conv(x)) in the stage (the conv halo
// of a tile is read from x, or the incoming conv state before step 0) and
// leaves the conv adjoint, whose d_x crosses tile and segment borders, to a
// pass of its own over d_u.
#pragma once
#include "bwd_table.h"
#include "scan_carry.h"
#include "scan_common.h"

namespace mscan {

// Sum a group-private block red[c][o] (CPW channels x NO outputs, row
// stride NO + 1) over c; the group is the CPW consecutive lanes of one wave
// with channel index c.  Each lane gets NOL = max(1, NO / CPW) results in
// out[]; group_sum_output() names the output of out[k] on lane c (-1: none).
template <int NO, int CPW>
constexpr int group_sum_outputs_per_lane() {
  return NO > CPW ? NO / CPW : 1;
}

template <int NO, int CPW>
__device__ __forceinline__ int group_sum_output(int c, int k) {
  if constexpr (NO >= CPW) return c + k * CPW;
  else return c < NO ? c : -1;
}

template <int NO, int CPW>
__device__ __forceinline__ void group_channel_sum(const float* red, int c,
                                                  float (&out)[group_sum_outputs_per_lane<NO, CPW>()]) {
  if constexpr (NO >= CPW) {
    // every lane sums whole columns: outputs c, c + CPW, ...
    static_assert(NO % CPW == 0, "outputs per block");
#pragma unroll
    for (int k = 0; k < NO / CPW; ++k) {
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < CPW; ++m) acc += red[m * (NO + 1) + c + k * CPW];
      out[k] = acc;
    }
  } else {
    // CPW / NO lanes per output, each summing NO channels, then a butterfly
    static_assert((CPW % NO) == 0, "outputs per block");
    constexpr int LPO = CPW / NO;    // lanes per output
    constexpr int CPL = CPW / LPO;   // channels per lane
    const int o = c % NO, part = c / NO;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) acc += red[(part * CPL + m) * (NO + 1) + o];
#pragma unroll
    for (int off = NO; off < CPW; off <<= 1) acc += __shfl_xor(acc, off, 64);
    out[0] = acc;
  }
}

// The same sum when channels c and c + 16 of the group were already added
// in registers (a v_permlane16_swap of two values, see the step loops): the
// block holds 16 channel-pair rows, red[cp][o] (row stride NO + 1), and LPO
// = 32 / NO lanes share an output, each adding NO / 2 rows before a
// butterfly over them.  Lane c < NO ends with output c.
template <int NO>
__device__ __forceinline__ float group_pair_sum(const float* red, int c) {
  static_assert(NO >= 2 && NO <= 16 && 32 % NO == 0, "outputs per block");
  constexpr int LPO = 32 / NO, RPL = 16 / LPO;
  const int o = c % NO, part = c / NO;
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < RPL; ++m) acc += red[(part * RPL + m) * (NO + 1) + o];
#pragma unroll
  for (int off = NO; off < 32; off <<= 1) acc += __shfl_xor(acc, off, 64);
  return acc;
}

// Two values a, b per lane, lanes c and c + 16 (c < 16, in each 32-lane half)
// holding one channel pair: one v_permlane16_swap and one add leave lane c
// with a(c) + a(c + 16) and lane c + 16 with b(c) + b(c + 16).
__device__ __forceinline__ float pair16(float a, float b) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Bytes of the raw tile: x (with the conv halo) | delta_raw | dout | z | y.
// It lives in dynamic LDS: the compiler then sees it as an object of its own
// and does not hold LDS accesses to the other arrays until the tile's
// asynchronous copies land (with all arrays static it did, at the first
// channel-sum read after the copies were issued).
template <Act A, int L, bool FUSED, int CPW>
constexpr int bwd_raw_bytes() {
  constexpr int ES = A == Act::F32 ? 4 : 2;
  constexpr int RPI = rows_per_inst<ES, CPW>();
  return (round_up(L + (FUSED ? 3 : 0), RPI) + 4 * round_up(L, RPI)) * CPW * ES;
}

// WPE: waves per SIMD the register allocation must allow (the compiler
// keeps the kernel within 512 / WPE registers).
template <Act A, int DS, int SPL, int L, bool FUSED, int CPW, int PD, int SUB, int WPE>
__global__ void __launch_bounds__(CPW * (DS / SPL)) __attribute__((amdgpu_waves_per_eu(WPE)))
scan_bwd_kernel(const BwdArgs p) {
  constexpr int G = DS / SPL;          // state groups
  constexpr int NT = CPW * G;          // threads: (state group, channel)
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(CPW == 32, "a wave holds two state groups of the same channels (lanes l and l + 32)");
  // SUB steps per sub-tile (the unit of the channel sums and the epilogue).
  // Item (step tt of the tile, channel c) is staged, and finished in the
  // epilogue, by thread (tt % G, c) as its item number tt / G; SUB divides G
  // so the items of one sub-tile belong to one block of SUB state groups.
  static_assert(L % SUB == 0 && G % SUB == 0 && L % G == 0, "sub-tiles, items");
  constexpr int NSUB = L / SUB;        // sub-tiles per tile
  constexpr int NIT = L / G;           // staged items per thread
  constexpr int NO = SUB * SPL;        // channel sums per group per sub-tile
  static_assert(PD >= 1 && PD <= L, "operand look-ahead");
  constexpr int NOL = group_sum_outputs_per_lane<NO, CPW>();
  // channel sums pre-added over channel pairs (c, c + 16) in registers when
  // the thread's states come in pairs (d_B / d_C: half the LDS traffic)
  constexpr bool PAIR = SPL % 2 == 0 && NO <= 16;
  static_assert(!PAIR || NOL == 1, "one output per lane");
  constexpr int KMAX = FUSED ? 4 : 1;  // conv taps supported: 1..4
  constexpr int ES = A == Act::F32 ? 4 : 2;
  constexpr int RB = CPW * ES;         // bytes per raw row
  constexpr int RPI = rows_per_inst<ES, CPW>();
  constexpr int XR = round_up(L + KMAX - 1, RPI);   // raw x rows: conv halo, then the tile
  constexpr int TR = round_up(L, RPI);
  constexpr int NBC = L * 2 * DS;      // B/C values per tile
  static_assert(NBC % NT == 0, "B/C values of a tile spread evenly over the threads");
  constexpr int BCPT = NBC / NT;
  // The cross-state partials are double-buffered when LDS allows it: the
  // next sub-tile's producers then need not wait for this sub-tile's
  // epilogue (one barrier per sub-tile instead of two).
  constexpr int LDS_FIXED = (XR + 4 * TR) * RB + L * CPW * 16 + (FUSED ? (L + KMAX - 1) * CPW * 4 : 4) +
                            L * 2 * DS * 4 + G * CPW * (NO + 1) * 4;
  constexpr int SPS = SUB * CPW + group_pad<CPW>(SUB * CPW);
  constexpr int PART = 2 * G * SPS * 4;
  // double-buffer when LDS still allows the workgroups per CU that WPE waves
  // per SIMD need (CPW * G / 64 waves per workgroup, 4 SIMDs per CU)
  constexpr int WG_PER_CU = (WPE * 4) / ((CPW * G + 63) / 64) > 0 ? (WPE * 4) / ((CPW * G + 63) / 64) : 1;
  constexpr int NBUF = LDS_FIXED + 2 * PART <= kLdsBytes / WG_PER_CU - 1024 ? 2 : 1;
  using io = IO<A>;

  // raw tile: x (with halo) | delta_raw | dout | z | y
  static_assert(bwd_raw_bytes<A, L, FUSED, CPW>() == (XR + 4 * TR) * RB, "raw tile size");
  extern __shared__ __attribute__((aligned(16))) char s_raw[];
  __shared__ float4 s_st[L][CPW];      // delta, delta*u, dy, u
  __shared__ float s_x[FUSED ? L + KMAX - 1 : 1][CPW];
  __shared__ float s_bc[L][DS][2];     // (B_t[n], C_t[n]) per state
  // per-group partials per (step of the sub-tile, channel), padded against
  // bank conflicts
  __shared__ float2 s_part[NBUF][G][SPS];   // per-group (sum_n dh B, sum_n dh A dA h_{t-1})
  __shared__ float s_red[G][CPW * (NO + 1)];
  // the compiler checks only the static arrays; with the dynamic raw tile a
  // launch over the limit fails at dispatch
  static_assert(bwd_raw_bytes<A, L, FUSED, CPW>() + sizeof(s_st) + sizeof(s_x) + sizeof(s_bc) + sizeof(s_part) +
                        sizeof(s_red) <= kLdsBytes,
                "workgroup LDS (static + dynamic raw tile) exceeds what gfx950 allows");

  const int tid = threadIdx.x;
  const int c = tid % CPW;             // channel within the group
  const int g = tid / CPW;             // state group
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int NW = (NT + 63) / 64;
  const int64_t ngrp = (p.Di + CPW - 1) / CPW;
  const int64_t nwg = ngrp * p.B;
  const int64_t seg = blockIdx.x / nwg;
  const int64_t wg = xcd_group_map<line_sharing_groups<ES, CPW>()>(blockIdx.x % nwg, nwg);
  const int64_t b = wg / ngrp;
  const int64_t cg = wg % ngrp;
  const int64_t i0 = cg * CPW;
  const int64_t i = i0 + c;
  const bool on = i < p.Di;
  const int64_t T = p.T, Di = p.Di, BT = p.B * p.T, row0 = b * p.T;
  const bool gate = p.z != nullptr;
  const int K = FUSED ? p.K : 0;
  float* red = s_red[g];
  lds_char_t* raw_l = (lds_char_t*)s_raw;
  const char* raw_x = s_raw;
  const char* raw_dr = s_raw + XR * RB;
  const char* raw_go = s_raw + (XR + TR) * RB;
  const char* raw_z = s_raw + (XR + 2 * TR) * RB;
  const char* raw_y = s_raw + (XR + 3 * TR) * RB;

  float a2[SPL], an[SPL], carry[SPL], dacc[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int n = g * SPL + s;
    an[s] = on ? -expf(p.a_log[i * DS + n]) : 0.0f;
    a2[s] = an[s] * kLog2e;
    carry[s] = 0.0f;
    dacc[s] = 0.0f;
  }
  if (on && p.S > 1) {   // the carry handed back by the later segments (mscan_carry_fold_kernel)
#pragma unroll
    for (int s = 0; s < SPL; ++s) carry[s] = p.seg_c[((b * p.S + seg) * Di + i) * DS + g * SPL + s];
  }
  const float Dv = (on && p.D) ? p.D[i] : 0.0f;
  float cw[KMAX];
  float cb = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) cw[k] = (FUSED && on && k < K) ? p.conv_w[i * K + k] : 0.0f;
  if (FUSED) cb = (on && p.conv_b) ? p.conv_b[i] : 0.0f;
  float acc_dD = 0.0f;

  // ---- prefetch of one tile: raw activations to LDS (async), B/C rows and
  // the checkpoint to registers (B/C as raw bits, converted in the stage, so
  // nothing waits for these loads before the tile's own copies are waited for)
  uint32_t bcn[BCPT];
  float hn[SPL];
  auto prefetch = [&](int64_t kt) {
    const int64_t t0 = kt * L;
    async_rows<ES, CPW>(raw_l, p.x, row0, t0 - (KMAX - 1), T, Di, i0, XR, wave, NW, lane, Di);
    async_rows<ES, CPW>(raw_l + XR * RB, p.delta_raw, row0, t0, T, Di, i0, TR, wave, NW, lane, Di);
    async_rows<ES, CPW>(raw_l + (XR + TR) * RB, p.dout, row0, t0, T, Di, i0, TR, wave, NW, lane, Di);
    if (gate) {
      async_rows<ES, CPW>(raw_l + (XR + 2 * TR) * RB, p.z, row0, t0, T, Di, i0, TR, wave, NW, lane, p.ldz);
      async_rows<ES, CPW>(raw_l + (XR + 3 * TR) * RB, p.y_saved, row0, t0, T, Di, i0, TR, wave, NW, lane, Di);
    }
#pragma unroll
    for (int q = 0; q < BCPT; ++q) {
      const int j = tid + q * NT;
      const int tt = j / (2 * DS), m = j % (2 * DS);
      const int64_t t = t0 + tt < T ? t0 + tt : T - 1;   // rows past the end: zeroed in the stage
      bcn[q] = io::ldraw(p.xdbl, (row0 + t) * p.X + p.R + m);
    }
#pragma unroll
    for (int s = 0; s < SPL; ++s)
      hn[s] = on ? p.ckpt[((b * p.nC + kt) * DS + g * SPL + s) * Di + i] : 0.0f;
  };

  const int64_t ntiles = (T + L - 1) / L;
  const int64_t kb = seg * p.seg_tiles;                               // this segment's tiles
  const int64_t ke = kb + p.seg_tiles < ntiles ? kb + p.seg_tiles : ntiles;
  prefetch(ke - 1);

  for (int64_t kt = ke - 1; kt >= kb; --kt) {
    const int64_t t0 = kt * L;
    const int len = static_cast<int>(T - t0 < L ? T - t0 : L);
    float e_sig[NIT];
    float h[SPL], h_in[SPL];   // h_in: the state entering the tile

    // ---------------------------------------------------------------- stage
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SPL; ++s) h[s] = h_in[s] = hn[s];
#pragma unroll
    for (int q = 0; q < BCPT; ++q) {
      const int j = tid + q * NT;
      const int tt = j / (2 * DS), m = j % (2 * DS);   // row order: B_0..B_{DS-1}, C_0..C_{DS-1}
      (&s_bc[0][0][0])[tt * 2 * DS + (m < DS ? 2 * m : 2 * (m - DS) + 1)] = tt < len ? io::cvt(bcn[q]) : 0.0f;
    }
    if (FUSED) {
      for (int j = tid; j < (L + KMAX - 1) * CPW; j += NT) {
        const int r = j / CPW, cc = j % CPW;
        const int64_t s = t0 - (KMAX - 1) + r;
        float xv = 0.0f;
        if (i0 + cc < Di) {
          if (s >= 0) xv = raw_ld<A>(raw_x, r * CPW + cc);
          else if (p.conv_state0 && s >= -(int64_t)K) xv = p.conv_state0[(b * Di + i0 + cc) * K + (K + s)];
        }
        s_x[r][cc] = xv;
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int tt = g + G * k;
      float dl = 0.0f, u = 0.0f, sig = 0.0f, dy = 0.0f;
      if (tt < len && on) {
        const int64_t e = (row0 + t0 + tt) * Di + i;
        const float dr = raw_ld<A>(raw_dr, tt * CPW + c);
        dl = softplus(dr);
        sig = sigmoid(dr);
        if (FUSED) {
          float pre = cb;
#pragma unroll
          for (int k2 = 0; k2 < KMAX; ++k2)
            if (k2 < K) pre = fmaf(cw[k2], s_x[tt + (KMAX - 1) - (K - 1) + k2][c], pre);
          u = pre * sigmoid(pre);
        } else {
          u = raw_ld<A>(raw_x, tt * CPW + c);
        }
        const float go = raw_ld<A>(raw_go, tt * CPW + c);
        if (gate) {
          const float zv = raw_ld<A>(raw_z, tt * CPW + c);
          const float sz = sigmoid(zv);
          dy = go * zv * sz;
          const float yv = raw_ld<A>(raw_y, tt * CPW + c);
          io::st(p.d_z, (row0 + t0 + tt) * p.ldz + i, go * yv * (sz * (1.0f + zv * (1.0f - sz))));
        } else {
          dy = go;
        }
      }
      s_st[tt][c] = make_float4(dl, dl * u, dy, u);
      e_sig[k] = sig;
    }
    __syncthreads();
    if (kt > kb) prefetch(kt - 1);
    // Wave priorities: the tile boundary (stage, copies, barriers) issues at
    // the normal one, the recompute one higher and the reverse pass higher
    // still, so that on a SIMD shared by several workgroups the waves deepest
    // into a tile go first (measured: T=8192 backward 1.69 -> 1.64 ms with the
    // two loops raised alike, a further 2 % with the reverse pass above the
    // recompute).
    __builtin_amdgcn_s_setprio(1);

    // Step operands {delta, delta*u, dy, u} and this thread's B_t, C_t are
    // read PD steps before their step into a ring of registers (slot = steps
    // since the start of the sweep, mod PD); the scheduling barrier per step
    // keeps the compiler from moving the reads closer to their use, so a
    // wave waits for LDS about once per sweep rather than once per step.
    float4 q_st[PD];
    float q_b[PD][SPL], q_c[PD][SPL];
    auto operands = [&](int tt, int sl) {
      q_st[sl] = s_st[tt][c];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        q_b[sl][s] = s_bc[tt][g * SPL + s][0];
        q_c[sl][s] = s_bc[tt][g * SPL + s][1];
      }
    };

    // ------------------------------------------------------------ recompute
    float hs[L][SPL], das[L][SPL];
#pragma unroll
    for (int d = 0; d < PD; ++d) operands(d, d);
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        const int tt = sb * SUB + q;
        const int sl = tt % PD;
        const float4 cur = q_st[sl];
        float cB[SPL];
#pragma unroll
        for (int s = 0; s < SPL; ++s) cB[s] = q_b[sl][s];
        if (tt + PD < L) operands(tt + PD, sl);
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const float dA = exp2_fast(cur.x * a2[s]);
          h[s] = fmaf(dA, h[s], cur.y * cB[s]);
          hs[tt][s] = h[s];
          das[tt][s] = dA;
          if constexpr (!PAIR) red[c * (NO + 1) + q * SPL + s] = cur.z * h[s];
        }
        if constexpr (PAIR) {   // states s, s+1: channels c and c + 16 added first
#pragma unroll
          for (int s = 0; s < SPL; s += 2)
            red[(c & 15) * (NO + 1) + q * SPL + s + (c >> 4)] = pair16(cur.z * h[s], cur.z * h[s + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
      float v[NOL];
      if constexpr (PAIR) v[0] = group_pair_sum<NO>(red, c);
      else group_channel_sum<NO, CPW>(red, c, v);
#pragma unroll
      for (int k = 0; k < NOL; ++k) {
        const int o = group_sum_output<NO, CPW>(c, k);   // o = step-in-sub-tile * SPL + state
        const int tt = sb * SUB + o / SPL;
        if (o >= 0 && tt < len)
          p.part_bc[(cg * BT + row0 + t0 + tt) * (2 * DS) + DS + g * SPL + o % SPL] = v[k];
      }
      wave_lds_sync();
    }

    __builtin_amdgcn_s_setprio(2);
    // -------------------------------------------------------------- reverse
#pragma unroll
    for (int d = 0; d < PD; ++d) operands(L - 1 - d, d);
#pragma unroll
    for (int sb = NSUB - 1; sb >= 0; --sb) {
      const int bi = NBUF == 2 ? (sb & 1) : 0;
#pragma unroll
      for (int q = SUB - 1; q >= 0; --q) {
        const int tt = sb * SUB + q;
        const int sl = (L - 1 - tt) % PD;
        const float4 cur = q_st[sl];
        float cB[SPL], cC[SPL];
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          cB[s] = q_b[sl][s];
          cC[s] = q_c[sl][s];
        }
        if (tt - PD >= 0) operands(tt - PD, sl);
        float su = 0.0f, sd = 0.0f;
        float dbv[SPL];   // the d_B channel-sum terms dh * delta * u
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const float dh = fmaf(cur.z, cC[s], carry[s]);
          // dA_t h_{t-1} from the saved factors (forming it as h_t - delta u B
          // would cancel when dA is small: the difference of two nearly equal
          // numbers, whose rounding error the factor A of d_a_log then scales)
          const float dah = das[tt][s] * (tt == 0 ? h_in[s] : hs[tt > 0 ? tt - 1 : 0][s]);
          const float qv = dh * dah;
          dacc[s] = fmaf(qv, cur.x, dacc[s]);
          carry[s] = dh * das[tt][s];
          su = fmaf(dh, cB[s], su);
          sd = fmaf(qv, an[s], sd);
          if constexpr (PAIR) dbv[s] = dh * cur.y;
          else red[c * (NO + 1) + q * SPL + s] = dh * cur.y;
        }
        if constexpr (PAIR) {
#pragma unroll
          for (int s = 0; s < SPL; s += 2) red[(c & 15) * (NO + 1) + q * SPL + s + (c >> 4)] = pair16(dbv[s], dbv[s + 1]);
        }
        // the wave's two state groups (lanes l and l + 32, one channel)
        // added in registers: after the swap the lower half holds both
        // groups' su, the upper half both groups' sd, for its channel
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(su), __float_as_uint(sd), false, false);
        reinterpret_cast<float*>(&s_part[bi][wave][q * CPW + c])[lane >> 5] =
            __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
      {
        float v[NOL];
        if constexpr (PAIR) v[0] = group_pair_sum<NO>(red, c);
        else group_channel_sum<NO, CPW>(red, c, v);
#pragma unroll
        for (int k = 0; k < NOL; ++k) {
          const int o = group_sum_output<NO, CPW>(c, k);
          const int tt = sb * SUB + o / SPL;
          if (o >= 0 && tt < len)
            p.part_bc[(cg * BT + row0 + t0 + tt) * (2 * DS) + g * SPL + o % SPL] = v[k];
        }
      }
      lds_barrier();

      // ---- epilogue: the sub-tile's items belong to state groups
      // [gb, gb + SUB), item number kk; thread g finishes step q = g - gb
      const int kk = sb * SUB / G, gb = sb * SUB % G;
      const int q = g - gb;
      const bool mine = q >= 0 && q < SUB;
      const int tt = sb * SUB + q;
      const bool live = mine && tt < len && on;
      const int64_t e = (row0 + t0 + tt) * Di + i;
      if (live) {
        const float4 st = s_st[tt][c];   // delta, delta*u, dy, u
        float su = 0.0f, sd = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {   // the waves' pair sums, in wave order
          const float2 pv = s_part[bi][w][q * CPW + c];
          su += pv.x;
          sd += pv.y;
        }
        const float du = fmaf(st.x, su, Dv * st.z);
        const float ddl = fmaf(st.w, su, sd);
        io::st(p.d_delta_raw, e, ddl * e_sig[kk]);
        acc_dD = fmaf(st.z, st.w, acc_dD);
        if (FUSED) p.du_out[e] = du;   // through SiLU and the conv in scan_conv.h
        else io::st(p.d_x, e, du);
      }
      if (NBUF == 1) lds_barrier();
    }
  }
  __syncthreads();

  // ------------------------------------------------ per batch-row partials
  const int64_t pb = ((seg * p.B + b) * Di + i) * p.PW;
  if (on) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) p.part_par[pb + g * SPL + s] = an[s] * dacc[s];
  }
  // d_D: the state groups' partial sums of this thread's items, added in
  // group order (layout within PW: [Ds a_log | 1 D])
  s_part[0][g][c].x = acc_dD;
  __syncthreads();
  if (g == 0 && on) {
    float tot = 0.0f;
    for (int w = 0; w < G; ++w) tot += s_part[0][w][c].x;
    p.part_par[pb + DS] = tot;
  }
}

// ------------------------------------------------------------------ launch
template <Act A, int DS, int SPL, int L, int SUB, int PD, int WPE, int PD_FUSED, int WPE_FUSED>
static hipError_t launch_bwd_t(const BwdArgs& p, hipStream_t st) {
  constexpr int G = DS / SPL;
  constexpr int CPW = kBwdCpw;
  const int64_t ng = (p.Di + CPW - 1) / CPW;
  dim3 grid(static_cast<unsigned>(ng * p.B * p.S));
  constexpr unsigned raw_fused = bwd_raw_bytes<A, L, true, CPW>();
  constexpr unsigned raw_plain = bwd_raw_bytes<A, L, false, CPW>();
  if (p.K > 0)
    hipLaunchKernelGGL((scan_bwd_kernel<A, DS, SPL, L, true, CPW, PD_FUSED, SUB, WPE_FUSED>), grid, dim3(CPW * G),
                       raw_fused, st, p);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<A, DS, SPL, L, false, CPW, PD, SUB, WPE>), grid, dim3(CPW * G), raw_plain,
                       st, p);
  return hipGetLastError();
}

// main backward: one launch over all segments (the aggregate pass, when
// S > 1, is enqueued before it by the caller)
template <Act A>
hipError_t launch_bwd_a(const BwdArgs& p, int ds, int L, hipStream_t st) {
  // the configurations are listed in bwd_table.h
#define MSCAN_CASE(DS_, L_, SPL_, SUB_, PD_, W_, PDF_, WF_) \
  if (ds == DS_ && L == L_) return launch_bwd_t<A, DS_, SPL_, L_, SUB_, PD_, W_, PDF_, WF_>(p, st);
  MSCAN_BWD_CONFIGS(MSCAN_CASE)
#undef MSCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace mscan
