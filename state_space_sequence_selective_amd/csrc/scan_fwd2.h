// Forward of the selective-scan layer core with one channel per lane
// (gfx950).
//
// Steps (mamba-rs 0.3.1 src/mamba_ssm/gpu/forward_mixed.rs, per-layer
// forward): F4a causal depthwise conv1d + SiLU (fused entry only), F4c
// delta = softplus(delta_raw), F4d the f32 recurrence
//   h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t,  y_t = C_t . h_t + D u_t
// with A = -exp(a_log) (mamba-rs 0.7.3 trainer.rs, recompute_a_neg_all),
// and F4e out = y * silu(z).
//
// Mapping.  A workgroup is one wave: 64 consecutive channels of one batch
// row (lane = channel), every state of a channel in that lane's registers,
// walking one segment of the sequence.  Per step a lane does its channel's
// softplus / conv / gate once and the DS state updates, and sums C.h over
// its own states, so the step loop touches no LDS and has no barrier.
// Inputs arrive by asynchronous copies (global_load_lds, no registers) into
// a ring of three per-wave LDS buffers, issued two 8-step tiles ahead: the
// tile's x / delta_raw / z rows of the wave's 64 channels, and its B_t / C_t
// rows from an f32 copy of the B / C columns that bc_f32_kernel writes
// first.  B_t and C_t are the same for every channel of a batch row, so a
// step reads them as LDS broadcasts (every lane the same address).  (Scalar
// loads of B / C into SGPRs were tried first: a scalar wait is a wait for
// every scalar load in flight, so they could run only one step ahead, and
// each step stalled on a cache miss.)
//
// Modes:
//   MAIN  : the forward proper (out, y_save, u_out, checkpoints every L
//           steps, h_last, conv_state_last).
//   AGG   : segments 0 .. S-2 scanned from a zero state; only their end
//           state and sum of delta are kept.  MAIN then starts segment s from
//           h0 folded through the pairs of segments 0 .. s-1:
//             h <- exp(A * sum delta) h + H      (exp of a sum = product of dA).
//   REGEN : for the backward, from the checkpoints of an interval L > 16:
//           the state entering every 16th step of each L-step chunk (one
//           wave per chunk), written as 16-step checkpoints.
#pragma once
#include <type_traits>

#include "scan_common.h"

namespace mscan {

enum : int { kFwdMain = 0, kFwdAgg = 1, kFwdRegen = 2 };

constexpr int kFwd2Tile = 8;   // steps per prefetch tile

struct Fwd2Args {
  const void* x;            // u (scan entry) or conv input (fused entry) [B,T,Di]
  const void* delta_raw;    // [B,T,Di]
  const float* a_log;       // [Di,Ds]
  const float* bc;          // [B*T, 2*Ds] f32: B_t then C_t
  const float* D;           // [Di] or null
  const void* z;            // [B,T,Di] (rows ldz elements apart) or null
  const float* h0;          // [B,Di,Ds] or null
  const float* conv_w;      // [Di,K] (K > 0)
  const float* conv_b;      // [Di] or null
  const float* conv_state0; // [B,Di,K] or null
  void* out;                // [B,T,Di]
  void* u_out;              // [B,T,Di] or null
  void* y_save;             // [B,T,Di] or null
  float* h_last;            // [B,Di,Ds] or null
  float* conv_state_last;   // [B,Di,K] or null
  float* ckpt;              // MAIN: written, or null; REGEN: read.  [B,nC,Ds,Di]
  float* sub;               // REGEN: [B,ceil(T/16),Ds,Di]
  float* seg_h;             // [B,S,Ds,Di] end state of each segment scanned from zero
  float* seg_sd;            // [B,S,Di] sum of delta over each segment
  int64_t B, T, Di, nC;
  int64_t ldz;              // elements between rows of z (>= Di)
  int64_t seg_steps;        // steps per segment (a multiple of 16); REGEN: L
  int K;                    // conv taps, 0 = no conv
  int L;                    // checkpoint interval (a multiple of 16)
  int S;                    // segments (REGEN: chunks)
};

struct BcArgs {
  const void* xdbl;         // [B*T, X] act
  float* bc;                // [B*T, 2*Ds] f32
  int64_t rows, X, R, Ds;
};

// f32 copy of the B / C columns of xdbl, one row per token.
template <Act A>
__global__ void __launch_bounds__(256) bc_f32_kernel(const BcArgs p) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t W = 2 * p.Ds;
  if (j >= p.rows * W) return;
  const int64_t r = j / W, m = j % W;
  p.bc[j] = IO<A>::ld(p.xdbl, r * p.X + p.R + m);
}

typedef const __attribute__((address_space(4))) float const_f32;

// Waves per SIMD the register allocation must allow: the ring of three LDS
// buffers allows three to four per SIMD at d_state 16, so registers should
// not be the tighter limit.
template <int DS>
constexpr int fwd2_waves_per_eu() {
  return DS <= 16 ? 4 : (DS == 32 ? 3 : 2);
}

template <Act A, int DS, bool FUSED, int MODE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(fwd2_waves_per_eu<DS>())))
scan_fwd2_kernel(const Fwd2Args p) {
  constexpr int DSB = DS < 8 ? DS : 8;     // states per scalar-load batch
  constexpr int NB = DS / DSB;             // batches per step
  static_assert(NB * DSB == DS, "d_state");
  constexpr int U = kFwd2Tile;
  constexpr int KMAX = FUSED ? 4 : 1;
  using io = IO<A>;

  const int lane = threadIdx.x;
  const int64_t ncb = (p.Di + 63) / 64;
  const int64_t nwg = ncb * p.B;
  const int64_t seg = blockIdx.x / nwg;
  const int64_t b = (blockIdx.x % nwg) / ncb;
  const int64_t i = (blockIdx.x % ncb) * 64 + lane;
  const bool on = i < p.Di;
  const int64_t ic = on ? i : p.Di - 1;    // loads of lanes past d_inner stay in bounds
  const int64_t T = p.T, Di = p.Di, row0 = b * T;
  const bool gate = MODE == kFwdMain && p.z != nullptr;
  const int K = FUSED ? p.K : 0;

  // this wave's steps
  const int64_t t_begin = seg * p.seg_steps;
  const int64_t t_end = t_begin + p.seg_steps < T ? t_begin + p.seg_steps : T;

  float a2[DS], h[DS];
#pragma unroll
  for (int n = 0; n < DS; ++n) a2[n] = -expf(p.a_log[ic * DS + n]) * kLog2e;
  if constexpr (MODE == kFwdRegen) {
#pragma unroll
    for (int n = 0; n < DS; ++n) h[n] = p.ckpt[((b * p.nC + seg) * DS + n) * Di + ic];
  } else if constexpr (MODE == kFwdAgg) {
#pragma unroll
    for (int n = 0; n < DS; ++n) h[n] = 0.0f;
  } else {
    // h0 folded through the (sum of delta, end state) pairs of segments
    // 0 .. seg-1 in order.  QU segments' loads are issued before their FMAs
    // (indexes past seg-1 clamped, their values unused), so the fold waits
    // about seg / QU memory round trips rather than one per segment and state.
    constexpr int QU = DS <= 16 ? 64 / DS : (DS == 32 ? 2 : 1);
#pragma unroll
    for (int n = 0; n < DS; ++n) h[n] = p.h0 ? p.h0[(b * Di + ic) * DS + n] : 0.0f;
    for (int64_t q0 = 0; q0 < seg; q0 += QU) {
      float sd[QU], hs[QU][DS];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int64_t r = b * p.S + (q0 + u < seg ? q0 + u : seg - 1);
        sd[u] = p.seg_sd[r * Di + ic];
#pragma unroll
        for (int n = 0; n < DS; ++n) hs[u][n] = p.seg_h[(r * DS + n) * Di + ic];
      }
#pragma unroll
      for (int u = 0; u < QU; ++u)
        if (q0 + u < seg) {
#pragma unroll
          for (int n = 0; n < DS; ++n) h[n] = fmaf(exp2_fast(a2[n] * sd[u]), h[n], hs[u][n]);
        }
    }
  }
  const float Dv = (MODE == kFwdMain && p.D) ? p.D[ic] : 0.0f;
  // conv taps, zero-padded at the front to KMAX (tap KMAX-1 multiplies the
  // current input), and the window of the KMAX-1 inputs before the current
  // step, oldest first: xw[k] = x_{t-(KMAX-1)+k}.  Padding keeps the step
  // free of branches on K.
  float cw[KMAX], xw[KMAX];
  float cb = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int j = k - (KMAX - K);   // tap index of slot k
    cw[k] = (FUSED && j >= 0) ? p.conv_w[ic * K + j] : 0.0f;
    xw[k] = 0.0f;
  }
  if constexpr (FUSED) {
    cb = p.conv_b ? p.conv_b[ic] : 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX - 1; ++k) {   // inputs before the first step
      const int64_t s = t_begin - (KMAX - 1) + k;
      float xv = 0.0f;
      if (s >= 0) xv = io::ld(p.x, (row0 + s) * Di + ic);
      else if (p.conv_state0 && s >= -static_cast<int64_t>(K)) xv = p.conv_state0[(b * Di + ic) * K + (K + s)];
      xw[k] = xv;
    }
  }

  // ---- LDS ring: per tile, B/C rows [U][2*DS] f32, then x | delta_raw | z
  // rows [3][U][64 channels] of raw elements.  Copies of tile k go to
  // buffer k % 3 and are issued at the end of tile k - 2.
  constexpr int ES = A == Act::F32 ? 4 : 2;
  constexpr int NBUF = 3;
  constexpr int BCB = U * 2 * DS * 4;                 // B/C bytes per tile
  constexpr int BCG = BCB % 1024 == 0 ? 16 : 4;       // bytes per lane per B/C copy instruction
  constexpr int NBC = BCB / (64 * BCG);               // B/C copy instructions per tile
  static_assert(NBC * 64 * BCG == BCB, "B/C tile");
  static_assert(U % 2 == 0, "two 16-bit rows per copy instruction");
  constexpr int RB = 64 * ES;                         // one row of the wave's channels
  constexpr int RPI = 256 / RB;                       // rows per 4-byte-granule copy instruction
  constexpr int NACT = (MODE == kFwdMain ? 3 : 2) * U / RPI;   // activation copy instructions per tile
  constexpr int NCOPY = NBC + NACT;
  static_assert(NCOPY <= 63, "copies in flight that one s_waitcnt can express");
  constexpr int ACT0 = BCB;                           // byte offset of the x rows
  constexpr int BUFB = BCB + 3 * U * RB;
  __shared__ __attribute__((aligned(16))) char s_buf[NBUF][BUFB];

  const void* zsrc = gate ? p.z : p.x;   // unused without the gate
  // lane j of a copy instruction covers channels cb*64 + 2j' .. (16-bit: two
  // per lane, two rows per instruction) or cb*64 + j (f32): clamped to
  // d_inner, so no copy leaves the tensor (d_inner % 4 == 0)
  const int cpl = ES == 2 ? 2 : 1;                    // channels per lane per copy
  const int lrow = ES == 2 ? lane >> 5 : 0;           // row of this lane within an instruction
  int64_t cch = (blockIdx.x % ncb) * 64 + (ES == 2 ? (lane & 31) * 2 : lane);
  if (cch > Di - cpl) cch = Di - cpl;
  auto issue = [&](int64_t t0) {
    lds_char_t* dst = (lds_char_t*)s_buf[((t0 - t_begin) / U) % NBUF];
    // B/C: the tile's rows are contiguous in p.bc; rows past the end of the
    // sequence re-read its last row
#pragma unroll
    for (int q = 0; q < NBC; ++q) {
      const int64_t byte = static_cast<int64_t>(q) * 64 * BCG + static_cast<int64_t>(lane) * BCG;
      int64_t r = t0 + byte / (2 * DS * 4);
      const int64_t within = byte % (2 * DS * 4);
      r = r < T ? r : T - 1;
      const char* g = reinterpret_cast<const char*>(p.bc) + (row0 + r) * (2 * DS * 4) + within;
      if constexpr (BCG == 16) __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + q * 64 * BCG), 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + q * 64 * BCG), 4, 0, 0);
    }
    const void* srcs[3] = {p.x, p.delta_raw, zsrc};
    const int64_t lds_[3] = {Di, Di, gate ? p.ldz : Di};   // row strides
#pragma unroll
    for (int a = 0; a < (MODE == kFwdMain ? 3 : 2); ++a) {
#pragma unroll
      for (int q = 0; q < U / RPI; ++q) {
        int64_t t = t0 + q * RPI + lrow;
        t = t < T ? t : T - 1;
        const char* g = static_cast<const char*>(srcs[a]) + ((row0 + t) * lds_[a] + cch) * ES;
        __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + ACT0 + (a * U + q * RPI) * RB), 4, 0, 0);
      }
    }
  };
  // the copies of the tile at buffer `buf` have landed (only the next tile's
  // copies, the NCOPY youngest memory operations, may still be in flight)
  auto wait_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitVm(NCOPY));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto raw_act = [&](const char* buf, int a, int k) -> uint32_t {
    const char* q = buf + ACT0 + (a * U + k) * RB + lane * ES;
    if constexpr (ES == 4) return *reinterpret_cast<const uint32_t*>(q);
    else return *reinterpret_cast<const uint16_t*>(q);
  };

  constexpr int ESo = ES;
  const uint32_t voff = static_cast<uint32_t>(ic) * ESo;
  const uint32_t rstride = static_cast<uint32_t>(Di) * ESo;
  auto rsrc = [&](const void* base, int64_t t0) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(base)) + (row0 + t0) * Di * ESo, 0, 0x7fffffff, 0x00020000);
  };
  // typed store of v at step row so (bytes) of the tile whose descriptor is r
  auto st1 = [&](__amdgpu_buffer_rsrc_t r, uint32_t so, float v) {
    if constexpr (A == Act::F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, so, 0);
    else if constexpr (A == Act::BF16)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, voff, so, 0);
    else __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v)), r, voff, so, 0);
  };

  float sd_acc = 0.0f;   // AGG: the segment's sum of delta

  struct Outs {
    __amdgpu_buffer_rsrc_t out, y, u;
  };
  auto outs_at = [&](int64_t t0) {
    Outs o;
    o.out = rsrc(p.out, t0);
    o.y = rsrc(p.y_save ? p.y_save : p.out, t0);
    o.u = rsrc(p.u_out ? p.u_out : p.out, t0);
    return o;
  };
  // one step: per-lane work, then the states.  Only the last tile of a
  // segment can reach past its end (CHECK): the others skip the test.
  auto step = [&](auto check, int64_t t, const char* buf, int k, const Outs& o) {
    constexpr bool CHECK = decltype(check)::value;
    const bool live = !CHECK || t < t_end;   // wave-uniform
    float dl = softplus(io::cvt(raw_act(buf, 1, k)));
    float u;
    if constexpr (FUSED) {
      const float xn = io::cvt(raw_act(buf, 0, k));
      // padded taps are skipped by a select, not multiplied by zero: a
      // non-finite input they would see must not reach the sum
      float pre = cb;
#pragma unroll
      for (int k2 = 0; k2 < KMAX - 1; ++k2) pre = k2 >= KMAX - K ? fmaf(cw[k2], xw[k2], pre) : pre;
      pre = fmaf(cw[KMAX - 1], xn, pre);
      // slide the window: x_{t-(KMAX-2)..t} for the next step
#pragma unroll
      for (int k2 = 0; k2 < KMAX - 2; ++k2) xw[k2] = xw[k2 + 1];
      xw[KMAX - 2] = xn;
      u = pre * sigmoid(pre);
    } else {
      u = io::cvt(raw_act(buf, 0, k));
    }
    if (!live) {   // steps past the segment end leave the state unchanged
      dl = 0.0f;
      u = 0.0f;
    }
    const float du = dl * u;
    float y = Dv * u;
    if constexpr (MODE == kFwdAgg) sd_acc += dl;
    const float4* bcv = reinterpret_cast<const float4*>(buf + k * 2 * DS * 4);   // B_t | C_t, broadcast
#pragma unroll
    for (int n4 = 0; n4 < DS / 4; ++n4) {
      const float4 bb = bcv[n4];
      const float bq[4] = {bb.x, bb.y, bb.z, bb.w};
      float4 cc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if constexpr (MODE == kFwdMain) cc = bcv[DS / 4 + n4];
      const float cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int s = n4 * 4 + m;
        const float dA = exp2_fast(dl * a2[s]);
        h[s] = fmaf(dA, h[s], du * bq[m]);
        if constexpr (MODE == kFwdMain) y = fmaf(cq[m], h[s], y);
      }
    }
    if constexpr (MODE == kFwdMain) {
      if (live && on) {
        const uint32_t so = static_cast<uint32_t>(k) * rstride;
        if (gate) {
          const float zv = io::cvt(raw_act(buf, 2, k));
          st1(o.out, so, y * (zv * sigmoid(zv)));
        } else {
          st1(o.out, so, y);
        }
        if (p.y_save) st1(o.y, so, y);
        if (FUSED && p.u_out) st1(o.u, so, u);
      }
    }
  };

  // checkpoints fall on 16-step boundaries, i.e. at the start of even tiles
  int64_t ck = (t_begin + p.L - 1) / p.L;   // MAIN: the next checkpoint, at step ck * L
  auto boundary = [&](int64_t t0) {
    if constexpr (MODE == kFwdMain) {
      if (t0 == ck * p.L) {
        if (p.ckpt && on) {
#pragma unroll
          for (int n = 0; n < DS; ++n) p.ckpt[((b * p.nC + ck) * DS + n) * Di + i] = h[n];
        }
        ++ck;
      }
    } else if constexpr (MODE == kFwdRegen) {
      if ((t0 & 15) == 0 && t0 < t_end && on) {
        const int64_t c = t0 >> 4, n16 = (T + 15) >> 4;
#pragma unroll
        for (int n = 0; n < DS; ++n) p.sub[((b * n16 + c) * DS + n) * Di + i] = h[n];
      }
    }
  };

  // tiles k = 0, 1, ...: copies of tile k+2 are issued once tile k is done;
  // the buffer they fill last held tile k-1
  issue(t_begin);
  issue(t_begin + U);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += U) {
    wait_tile();
    const char* buf = s_buf[((t0 - t_begin) / U) % NBUF];
    boundary(t0);
    const Outs o = outs_at(t0);
    __builtin_amdgcn_s_setprio(1);
    // without the stores of the main pass to pace it, the compiler would
    // hoist the reads and per-step work of all U steps (twice the
    // registers): a compiler-only memory barrier keeps them per step
    if (t0 + U <= t_end) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        step(std::false_type{}, t0 + k, buf, k, o);
        if constexpr (MODE != kFwdMain) __asm__ __volatile__("" ::: "memory");
      }
    } else {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        step(std::true_type{}, t0 + k, buf, k, o);
        if constexpr (MODE != kFwdMain) __asm__ __volatile__("" ::: "memory");
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // the LDS reads of the tile before this one are complete before copies
    // overwrite its buffer
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);
    issue(t0 + 2 * U);
  }
  // drain the copies still in flight before the wave's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  if constexpr (MODE == kFwdAgg) {
    if (on) {
      const int64_t r = b * p.S + seg;
#pragma unroll
      for (int n = 0; n < DS; ++n) p.seg_h[(r * DS + n) * Di + i] = h[n];
      p.seg_sd[r * Di + i] = sd_acc;
    }
    return;
  }
  if constexpr (MODE == kFwdMain) {
    if (seg != p.S - 1 || !on) return;   // the last segment ends the sequence
    if (p.h_last) {
#pragma unroll
      for (int n = 0; n < DS; ++n) p.h_last[(b * Di + i) * DS + n] = h[n];
    }
    if (FUSED && p.conv_state_last) {
      for (int k = 0; k < K; ++k) {
        const int64_t s = T - K + k;
        float xv;
        if (s >= 0) xv = io::ld(p.x, (row0 + s) * Di + i);
        else xv = p.conv_state0 ? p.conv_state0[(b * Di + i) * K + (K + s)] : 0.0f;
        p.conv_state_last[(b * Di + i) * K + k] = xv;
      }
    }
  }
}

// ------------------------------------------------------------------ launch
template <Act A>
hipError_t launch_bc_f32(const BcArgs& p, hipStream_t st) {
  const int64_t n = p.rows * 2 * p.Ds;
  hipLaunchKernelGGL(bc_f32_kernel<A>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <Act A, int DS, bool FUSED, int MODE>
static hipError_t launch_fwd2_m(const Fwd2Args& p, int64_t waves, hipStream_t st) {
  hipLaunchKernelGGL((scan_fwd2_kernel<A, DS, FUSED, MODE>), dim3(static_cast<unsigned>(waves)), dim3(64), 0, st, p);
  return hipGetLastError();
}

// MAIN (with its AGG pass first when segmented) or REGEN.
template <Act A, int DS>
static hipError_t launch_fwd2_ds(const Fwd2Args& p, bool regen, hipStream_t st) {
  const int64_t nwg = (p.Di + 63) / 64 * p.B;
  const bool fused = p.K > 0;
  if (regen)
    return fused ? launch_fwd2_m<A, DS, true, kFwdRegen>(p, nwg * p.S, st)
                 : launch_fwd2_m<A, DS, false, kFwdRegen>(p, nwg * p.S, st);
  if (p.S > 1) {
    const hipError_t e = fused ? launch_fwd2_m<A, DS, true, kFwdAgg>(p, nwg * (p.S - 1), st)
                               : launch_fwd2_m<A, DS, false, kFwdAgg>(p, nwg * (p.S - 1), st);
    if (e != hipSuccess) return e;
  }
  return fused ? launch_fwd2_m<A, DS, true, kFwdMain>(p, nwg * p.S, st)
               : launch_fwd2_m<A, DS, false, kFwdMain>(p, nwg * p.S, st);
}

template <Act A>
hipError_t launch_fwd2_a(const Fwd2Args& p, int ds, bool regen, hipStream_t st) {
  switch (ds) {
    case 4: return launch_fwd2_ds<A, 4>(p, regen, st);
    case 8: return launch_fwd2_ds<A, 8>(p, regen, st);
    case 16: return launch_fwd2_ds<A, 16>(p, regen, st);
    case 32: return launch_fwd2_ds<A, 32>(p, regen, st);
    case 64: return launch_fwd2_ds<A, 64>(p, regen, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mscan
