// Device helpers and kernel argument blocks shared by the selective-scan
// kernels (gfx950).  Every kernel takes ONE argument struct, so no two
// pointers can be swapped by argument order at a launch site.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

enum class Act : int { F32 = 0, BF16 = 1, F16 = 2 };

constexpr float kLog2e = 1.4426950408889634f;

// Channels per backward workgroup.  A thread is (state group, channel).
// The backward balances through sequence segments and uses 32 channels,
// which halves its per-group d_B/d_C partials against 16.
constexpr int kBwdCpw = 32;

// LDS a workgroup may hold on gfx950 (static and dynamic together)
constexpr int kLdsBytes = 160 * 1024;

// Forward sequences up to this length take scan_step_kernel (one thread per
// channel, no staging); it must not exceed the smallest checkpoint interval.
constexpr int kStepMaxT = 16;

// ---------------------------------------------------------------- dtype I/O
template <Act A>
struct IO;

// ld: load and convert to f32.  ldraw / cvt: the same split in two, so a
// value can be fetched early and converted where it is used; converting at
// once would make the compiler wait for the load right there.
template <>
struct IO<Act::F32> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ uint32_t ldraw(const void* p, int64_t i) {
    return static_cast<const uint32_t*>(p)[i];
  }
  static __device__ __forceinline__ float cvt(uint32_t b) { return __uint_as_float(b); }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};

template <>
struct IO<Act::BF16> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    const uint32_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(b << 16);
  }
  static __device__ __forceinline__ uint32_t ldraw(const void* p, int64_t i) {
    return static_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ float cvt(uint32_t b) { return __uint_as_float(b << 16); }
  // hardware conversion (v_cvt_pk_bf16_f32), round to nearest even
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);
  }
};

template <>
struct IO<Act::F16> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
  static __device__ __forceinline__ uint32_t ldraw(const void* p, int64_t i) {
    return static_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ float cvt(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  // the hardware conversion rounds to nearest even (default mode)
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
  }
};

// sum_{r < n} src[r * stride] in ascending r.  Eight loads are issued before
// their adds so each thread keeps several in flight; the adds keep the order
// (the result is that of the plain sequential loop, bit for bit).
template <int U = 8>   // loads issued before their adds
__device__ __forceinline__ float ordered_sum(const float* src, int64_t n, int64_t stride) {
  float acc = 0.0f;
  int64_t r = 0;
  for (; r + U <= n; r += U) {
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = src[(r + k) * stride];
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  for (; r < n; ++r) acc += src[r * stride];
  return acc;
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + e) for e in [0, 1].  w = 1 + e is rounded; c = (w - 1) - e is
// that rounding error exactly (w - 1 is exact for w in [1, 2], and so is the
// difference of two numbers this close), so log(1 + e) = log(w - c), which
// is log(w) - c / w to first order.  Taking c for c / w leaves an error of
// about c e, i.e. a relative error of about |c| <= 2^-24 whatever e is; for
// w = 1 (e below half an ulp of 1) it returns e exactly.  The same accuracy
// as the classic correction log(w) e / (w - 1) (Goldberg, "What every
// computer scientist should know about floating-point arithmetic",
// Theorem 4) without its reciprocal and select.
__device__ __forceinline__ float log1p_small(float e) {
  const float w = 1.0f + e;
  const float c = (w - 1.0f) - e;
  return fmaf(__builtin_amdgcn_logf(w), 0.6931471805599453f, -c);
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|)
__device__ __forceinline__ float softplus(float x) {
  return fmaxf(x, 0.0f) + log1p_small(exp2_fast(-fabsf(x) * kLog2e));
}

// logistic sigmoid; exp2 of a large positive argument gives +inf and the
// reciprocal then gives 0, which is the right limit.
__device__ __forceinline__ float sigmoid(float x) {
  return rcp_fast(1.0f + exp2_fast(-x * kLog2e));
}

// ---------------------------------------------------------------- XCD mapping
// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// linear id.  Q neighbouring channel groups share every 128-byte line of an
// activation row, so the logical workgroups Q*r .. Q*r + Q-1 are given the
// linear ids x + 8m, x + 8(m+1), ..., x + 8(m+Q-1) of one XCD x (same L2).
// Ids past the last whole block of 8*Q keep their own index.  A bijection on
// [0, n); returns the logical id.
template <int Q>
__device__ __forceinline__ int64_t xcd_group_map(int64_t k, int64_t n) {
  static_assert(Q >= 1, "group size");
  if (Q == 1) return k;
  const int64_t full = n - n % (8 * Q);
  if (k >= full) return k;
  const int64_t x = k & 7, j = k >> 3;   // XCD, round
  return (j / Q) * (8 * Q) + Q * x + (j % Q);
}

// Padding (in floats) for an LDS array [group][stride] that the rows of a
// wave (one row = CPW lanes = one state group) write at the same offset.
// LDS serves 32 lanes (one per bank) at a time; with CPW = 16 two groups
// share those 32 lanes, and a stride that is a multiple of 32 banks puts both
// on the same 16 banks.  A 16-float pad moves every other group to the other
// half of the banks.
template <int CPW>
constexpr int group_pad(int stride) {
  return (CPW < 32 && stride % 32 == 0) ? 16 : 0;
}

// channel groups of CPW channels of ES-byte elements that share a 128-byte line
template <int ES, int CPW>
constexpr int line_sharing_groups() {
  return CPW * ES >= 128 ? 1 : 128 / (CPW * ES);
}

// ---------------------------------------------------------------- barriers
// __syncthreads() is a workgroup-scope release/acquire around s_barrier; the
// release also waits for every global_load_lds copy in flight (they write
// LDS), which would turn a copy meant to overlap the next tile's work into a
// synchronous one.  The two helpers below order LDS traffic only: the fences
// are wavefront-scope (no hardware wait, but the compiler keeps memory
// accesses on their side), the hardware wait is lgkmcnt(0), i.e. this wave's
// LDS reads and writes are done.  Code that reads data brought in by
// global_load_lds waits for it explicitly (s_waitcnt 0) before a barrier.
constexpr int kWaitLgkmOnly = 0xC07F;   // s_waitcnt vmcnt(63) expcnt(7) lgkmcnt(0)

// s_waitcnt operand that waits until at most n (0..63) vector-memory
// operations of this wave are in flight, and for nothing else (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8); }

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Ordering point for LDS traffic between the lanes of one wave.  A wave's
// LDS instructions execute in issue order, so keeping the compiler from
// moving accesses across this point is enough.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- LDS staging
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int round_up(int n, int m) { return (n + m - 1) / m * m; }

// Rows one async_rows instruction covers: lanes move 4-byte granules
// (16-bit types: 2 channels) or 16-byte granules (f32: 4 channels).
template <int ES, int CPW>
constexpr int rows_per_inst() {
  return 64 / (CPW / ((ES == 4 ? 16 : 4) / ES));
}

// Asynchronous copy (global_load_lds, no registers) of `nrows` time rows of
// one CPW-channel group of an activation tensor [B, T, Di] (rows `ld`
// elements apart, ld >= Di) into LDS, one row of CPW * ES bytes after another
// starting at `dst`.  Time rows are clamped to [0, T) and granules past Di
// re-read the last granule of the row, so no load leaves the tensor
// (Di % 4 == 0).  nrows must be a multiple of
// rows_per_inst; instructions are spread over the waves.  The caller ends
// the copy with a full s_waitcnt and a workgroup barrier.
template <int ES, int CPW>
__device__ __forceinline__ void async_rows(lds_char_t* dst, const void* src, int64_t row0, int64_t t_lo,
                                           int64_t T, int64_t Di, int64_t i0, int nrows, int wave,
                                           int nwaves, int lane, int64_t ld) {
  constexpr int GB = ES == 4 ? 16 : 4;   // bytes per lane
  constexpr int GC = GB / ES;            // channels per lane
  constexpr int LPR = CPW / GC;          // lanes per row
  constexpr int RPI = 64 / LPR;          // rows per instruction
  static_assert(LPR >= 1 && 64 % LPR == 0, "row width");
  const int ninst = nrows / RPI;
  int64_t ch = i0 + (lane % LPR) * GC;
  if (ch > Di - GC) ch = Di - GC;
  const char* base = static_cast<const char*>(src) + (row0 * ld + ch) * ES;
  const int64_t rstride = ld * ES;
  for (int j = wave; j < ninst; j += nwaves) {
    int64_t t = t_lo + j * RPI + lane / LPR;
    t = t < 0 ? 0 : (t >= T ? T - 1 : t);
    const char* g = base + t * rstride;
    if constexpr (ES == 4)
      __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + j * 64 * GB), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + j * 64 * GB), 4, 0, 0);
  }
}

// element idx of a raw LDS tile (row-major, CPW channels per row) as f32
template <Act A>
__device__ __forceinline__ float raw_ld(const char* base, int idx);
template <>
__device__ __forceinline__ float raw_ld<Act::F32>(const char* base, int idx) {
  return reinterpret_cast<const float*>(base)[idx];
}
template <>
__device__ __forceinline__ float raw_ld<Act::BF16>(const char* base, int idx) {
  return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(base)[idx]) << 16);
}
template <>
__device__ __forceinline__ float raw_ld<Act::F16>(const char* base, int idx) {
  return static_cast<float>(reinterpret_cast<const _Float16*>(base)[idx]);
}

// ---------------------------------------------------------------- arguments
// short-sequence forward (scan_step_kernel)
struct FwdArgs {
  const void* x;            // u (scan entry) or conv input (fused entry) [B,T,Di]
  const void* delta_raw;    // [B,T,Di]
  const float* a_log;       // [Di,Ds]
  const void* xdbl;         // [B,T,X]
  const float* D;           // [Di] or null
  const void* z;            // [B,T,Di] or null
  const float* h0;          // [B,Di,Ds] or null
  const float* conv_w;      // [Di,K] (K > 0)
  const float* conv_b;      // [Di] or null
  const float* conv_state0; // [B,Di,K] or null
  void* out;                // [B,T,Di]
  void* u_out;              // [B,T,Di] or null
  void* y_save;             // [B,T,Di] or null
  float* h_last;            // [B,Di,Ds] or null
  float* conv_state_last;   // [B,Di,K] or null
  float* ckpt;              // [B,nC,Ds,Di] or null
  int64_t B, T, Di, R, X, nC;
  int64_t ldz;              // elements between rows of z (>= Di)
  int K;                    // conv taps, 0 = no conv
};

struct BwdArgs {
  const void* x;
  const void* delta_raw;
  const float* a_log;
  const void* xdbl;
  const float* D;
  const void* z;            // [B,T,Di], rows ldz elements apart (gate only)
  const void* y_saved;      // [B,T,Di] (gate only)
  const float* conv_w;
  const float* conv_b;
  const float* conv_state0;
  const float* ckpt;        // [B,nC,Ds,Di]
  const void* dout;
  void* d_x;                // d_u [B,T,Di] (scan entry)
  float* du_out;            // d_u [B,T,Di] f32 (fused entry: the conv adjoint pass reads it)
  void* d_delta_raw;        // [B,T,Di]
  void* d_z;                // [B,T,Di], rows ldz elements apart (gate only)
  float* part_bc;           // [nG, B*T, 2*Ds]: per channel-group sums of d_B | d_C
  float* part_par;          // [S, B, Di, PW]: per segment and batch row d_a_log | d_D
  // segmented schedule: segment s covers tiles [s * seg_tiles, ...) of L steps
  const float* seg_c;       // [B,S,Di,Ds] carry entering each segment's reverse sweep (S > 1)
  int64_t B, T, Di, R, X, nC;
  int64_t ldz;              // elements between rows of z and d_z (>= Di)
  int64_t seg_tiles;        // tiles per segment
  int K;
  int L;
  int PW;                   // Ds + 1
  int S;                    // segments
};

// aggregate pass of the segmented backward
struct CarryArgs {
  const void* delta_raw;    // [B,T,Di]
  const float* a_log;       // [Di,Ds]
  const void* xdbl;         // [B,T,X]
  const void* z;            // [B,T,Di], rows ldz elements apart, or null
  const void* dout;         // [B,T,Di]
  float* seg_q;             // [B,S,Di,Ds] out
  float* seg_sd;            // [B,S,Di] out
  int64_t B, T, Di, R, X;
  int64_t ldz;              // elements between rows of z (>= Di)
  int64_t seg_steps;        // steps per (sub-)segment (a multiple of 16)
  int S;                    // sub-segments
  int first;                // the first sub-segment computed (those before it hand nothing on)
};

// the carry pass's sub-segment pairs folded into each segment's starting carry
struct CarryFoldArgs {
  const float* a_log;       // [Di,Ds]
  const float* seg_q;       // [B,S*F,Di,Ds]
  const float* seg_sd;      // [B,S*F,Di]
  float* seg_c;             // [B,S,Di,Ds] out
  int64_t B, Di, Ds;
  int S;                    // segments
  int F;                    // sub-segments per segment
};

struct ReduceArgs {
  const float* part_bc;
  const float* part_par;    // [par_rows, Di, PW]: d_a_log | d_D
  const float* part_conv;   // [conv_rows, Di, K + 1]: d_conv_w | d_conv_b (K > 0)
  float* d_xdbl;            // [B,T,X], B/C columns +=
  float* d_a_log;           // [Di,Ds] +=
  float* d_D;               // [Di] +=
  float* d_conv_w;          // [Di,K] += or null
  float* d_conv_b;          // [Di] += or null
  int64_t B, T, Di, Ds, R, X, nG;
  int64_t par_rows;         // rows of part_par summed per element: segments * B
  int64_t conv_rows;        // rows of part_conv: B * conv tiles
  int K;
  int PW;                   // Ds + 1
};

}  // namespace mscan
