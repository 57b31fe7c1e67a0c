// The layer's skinny projections x_proj -> dt_proj on the matrix cores
// (gfx950, v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit activations.
//
// Steps F4b and F4c of the per-layer forward (mamba-rs 0.3.1
// src/mamba_ssm/gpu/forward_mixed.rs): xdbl = u W_x^T ([N, d_inner] x
// [d_inner, X], X = dt_rank + 2 d_state), then delta_raw = xdbl[:, :R] W_dt^T
// + b_dt ([N, R] x [R, d_inner]); the backward takes the adjoint in the same
// two shapes: d_xdbl[:, :R] = d_delta_raw W_dt, then d_u_extra = d_xdbl W_x
// (the whole d_xdbl row rounded to the activation dtype first; its B / C
// columns come from the core).  Each direction is three launches:
//
//   contract  part[g] = A[:, K_g] B[:, K_g]^T: the long product over
//             d_inner (K), split into G groups of K so the grid fills the
//             chip; f32 partials.
//   round     the G partials added in group order and rounded to the
//             activation dtype where the library product would store them
//             (xdbl; the d_xdbl row).
//   expand    out = x[:, :kmax] W^T (+ bias): the short product (K <= 256)
//             into the wide [N, d_inner] output.
//
// Matrix-core tile: one instruction multiplies A (16 x 32; lane l holds row
// l % 16, k = 8 (l / 16) .. + 7) by B (32 x 16; column l % 16, the same k)
// into a 16 x 16 f32 accumulator whose lane l holds rows 4 (l / 16) + e,
// column l % 16.  Operands come from LDS in that layout; global memory is
// read and written in whole row segments (neighbouring lanes, neighbouring
// addresses), the LDS rows padded so that the 16 lanes of a 16-byte access
// hit distinct banks.  A wave64 vector instruction occupies its SIMD for 4
// cycles, so the tiles are sized to give each operand load several products.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layer_kernels.h"
#include "scan_common.h"

namespace mlayer {
namespace {

using mscan::Act;

constexpr int kThr = 256;   // 4 waves
constexpr int kTok = 64;    // token rows per workgroup (4 tiles of 16)
constexpr int kMaxX = 256;  // longest xdbl row taken
constexpr int kPadE = 8;    // LDS row padding (elements)
constexpr int kDepth = 4;   // k steps the contraction's loads run ahead

template <Act A>
struct Mfma;

template <>
struct Mfma<Act::BF16> {
  typedef __bf16 elem;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 mma(const v8& a, const v8& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<Act::F16> {
  typedef _Float16 elem;
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 mma(const v8& a, const v8& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// the wave's index in the workgroup, in a scalar register (loops and
// branches over it stay uniform)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ------------------------------------------------------------ contract
// Workgroup (token block tb, K group g): rows n0 .. n0 + 63 of A [N][K] times
// the C rows of B [C][K] over the 32-wide k steps [g kchunk, (g + 1) kchunk),
// into part[g][n][c] (f32).  Each step stages A's 64 x 32 and B's C x 32
// slices in LDS (double buffered, one barrier per step); wave w multiplies
// the 4 token tiles by the column tiles w, w + 4, ... (CTW of them).  The
// global loads run kDepth steps ahead in registers (one round trip to memory
// per step would otherwise bound the kernel).  Rows past N or C are clamped
// to the last row; their products are dropped.
template <Act A, int CTW>
__global__ void __launch_bounds__(kThr) contract_kernel(const ContractArgs p) {
  using M = Mfma<A>;
  typedef typename M::elem elem;
  typedef typename M::v8 v8;
  typedef typename M::f4 f4;
  constexpr int RS = 32 + kPadE;   // LDS row stride (elements): 80 bytes
  constexpr int CB = 64 * CTW;     // B rows staged
  __shared__ __attribute__((aligned(16))) elem sa[2][kTok * RS];
  __shared__ __attribute__((aligned(16))) elem sb[2][CB * RS];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t tb = blockIdx.x / p.G, grp = blockIdx.x % p.G;
  const int64_t n0 = tb * kTok;
  const int64_t KS = p.K / 32;
  const int64_t s0 = grp * p.kchunk, s1 = s0 + p.kchunk < KS ? s0 + p.kchunk : KS;
  const int C = p.C, CT = (C + 15) / 16;
  // coalesced staging: thread t moves row t / 4 (+ 64 i), k chunk t % 4
  const int sr = tid >> 2, sc = tid & 3;
  const elem* a_src = static_cast<const elem*>(p.a) + (n0 + sr < p.N ? n0 + sr : p.N - 1) * p.K + 8 * sc;
  const elem* b_src[CTW];
#pragma unroll
  for (int i = 0; i < CTW; ++i) {
    const int c = sr + 64 * i;
    b_src[i] = static_cast<const elem*>(p.b) + static_cast<int64_t>(c < C ? c : C - 1) * p.K + 8 * sc;
  }
  v8 ra[kDepth], rb[kDepth][CTW];
  auto fetch = [&](int64_t s, v8& a, v8(&b)[CTW]) {
    a = *reinterpret_cast<const v8*>(a_src + 32 * s);
#pragma unroll
    for (int i = 0; i < CTW; ++i) b[i] = *reinterpret_cast<const v8*>(b_src[i] + 32 * s);
  };
  f4 acc[4][CTW];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int cj = 0; cj < CTW; ++cj) acc[ti][cj] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // The loads are unconditional (steps past s1 reload step s1 - 1) and the
  // rounds of kDepth steps are not cut short (the steps past s1 stage zeros),
  // so the loop body is straight-line code: a wait for one step's operands
  // then leaves the later steps' loads in flight.
#pragma unroll
  for (int d = 0; d < kDepth; ++d) fetch(s0 + d < s1 ? s0 + d : s1 - 1, ra[d], rb[d]);
  for (int64_t sb0 = s0; sb0 < s1; sb0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int64_t s = sb0 + d;
      const bool live = s < s1;
      const int buf = d & 1;   // kDepth is even: the buffers alternate step to step
      *reinterpret_cast<v8*>(&sa[buf][sr * RS + 8 * sc]) = live ? ra[d] : v8{};
#pragma unroll
      for (int i = 0; i < CTW; ++i) *reinterpret_cast<v8*>(&sb[buf][(sr + 64 * i) * RS + 8 * sc]) = rb[d][i];
      __syncthreads();
      fetch(s + kDepth < s1 ? s + kDepth : s1 - 1, ra[d], rb[d]);
      v8 av[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) av[ti] = *reinterpret_cast<const v8*>(&sa[buf][(16 * ti + r) * RS + 8 * g4]);
#pragma unroll
      for (int cj = 0; cj < CTW; ++cj)
        if (w + 4 * cj < CT) {
          const v8 bv = *reinterpret_cast<const v8*>(&sb[buf][(16 * (w + 4 * cj) + r) * RS + 8 * g4]);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) acc[ti][cj] = M::mma(av[ti], bv, acc[ti][cj]);
        }
    }
  }
  // accumulator lane (r, g4), element e of (ti, cj): token 16 ti + 4 g4 + e,
  // column 16 (w + 4 cj) + r
  float* part = p.part + grp * p.N * C;
#pragma unroll
  for (int cj = 0; cj < CTW; ++cj) {
    const int c = 16 * (w + 4 * cj) + r;
    if (c < C) {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = n0 + 16 * ti + 4 * g4 + e;
          if (n < p.N) part[n * C + c] = acc[ti][cj][e];
        }
    }
  }
}

// ------------------------------------------------------------ round
// out[n][c] = round(sum_g part[g][n][c]) for c < C; for C <= c < X,
// round(tail[n][c]) (the backward's B / C columns).  One thread per element.
template <Act A>
__global__ void __launch_bounds__(256) round_kernel(const float* __restrict__ part, const float* __restrict__ tail,
                                                    void* __restrict__ out, int64_t N, int C, int X, int G) {
  typedef typename Mfma<A>::elem elem;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= N * X) return;
  const int64_t n = i / X;
  const int c = static_cast<int>(i - n * X);
  float v;
  if (c < C) {
    v = part[n * C + c];
    for (int g = 1; g < G; ++g) v += part[(static_cast<int64_t>(g) * N + n) * C + c];
  } else {
    v = tail[i];
  }
  static_cast<elem*>(out)[i] = static_cast<elem>(v);
}

// ------------------------------------------------------------ expand
// Workgroup (64 tokens, cpb blocks of 256 channels): out[n][c] =
// sum_{k < kmax} x[n][k] w[c][k] (+ bias[c], rounded, when Fwd; else f32).
// x's 64 x kmax slice (zero past kmax) is staged in LDS once; for each
// channel block, wave w takes the channels c0 + 64 w .. (4 tiles) against the
// 4 token tiles, its w rows read straight in the matrix-core layout (shared
// by every token block, they stay in L2).  The next block's weights are
// requested before this block's results are stored (the memory counter is
// waited on in issue order), so the stores of one block overlap the loads
// of the next.  The accumulator holds 4 consecutive channels of one token per
// lane; each block's 64 x 256 tile goes through LDS to be written as whole
// rows.
template <Act A, bool Fwd>
__global__ void __launch_bounds__(kThr) expand_kernel(const ExpandArgs p) {
  using M = Mfma<A>;
  typedef typename M::elem elem;
  typedef typename M::v8 v8;
  typedef typename M::v4 v4;
  typedef typename M::f4 f4;
  constexpr int OS = Fwd ? 256 + 8 : 256 + 4;   // output tile row stride (elements)
  __shared__ __attribute__((aligned(16))) unsigned char so_raw[kTok * OS * (Fwd ? 2 : 4)];
  extern __shared__ __attribute__((aligned(16))) unsigned char sx_raw[];   // expand_x_lds_bytes(kmax)
  elem* sx = reinterpret_cast<elem*>(sx_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t CB = (p.Di + 255) / 256, GB = (CB + p.cpb - 1) / p.cpb;   // channel blocks, their groups
  const int64_t tb = blockIdx.x / GB, cb0 = (blockIdx.x % GB) * p.cpb;
  const int64_t cb1 = cb0 + p.cpb < CB ? cb0 + p.cpb : CB;
  const int64_t n0 = tb * kTok;
  const int kmax = p.kmax, KB = (kmax + 31) / 32;
  const int XS = 32 * KB + kPadE;   // staged x row stride (elements): 16 KB + 4 words, distinct banks per 16 lanes
  {
    // x[n0 .., :32 KB], zero past kmax and N
    const elem* x = static_cast<const elem*>(p.x);
    const int chunks = 4 * KB;
    for (int e = tid; e < kTok * chunks; e += kThr) {
      const int rr = e / chunks, ck = e - rr * chunks;
      v8 v{};
      if (n0 + rr < p.N && 8 * ck < kmax) v = *reinterpret_cast<const v8*>(x + (n0 + rr) * p.ldx + 8 * ck);
      *reinterpret_cast<v8*>(sx + rr * XS + 8 * ck) = v;
    }
  }
  const elem* wt = static_cast<const elem*>(p.w);
  // this wave's weights for k block kk of channel block cb (rows past Di:
  // the block's first row; k past kmax: the row's first 8, zeroed before use)
  auto fetch = [&](int64_t cb, int kk, v8(&d)[4]) {
    const int64_t cw = 256 * cb + 64 * w;
    const int64_t row = cw < p.Di ? cw + r : r;
    const int k = 32 * kk + 8 * g4 < kmax ? 32 * kk + 8 * g4 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = *reinterpret_cast<const v8*>(wt + (row + 16 * j) * p.ldw + k);
  };
  v8 a[4], an[4];
  fetch(cb0, 0, a);
  __syncthreads();
  for (int64_t cb = cb0; cb < cb1; ++cb) {
    const int64_t c0 = 256 * cb, cw = c0 + 64 * w;
    const int64_t cn = p.Di - c0 < 256 ? p.Di - c0 : 256;   // channels of this block (a multiple of 64)
    f4 acc[4][4];   // [channel tile j][token tile ti]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) acc[j][ti] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kk = 0; kk < KB; ++kk) {
      // the next weights: this block's next k block, else the next block's first
      if (kk + 1 < KB) fetch(cb, kk + 1, an);
      else if (cb + 1 < cb1) fetch(cb + 1, 0, an);
      v8 b[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) b[ti] = *reinterpret_cast<const v8*>(sx + (16 * ti + r) * XS + 32 * kk + 8 * g4);
      if (32 * kk + 32 > kmax) {   // only the last k block reaches past kmax
        const bool ok = 32 * kk + 8 * g4 < kmax;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = ok ? a[j] : v8{};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) acc[j][ti] = M::mma(a[j], b[ti], acc[j][ti]);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = an[j];
    }
    // lane (r, g4), element e of (j, ti): channel cw + 16 j + 4 g4 + e, token 16 ti + r
    if (cw < p.Di) {
      if (Fwd) {
        elem* so = reinterpret_cast<elem*>(so_raw);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 bias = *reinterpret_cast<const float4*>(p.bias + cw + 16 * j + 4 * g4);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            v4 o;
            o[0] = static_cast<elem>(acc[j][ti][0] + bias.x);
            o[1] = static_cast<elem>(acc[j][ti][1] + bias.y);
            o[2] = static_cast<elem>(acc[j][ti][2] + bias.z);
            o[3] = static_cast<elem>(acc[j][ti][3] + bias.w);
            *reinterpret_cast<v4*>(so + (16 * ti + r) * OS + 64 * w + 16 * j + 4 * g4) = o;
          }
        }
      } else {
        float* so = reinterpret_cast<float*>(so_raw);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti)
            *reinterpret_cast<float4*>(so + (16 * ti + r) * OS + 64 * w + 16 * j + 4 * g4) =
                make_float4(acc[j][ti][0], acc[j][ti][1], acc[j][ti][2], acc[j][ti][3]);
      }
    }
    __syncthreads();
    if (Fwd) {
      // 32 lanes x 16 bytes per token row
      const elem* so = reinterpret_cast<const elem*>(so_raw);
      for (int e = tid; e < kTok * 32; e += kThr) {
        const int rr = e >> 5, ck = e & 31;
        if (n0 + rr < p.N && 8 * ck < cn)
          *reinterpret_cast<v8*>(static_cast<elem*>(p.out) + (n0 + rr) * p.Di + c0 + 8 * ck) =
              *reinterpret_cast<const v8*>(so + rr * OS + 8 * ck);
      }
    } else {
      // 64 lanes x 16 bytes per token row
      const float* so = reinterpret_cast<const float*>(so_raw);
      for (int e = tid; e < kTok * 64; e += kThr) {
        const int rr = e >> 6, ck = e & 63;
        if (n0 + rr < p.N && 4 * ck < cn)
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (n0 + rr) * p.Di + c0 + 4 * ck) =
              *reinterpret_cast<const float4*>(so + rr * OS + 4 * ck);
      }
    }
    __syncthreads();   // the output tile is read before the next block writes it
  }
}

// out [C][ld] = in [Rw][C]^T (16-bit elements); columns Rw .. ld - 1 of out
// are zero.  32 x 32 tiles through LDS.
__global__ void __launch_bounds__(256) m_transpose_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                         int64_t Rw, int64_t C, int64_t ld) {
  __shared__ uint16_t t[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 32, c0 = static_cast<int64_t>(blockIdx.x) * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t rr = r0 + ty + i, c = c0 + tx;
    t[ty + i][tx] = (rr < Rw && c < C) ? in[rr * C + c] : uint16_t(0);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t c = c0 + ty + i, rr = r0 + tx;
    if (c < C && rr < ld) out[c * ld + rr] = t[tx][ty + i];
  }
}

hipError_t transpose16(const void* in, void* out, int64_t Rw, int64_t C, int64_t ld, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((C + 31) / 32), static_cast<unsigned>((ld + 31) / 32));
  hipLaunchKernelGGL(m_transpose_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(in),
                     static_cast<uint16_t*>(out), Rw, C, ld);
  return hipGetLastError();
}

template <Act A>
hipError_t launch_contract(const ContractArgs& c, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(((c.N + kTok - 1) / kTok) * c.G)), blk(kThr);
  switch ((((c.C + 15) / 16) + 3) / 4) {
    case 1: hipLaunchKernelGGL((contract_kernel<A, 1>), grid, blk, 0, st, c); break;
    case 2: hipLaunchKernelGGL((contract_kernel<A, 2>), grid, blk, 0, st, c); break;
    case 3: hipLaunchKernelGGL((contract_kernel<A, 3>), grid, blk, 0, st, c); break;
    default: hipLaunchKernelGGL((contract_kernel<A, 4>), grid, blk, 0, st, c); break;
  }
  return hipGetLastError();
}

template <Act A>
hipError_t launch_round(const float* part, const float* tail, void* out, int64_t N, int C, int X, int G,
                        hipStream_t st) {
  const int64_t n = N * X;
  hipLaunchKernelGGL((round_kernel<A>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, part, tail,
                     out, N, C, X, G);
  return hipGetLastError();
}

// dynamic LDS of an expand launch: x's staged 64 x kmax slice
size_t expand_x_lds_bytes(int kmax) { return static_cast<size_t>(kTok) * (32 * ((kmax + 31) / 32) + kPadE) * 2; }

// channel blocks per expand workgroup: about 384 workgroups (1.5 per
// compute unit), up to 4 blocks each; measured on the 130M and 2.8B widths
int64_t expand_cpb(int64_t N, int64_t Di) {
  const int64_t blocks = ((N + kTok - 1) / kTok) * ((Di + 255) / 256);
  int64_t c = blocks / 384;
  return c < 1 ? 1 : (c > 4 ? 4 : c);
}

template <Act A, bool Fwd>
hipError_t launch_expand(const ExpandArgs& e, hipStream_t st) {
  const int64_t CB = (e.Di + 255) / 256, GB = (CB + e.cpb - 1) / e.cpb;
  const dim3 grid(static_cast<unsigned>(((e.N + kTok - 1) / kTok) * GB)), blk(kThr);
  hipLaunchKernelGGL((expand_kernel<A, Fwd>), grid, blk, expand_x_lds_bytes(e.kmax), st, e);
  return hipGetLastError();
}

template <Act A>
hipError_t xdt_fwd(const XdtArgs& p, hipStream_t st) {
  int64_t kchunk = 1;
  const int64_t G = xdt_groups(p.N, p.Di, &kchunk);
  ContractArgs c;
  c.a = p.u;
  c.b = p.w_x;
  c.part = p.part;
  c.N = p.N;
  c.K = p.Di;
  c.C = p.X;
  c.G = G;
  c.kchunk = kchunk;
  hipError_t e = launch_contract<A>(c, st);
  if (e != hipSuccess) return e;
  e = launch_round<A>(p.part, nullptr, p.xdbl, p.N, p.X, p.X, static_cast<int>(G), st);
  if (e != hipSuccess) return e;
  ExpandArgs x;
  x.x = p.xdbl;
  x.ldx = p.X;
  x.kmax = p.R;
  x.w = p.w_dt;
  x.ldw = p.R;
  x.bias = p.b_dt;
  x.out = p.dr;
  x.N = p.N;
  x.Di = p.Di;
  x.cpb = expand_cpb(p.N, p.Di);
  return launch_expand<A, true>(x, st);
}

template <Act A>
hipError_t xdt_bwd(const XdtArgs& p, hipStream_t st) {
  const int64_t Xp = xdt_xT_stride(p.X);
  int64_t kchunk = 1;
  const int64_t G = xdt_groups(p.N, p.Di, &kchunk);
  ContractArgs c;
  c.a = p.d_dr;
  c.b = p.w_dtT;
  c.part = p.part;
  c.N = p.N;
  c.K = p.Di;
  c.C = p.R;
  c.G = G;
  c.kchunk = kchunk;
  hipError_t e = launch_contract<A>(c, st);
  if (e != hipSuccess) return e;
  e = launch_round<A>(p.part, p.d_xdbl, p.d_xdbl_a, p.N, p.R, p.X, static_cast<int>(G), st);
  if (e != hipSuccess) return e;
  ExpandArgs x;
  x.x = p.d_xdbl_a;
  x.ldx = p.X;
  x.kmax = p.X;
  x.w = p.w_xT;
  x.ldw = Xp;
  x.bias = nullptr;
  x.out = p.d_uex;
  x.N = p.N;
  x.Di = p.Di;
  x.cpb = expand_cpb(p.N, p.Di);
  return launch_expand<A, false>(x, st);
}

}  // namespace

int64_t xdt_groups(int64_t N, int64_t K, int64_t* kchunk) {
  const int64_t KS = K / 32, blocks = (N + kTok - 1) / kTok;
  int64_t G = (512 + blocks - 1) / blocks;
  const int64_t by_steps = KS / 4;   // at least 4 k steps per group
  G = G < by_steps ? G : by_steps;
  G = G < 1 ? 1 : G;
  const int64_t c = (KS + G - 1) / G;
  if (kchunk) *kchunk = c;
  return (KS + c - 1) / c;
}

bool xdt_supported(const XdtArgs& p, Act act) {
  return (act == Act::BF16 || act == Act::F16) && p.N >= 1 && p.Di >= 64 && p.Di % 64 == 0 && p.Di <= (1 << 24) &&
         p.R >= 8 && p.R % 8 == 0 && p.X % 8 == 0 && p.X > p.R && p.X <= kMaxX;
}

hipError_t launch_xdt_fwd(const XdtArgs& p, Act act, hipStream_t st) {
  return act == Act::BF16 ? xdt_fwd<Act::BF16>(p, st) : xdt_fwd<Act::F16>(p, st);
}

hipError_t launch_xdt_bwd_prep(const XdtArgs& p, Act, hipStream_t st) {
  // W_dt [Di][R] -> [R][Di]; W_x [X][Di] -> [Di][Xp], zero padded
  const hipError_t e = transpose16(p.w_dt, p.w_dtT, p.Di, p.R, p.Di, st);
  if (e != hipSuccess) return e;
  return transpose16(p.w_x, p.w_xT, p.X, p.Di, xdt_xT_stride(p.X), st);
}

hipError_t launch_xdt_bwd(const XdtArgs& p, Act act, hipStream_t st) {
  return act == Act::BF16 ? xdt_bwd<Act::BF16>(p, st) : xdt_bwd<Act::F16>(p, st);
}

}  // namespace mlayer
