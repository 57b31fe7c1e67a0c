// The layer's skinny projections x_proj -> dt_proj fused on the matrix cores
// (gfx950, v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit activations.
//
// Steps F4b and F4c of the per-layer forward (mamba-rs 0.3.1
// src/mamba_ssm/gpu/forward_mixed.rs): xdbl = u W_x^T ([N, d_inner] x
// [d_inner, X], X = dt_rank + 2 d_state), then delta_raw = xdbl[:, :R] W_dt^T
// + b_dt ([N, R] x [R, d_inner]).  Both are thin: X is 80 or 192 columns over
// K = d_inner, then K = dt_rank.  The work is bound by HBM (u read once,
// delta_raw written once), so one workgroup takes 16 token rows through both
// products: the xdbl rows stay on chip, rounded to the activation dtype where
// the product would store them.  The backward fuses the adjoint the same way:
// d_xdbl[:, :R] = d_delta_raw W_dt, the whole d_xdbl row rounded (its B / C
// columns come from the core), then d_u_extra = d_xdbl W_x.
//
// Matrix-core tile: one instruction multiplies A (16 x 32; lane l holds row
// l % 16, k = 8 (l / 16) .. + 7) by B (32 x 16; column l % 16, the same k)
// into a 16 x 16 f32 accumulator whose lane l holds rows 4 (l / 16) + e,
// column l % 16.  Loading that layout straight from row-major memory puts
// neighbouring lanes on different rows (one cache line per lane), so every
// operand is loaded coalesced instead (lane l: row l / 4, 16 bytes at k =
// 8 (l % 4)) and moved to its matrix-core lane with a cross-lane permute.
//
// First product (K = d_inner, few columns): the 8 waves of a workgroup split
// K (wave w takes the 32-wide k steps w, w + 8, ...) and each keeps every
// column tile of its 16 rows; the 8 partial tiles meet in LDS and are added
// in wave order, so the result does not depend on timing.  Operand rows past
// the matrix (the last token tile, the last column tile) are clamped to its
// last row, which keeps the loads branch-free; their products are dropped.
// Second product (K <= 256, d_inner columns): waves take groups of 4 channel
// tiles (64 channels) with the weight rows as A and the on-chip rows as B, so
// a lane ends with 4 consecutive channels of one token; the wave's 16 x 64
// tile goes through LDS so that the stores cover whole 128-byte (256-byte in
// f32) row segments, 16 bytes per lane (stores of scattered 8-byte pieces
// reach a fraction of the write bandwidth).  The
// backward reads W_dt and W_x transposed (each lane's 8 k values contiguous);
// a tiled transpose writes those copies per call.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layer_kernels.h"
#include "scan_common.h"

namespace mlayer {
namespace {

using mscan::Act;

constexpr int kRows = 16;          // token rows per workgroup
constexpr int kWaves = 8;
constexpr int kThr = 64 * kWaves;
constexpr int kMaxX = 256;         // longest xdbl row (dt_rank + 2 d_state) taken
constexpr int kSx = kMaxX + 8;     // row stride of the on-chip rows (elements)
constexpr int kGroup = 4;          // channel tiles per wave pass of the second product
constexpr int kSt16 = 64 + 8;      // row stride (elements) of a wave's 16-bit output tile
constexpr int kSt32 = 64 + 4;      // row stride (floats) of a wave's f32 output tile

// LDS floats of a workgroup: the partial tiles, reused for the output tiles
template <int CTM, bool F32Out>
constexpr int lds_floats() {
  constexpr int red = kWaves * kRows * (16 * CTM + 4);
  constexpr int st = F32Out ? kWaves * kRows * kSt32 : kWaves * kRows * kSt16 / 2;
  return red > st ? red : st;
}

// the wave's index in the workgroup, in a scalar register (loops over it
// stay uniform: scalar branches, unrollable)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// orders a wave's LDS stores before its loads of other lanes' data
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

template <Act A>
__device__ __forceinline__ typename Mfma<A>::v8 ld8(const typename Mfma<A>::elem* p) {
  return *reinterpret_cast<const typename Mfma<A>::v8*>(p);
}

// The permute: lane L = r + 16 g takes the 16 bytes that lane 4 r + g loaded
// (row r, k chunk g).  src_byte = 4 (4 (L % 16) + L / 16).
template <class V>
__device__ __forceinline__ V to_mfma(const V& v, int src_byte) {
  union U {
    V v;
    int i[4];
  };
  U in, out;
  in.v = v;
#pragma unroll
  for (int i = 0; i < 4; ++i) out.i[i] = __builtin_amdgcn_ds_bpermute(src_byte, in.i[i]);
  return out.v;
}

__device__ __forceinline__ int mfma_src_byte(int lane) { return (((lane & 15) << 2) | (lane >> 4)) << 2; }

template <Act A>
__device__ __forceinline__ typename Mfma<A>::elem round_to(float v) {
  return static_cast<typename Mfma<A>::elem>(v);   // round to nearest even
}

// Partial product of the first (K = d_inner) product: 16 rows of Am [., K]
// (rows from row0, clamped to N - 1) times the rows of Bm [ncols, K] (clamped
// to ncols - 1), k steps w, w + 8, ...; the wave's 16 x (16 CTM) tile goes to
// red [16][S].
template <Act A, int CTM>
__device__ __forceinline__ void skinny_partial(const typename Mfma<A>::elem* Am, const typename Mfma<A>::elem* Bm,
                                               int64_t N, int64_t K, int ncols, int64_t row0, float* red, int S) {
  using M = Mfma<A>;
  typedef typename M::v8 v8;
  typedef typename M::f4 f4;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int r = lane & 15, g = lane >> 4;      // matrix-core layout
  const int lr = lane >> 2, lc = lane & 3;     // coalesced load: row lr, k chunk lc
  const int src = mfma_src_byte(lane);
  const int64_t arow = row0 + lr < N ? row0 + lr : N - 1;
  const typename M::elem* ap = Am + arow * K + 8 * lc;
  int boff[CTM];
#pragma unroll
  for (int ct = 0; ct < CTM; ++ct) {
    const int c = 16 * ct + lr;
    boff[ct] = static_cast<int>((c < ncols ? c : ncols - 1) * K) + 8 * lc;
  }
  f4 acc[CTM];
#pragma unroll
  for (int ct = 0; ct < CTM; ++ct) acc[ct] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  const int KS = static_cast<int>(K / 32);
  // operands of the next k step are requested before this one's products
  v8 a, b[CTM], an, bn[CTM];
  if (w < KS) {
    a = ld8<A>(ap + 32 * w);
#pragma unroll
    for (int ct = 0; ct < CTM; ++ct) b[ct] = ld8<A>(Bm + boff[ct] + 32 * w);
  }
  for (int ks = w; ks < KS; ks += kWaves) {
    const int kn = ks + kWaves;
    if (kn < KS) {
      an = ld8<A>(ap + 32 * kn);
#pragma unroll
      for (int ct = 0; ct < CTM; ++ct) bn[ct] = ld8<A>(Bm + boff[ct] + 32 * kn);
    }
    const v8 am = to_mfma(a, src);
#pragma unroll
    for (int ct = 0; ct < CTM; ++ct) acc[ct] = M::mma(am, to_mfma(b[ct], src), acc[ct]);
    a = an;
#pragma unroll
    for (int ct = 0; ct < CTM; ++ct) b[ct] = bn[ct];
  }
#pragma unroll
  for (int ct = 0; ct < CTM; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(4 * g + e) * S + 16 * ct + r] = acc[ct][e];
}

// Second product for this wave: out[row0 + token][c] = sum_k sx[token][k]
// W[c][k] over k < kmax (K blocks of 32; W's rows ldw elements, ldw and kmax
// multiples of 8), for the channel groups t0 = 4 w,
// 4 w + 32, ... (4 tiles of 16 channels each).  Fwd: + bias[c], rounded to
// the activation dtype; else f32.  Pipelined one (group, k block) ahead: the
// next operands are requested before the current tile's stores, because the
// memory counter is waited on in issue order and a wait for loads issued
// after a store would also wait for the store.
template <Act A, bool Fwd>
__device__ __forceinline__ void expand_stage(const typename Mfma<A>::elem (*sx)[kSx], const typename Mfma<A>::elem* W,
                                             int64_t ldw, int kmax, int KB, const float* bias, void* out, int64_t Di,
                                             int64_t N, int64_t row0, float* lds_wave) {
  using M = Mfma<A>;
  typedef typename M::elem elem;
  typedef typename M::v8 v8;
  typedef typename M::v4 v4;
  typedef typename M::f4 f4;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int r = lane & 15, g = lane >> 4;
  const int lr = lane >> 2, lc = lane & 3, src = mfma_src_byte(lane);
  const int64_t CT = Di / 16;
  const int64_t ngr = CT > kGroup * w ? (CT - kGroup * w + kGroup * kWaves - 1) / (kGroup * kWaves) : 0;
  const int64_t nit = ngr * KB;
  if (nit == 0) return;
  auto load_a = [&](int64_t m, int kk, v8(&a)[kGroup]) {
    const int64_t t0 = kGroup * (w + kWaves * m);
    const int k = 32 * kk + 8 * lc;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int64_t t = t0 + j < CT ? t0 + j : CT - 1;
      // k past kmax: a valid address (the value is zeroed where it is used)
      a[j] = ld8<A>(W + (16 * t + lr) * ldw + (k < kmax ? k : 0));
    }
  };
  auto load_bias = [&](int64_t m, float4(&b)[kGroup]) {
    const int64_t t0 = kGroup * (w + kWaves * m);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int64_t t = t0 + j < CT ? t0 + j : CT - 1;
      b[j] = *reinterpret_cast<const float4*>(bias + 16 * t + 4 * g);
    }
  };
  v8 a[kGroup], an[kGroup];
  float4 bs[kGroup], bn[kGroup];
  load_a(0, 0, a);
  if (Fwd) load_bias(0, bs);
  f4 acc[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) acc[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  int64_t m = 0;
  int kk = 0;
  for (int64_t it = 0; it < nit; ++it) {
    int64_t m1 = m;
    int kk1 = kk + 1;
    if (kk1 == KB) {
      kk1 = 0;
      ++m1;
    }
    if (it + 1 < nit) {
      load_a(m1, kk1, an);
      if (Fwd && kk1 == 0) load_bias(m1, bn);
    }
    const v8 b = *reinterpret_cast<const v8*>(&sx[r][32 * kk + 8 * g]);
    const bool kok = 32 * kk + 8 * lc < kmax;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) acc[j] = M::mma(to_mfma(kok ? a[j] : v8{}, src), b, acc[j]);
    if (kk == KB - 1) {
      // the 16 x 64 tile (token r, channels 16 j + 4 g ..) through this
      // wave's LDS, then whole row segments
      const int64_t t0 = kGroup * (w + kWaves * m);
      if (Fwd) {
        elem* st = reinterpret_cast<elem*>(lds_wave);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          v4 o;
          o[0] = round_to<A>(acc[j][0] + bs[j].x);
          o[1] = round_to<A>(acc[j][1] + bs[j].y);
          o[2] = round_to<A>(acc[j][2] + bs[j].z);
          o[3] = round_to<A>(acc[j][3] + bs[j].w);
          *reinterpret_cast<v4*>(st + r * kSt16 + 16 * j + 4 * g) = o;
        }
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tr = (lane >> 3) + 8 * h, ck = lane & 7;   // token row, 8-channel chunk
          const v8 o = *reinterpret_cast<const v8*>(st + tr * kSt16 + 8 * ck);
          if (row0 + tr < N && t0 + (ck >> 1) < CT)
            *reinterpret_cast<v8*>(static_cast<elem*>(out) + (row0 + tr) * Di + 16 * t0 + 8 * ck) = o;
        }
      } else {
        float* st = lds_wave;
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          *reinterpret_cast<float4*>(st + r * kSt32 + 16 * j + 4 * g) =
              make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int tr = (lane >> 4) + 4 * h, ck = lane & 15;   // token row, 4-channel chunk
          const float4 o = *reinterpret_cast<const float4*>(st + tr * kSt32 + 4 * ck);
          if (row0 + tr < N && t0 + (ck >> 2) < CT)
            *reinterpret_cast<float4*>(static_cast<float*>(out) + (row0 + tr) * Di + 16 * t0 + 4 * ck) = o;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        acc[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        if (Fwd) bs[j] = bn[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) a[j] = an[j];
    m = m1;
    kk = kk1;
  }
}

// ------------------------------------------------------------ forward
template <Act A, int CTM>
__global__ void __launch_bounds__(kThr) xdt_fwd_kernel(const XdtArgs p) {
  using M = Mfma<A>;
  typedef typename M::elem elem;
  typedef typename M::v8 v8;
  typedef typename M::v4 v4;
  typedef typename M::f4 f4;
  constexpr int S = 16 * CTM + 4;   // partial row stride (floats): 4 g-groups land on distinct banks
  __shared__ __attribute__((aligned(16))) float lds[lds_floats<CTM, false>()];
  __shared__ __attribute__((aligned(16))) elem sx[kRows][kSx];   // rounded xdbl[:, :R], zero past R
  float(*red)[kRows * S] = reinterpret_cast<float(*)[kRows * S]>(lds);
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r = lane & 15, g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t N = p.N, Di = p.Di;
  const int X = p.X, R = p.R;
  const elem* u = static_cast<const elem*>(p.u);
  const elem* w_x = static_cast<const elem*>(p.w_x);
  const elem* w_dt = static_cast<const elem*>(p.w_dt);
  for (int e = tid; e < kRows * kSx; e += kThr)
    if (e % kSx >= R) sx[e / kSx][e % kSx] = round_to<A>(0.0f);
  // xdbl = u W_x^T, k split over the waves
  skinny_partial<A, CTM>(u, w_x, N, Di, X, row0, red[w], S);
  __syncthreads();
  for (int e = tid; e < kRows * X; e += kThr) {
    const int lr = e / X, c = e % X;
    float s = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += red[ww][lr * S + c];
    const elem v = round_to<A>(s);
    if (c < R) sx[lr][c] = v;
    if (row0 + lr < N) static_cast<elem*>(p.xdbl)[(row0 + lr) * X + c] = v;
  }
  __syncthreads();
  // delta_raw = round(xdbl[:, :R] W_dt^T + b_dt): A = W_dt rows (channels),
  // B = the on-chip rows (tokens)
  expand_stage<A, true>(sx, w_dt, R, R, (R + 31) / 32, p.b_dt, p.dr, Di, N, row0, lds + w * (kRows * kSt16 / 2));
}

// ------------------------------------------------------------ backward
template <Act A, int CTM>
__global__ void __launch_bounds__(kThr) xdt_bwd_kernel(const XdtArgs p) {
  using M = Mfma<A>;
  typedef typename M::elem elem;
  typedef typename M::v8 v8;
  typedef typename M::f4 f4;
  constexpr int S = 16 * CTM + 4;
  __shared__ __attribute__((aligned(16))) float lds[lds_floats<CTM, true>()];
  __shared__ __attribute__((aligned(16))) elem sx[kRows][kSx];   // rounded d_xdbl rows, zero past X
  float(*red)[kRows * S] = reinterpret_cast<float(*)[kRows * S]>(lds);
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r = lane & 15, g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t N = p.N, Di = p.Di;
  const int X = p.X, R = p.R;
  const int Xp = static_cast<int>(xdt_xT_stride(X));
  // the B / C columns of d_xdbl (the core's sums, f32), rounded
  for (int e = tid; e < kRows * kSx; e += kThr) {
    const int lr = e / kSx, c = e % kSx;
    if (c >= R) {
      float v = 0.0f;
      if (c < X && row0 + lr < N) v = p.d_xdbl[(row0 + lr) * X + c];
      sx[lr][c] = round_to<A>(v);
    }
  }
  // d_xdbl[:, :R] = d_delta_raw W_dt (rows of W_dt^T, [R][Di]), k split over the waves
  skinny_partial<A, CTM>(static_cast<const elem*>(p.d_dr), static_cast<const elem*>(p.w_dtT), N, Di, R, row0,
                         red[w], S);
  __syncthreads();
  for (int e = tid; e < kRows * R; e += kThr) {
    const int lr = e / R, c = e % R;
    float s = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += red[ww][lr * S + c];
    sx[lr][c] = round_to<A>(s);
  }
  __syncthreads();
  // the rounded d_xdbl rows are the x_proj weight product's operand
  for (int e = tid; e < kRows * X; e += kThr) {
    const int lr = e / X, c = e % X;
    if (row0 + lr < N) static_cast<elem*>(p.d_xdbl_a)[(row0 + lr) * X + c] = sx[lr][c];
  }
  // d_u_extra = d_xdbl W_x, f32: A = W_x^T rows (channels, zero padded to
  // Xp), B = the on-chip rows (tokens)
  expand_stage<A, false>(sx, static_cast<const elem*>(p.w_xT), Xp, Xp, (X + 31) / 32, nullptr, p.d_uex, Di, N, row0,
                         lds + w * (kRows * kSt32));
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

// column tiles a workgroup keeps for the first product: ceil(cols / 16)
// rounded up to an instantiated count
int col_tiles(int cols) {
  const int ct = (cols + 15) / 16;
  if (ct <= 2) return 2;
  if (ct <= 4) return 4;
  if (ct <= 6) return 6;
  if (ct <= 8) return 8;
  if (ct <= 12) return 12;
  return 16;
}

template <Act A>
hipError_t launch_fwd(const XdtArgs& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((p.N + kRows - 1) / kRows)), blk(kThr);
  switch (col_tiles(p.X)) {
    case 2: hipLaunchKernelGGL((xdt_fwd_kernel<A, 2>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((xdt_fwd_kernel<A, 4>), grid, blk, 0, st, p); break;
    case 6: hipLaunchKernelGGL((xdt_fwd_kernel<A, 6>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((xdt_fwd_kernel<A, 8>), grid, blk, 0, st, p); break;
    case 12: hipLaunchKernelGGL((xdt_fwd_kernel<A, 12>), grid, blk, 0, st, p); break;
    default: hipLaunchKernelGGL((xdt_fwd_kernel<A, 16>), grid, blk, 0, st, p); break;
  }
  return hipGetLastError();
}

template <Act A>
hipError_t launch_bwd(const XdtArgs& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((p.N + kRows - 1) / kRows)), blk(kThr);
  switch (col_tiles(p.R)) {
    case 2: hipLaunchKernelGGL((xdt_bwd_kernel<A, 2>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((xdt_bwd_kernel<A, 4>), grid, blk, 0, st, p); break;
    case 6: hipLaunchKernelGGL((xdt_bwd_kernel<A, 6>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((xdt_bwd_kernel<A, 8>), grid, blk, 0, st, p); break;
    case 12: hipLaunchKernelGGL((xdt_bwd_kernel<A, 12>), grid, blk, 0, st, p); break;
    default: hipLaunchKernelGGL((xdt_bwd_kernel<A, 16>), grid, blk, 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace

bool xdt_supported(const XdtArgs& p, Act act) {
  return (act == Act::BF16 || act == Act::F16) && p.N >= 1 && p.Di >= 32 && p.Di % 32 == 0 && p.Di <= (1 << 22) &&
         p.R >= 8 && p.R % 8 == 0 &&
         p.X > p.R && p.X <= kMaxX;
}

hipError_t launch_xdt_fwd(const XdtArgs& p, Act act, hipStream_t st) {
  return act == Act::BF16 ? launch_fwd<Act::BF16>(p, st) : launch_fwd<Act::F16>(p, st);
}

hipError_t launch_xdt_bwd(const XdtArgs& p, Act act, hipStream_t st) {
  // W_dt [Di][R] -> [R][Di]; W_x [X][Di] -> [Di][Xp], zero padded
  hipError_t e = transpose16(p.w_dt, p.w_dtT, p.Di, p.R, p.Di, st);
  if (e != hipSuccess) return e;
  e = transpose16(p.w_x, p.w_xT, p.X, p.Di, xdt_xT_stride(p.X), st);
  if (e != hipSuccess) return e;
  return act == Act::BF16 ? launch_bwd<Act::BF16>(p, st) : launch_bwd<Act::F16>(p, st);
}

}  // namespace mlayer
