// Kernels of the Mamba-1 layer around the scan core (gfx950): RMSNorm, the
// causal conv + SiLU of the x branch, the dt bias, casts and the
// fixed-order column reductions of the layer's parameter gradients.  The
// steps are those of the per-layer forward on the mamba-rs 0.3.1
// forward_mixed.rs page (F1 RMSNorm, F4a conv + SiLU, F4c dt bias) and their
// adjoints.  All of them stream HBM once; none needs LDS beyond a row
// reduction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layer_kernels.h"
#include "scan_common.h"

namespace mlayer {

using mscan::Act;
using mscan::IO;

namespace {

constexpr int kThreads = 256;

// sum over the 256 threads of a workgroup; every thread gets the result
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// Element of a [rows, Di] activation for a grid of rows * nchb workgroups,
// nchb = ceil(Di / 256) channel blocks per row: the row (and its step t)
// comes from one 32-bit division per workgroup, not a 64-bit one per
// element.  False past the last channel.
__device__ __forceinline__ bool row_channel(int64_t T, int64_t Di, unsigned nchb, int64_t* e, int64_t* i,
                                            int64_t* t) {
  const unsigned row = blockIdx.x / nchb;
  *i = static_cast<int64_t>(blockIdx.x - row * nchb) * kThreads + threadIdx.x;
  if (*i >= Di) return false;
  *t = static_cast<int64_t>(row % static_cast<unsigned>(T));
  *e = static_cast<int64_t>(row) * Di + *i;
  return true;
}

// F1: one workgroup per row
template <Act A>
__global__ void __launch_bounds__(kThreads) rmsnorm_fwd_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                              void* __restrict__ y, float* __restrict__ rstd,
                                                              int64_t dm, float eps) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * dm;
  float ss = 0.0f;
  for (int64_t j = threadIdx.x; j < dm; j += kThreads) ss = fmaf(xr[j], xr[j], ss);
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(dm) + eps);
  for (int64_t j = threadIdx.x; j < dm; j += kThreads) IO<A>::st(y, row * dm + j, xr[j] * r * w[j]);
  if (threadIdx.x == 0) rstd[row] = r;
}

// adjoint of F1 for one row: d_x = r w dy - x r^3 mean(dy w x);
// d_resid_in = d_resid_out + d_x (may alias)
__global__ void __launch_bounds__(kThreads) rmsnorm_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ rstd, const float* dres_out,
                                                              float* dres_in, int64_t dm) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const float* dyr = dy + row * dm;
  const float* xr = x + row * dm;
  float c = 0.0f;
  for (int64_t j = threadIdx.x; j < dm; j += kThreads) c = fmaf(dyr[j] * w[j], xr[j], c);
  c = block_sum(c, red) / static_cast<float>(dm);
  const float r = rstd[row];
  const float r3c = r * r * r * c;
  for (int64_t j = threadIdx.x; j < dm; j += kThreads) {
    const int64_t e = row * dm + j;
    dres_in[e] = dres_out[e] + (r * w[j] * dyr[j] - xr[j] * r3c);
  }
}

// part[blk, j] = sum over the rows of block blk of dy * x * rstd (the
// RMSNorm weight gradient), rows in ascending order
__global__ void __launch_bounds__(kThreads) rmsnorm_wgrad_part_kernel(const float* __restrict__ dy,
                                                                     const float* __restrict__ x,
                                                                     const float* __restrict__ rstd,
                                                                     float* __restrict__ part, int64_t rows,
                                                                     int64_t dm, int64_t rows_per_blk) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= dm) return;
  const int64_t blk = blockIdx.y;
  const int64_t r0 = blk * rows_per_blk;
  const int64_t r1 = r0 + rows_per_blk < rows ? r0 + rows_per_blk : rows;
  constexpr int U = 8;
  float acc = 0.0f;
  int64_t r = r0;
  for (; r + U <= r1; r += U) {   // eight rows' loads in flight, products added in row order
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = dy[(r + k) * dm + j] * x[(r + k) * dm + j] * rstd[r + k];
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  for (; r < r1; ++r) acc += dy[r * dm + j] * x[r * dm + j] * rstd[r];
  part[blk * dm + j] = acc;
}

// F4a: u = SiLU(b + sum_k w[i,k] x[t-K+1+k]) with zero history
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_silu_fwd_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ cw,
                                                                const float* __restrict__ cb, void* __restrict__ u,
                                                                int64_t T, int64_t Di, int K, unsigned nchb) {
  int64_t e, i, t;
  if (!row_channel(T, Di, nchb, &e, &i, &t)) return;
  float p = cb[i];
  for (int k = 0; k < K; ++k) {
    const int64_t back = K - 1 - k;   // tap k reads x_{t - back}
    if (t >= back) p = fmaf(cw[i * K + k], IO<A>::ld(x, e - back * Di), p);
  }
  IO<A>::st(u, e, p * sigmoid_f(p));
}

// adjoint of the SiLU: dp = (d_u + d_u_extra) * silu'(p), p recomputed
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_silu_dp_kernel(const void* __restrict__ x,
                                                               const float* __restrict__ cw,
                                                               const float* __restrict__ cb,
                                                               const void* __restrict__ du,
                                                               const float* __restrict__ du_extra,
                                                               float* __restrict__ dp, int64_t T, int64_t Di, int K,
                                                               unsigned nchb) {
  int64_t e, i, t;
  if (!row_channel(T, Di, nchb, &e, &i, &t)) return;
  float p = cb[i];
  for (int k = 0; k < K; ++k) {
    const int64_t back = K - 1 - k;
    if (t >= back) p = fmaf(cw[i * K + k], IO<A>::ld(x, e - back * Di), p);
  }
  const float s = sigmoid_f(p);
  dp[e] = (IO<A>::ld(du, e) + du_extra[e]) * (s * (1.0f + p * (1.0f - s)));
}

// adjoint of the conv for the input: d_x[s] = sum_k w[i,k] dp[s + K-1-k]
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_dx_kernel(const float* __restrict__ dp, const float* __restrict__ cw,
                                                          void* __restrict__ dx, int64_t T, int64_t Di, int K,
                                                          unsigned nchb) {
  int64_t e, i, t;
  if (!row_channel(T, Di, nchb, &e, &i, &t)) return;
  float g = 0.0f;
  for (int k = 0; k < K; ++k) {
    const int64_t ahead = K - 1 - k;   // dp_{t + ahead} read x_t through tap k
    if (t + ahead < T) g = fmaf(cw[i * K + k], dp[e + ahead * Di], g);
  }
  IO<A>::st(dx, e, g);
}

// conv weight / bias gradient partials over a block of steps of one batch
// row: part_w[(b, tb), i, k] = sum_t dp_t x_{t-K+1+k}, part_b[(b, tb), i] =
// sum_t dp_t; steps in ascending order
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_wgrad_part_kernel(const float* __restrict__ dp,
                                                                  const void* __restrict__ x,
                                                                  float* __restrict__ part_w,
                                                                  float* __restrict__ part_b, int64_t T, int64_t Di,
                                                                  int K, int64_t steps_per_blk, int64_t nblk_t) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= Di) return;
  const int64_t b = blockIdx.y / nblk_t, tb = blockIdx.y % nblk_t;
  const int64_t t0 = tb * steps_per_blk;
  const int64_t t1 = t0 + steps_per_blk < T ? t0 + steps_per_blk : T;
  float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float win[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // win[m] = x_{t-1-m} (zero before t = 0)
  for (int m = 0; m < 3; ++m)
    if (t0 - 1 - m >= 0) win[m] = IO<A>::ld(x, ((b * T) + t0 - 1 - m) * Di + i);
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t e = (b * T + t) * Di + i;
    const float xt = IO<A>::ld(x, e);
    const float g = dp[e];
    // tap k reads x_{t-(K-1-k)}: x_t for k = K-1, else win[K-2-k]
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < K) acc[k] = fmaf(g, k == K - 1 ? xt : win[K - 2 - k], acc[k]);
    acc[4] += g;
    win[2] = win[1];
    win[1] = win[0];
    win[0] = xt;
  }
  float* out = part_w + (static_cast<int64_t>(blockIdx.y) * Di + i) * K;
  for (int k = 0; k < K; ++k) out[k] = acc[k];
  part_b[static_cast<int64_t>(blockIdx.y) * Di + i] = acc[4];
}

// F4c tail: delta_raw = round(dt + b_dt[i])
template <Act A>
__global__ void __launch_bounds__(kThreads) bias_round_kernel(const float* __restrict__ dt,
                                                             const float* __restrict__ b, void* __restrict__ out,
                                                             int64_t T, int64_t Di, unsigned nchb) {
  int64_t e, i, t;
  if (!row_channel(T, Di, nchb, &e, &i, &t)) return;
  IO<A>::st(out, e, dt[e] + b[i]);
}

template <Act A>
__global__ void __launch_bounds__(kThreads) cast_kernel(const float* __restrict__ in, void* __restrict__ out,
                                                       int64_t n) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= n) return;
  IO<A>::st(out, e, in[e]);
}

// part[blk, j] = sum over the rows of block blk of m[r, j] (act dtype)
template <Act A>
__global__ void __launch_bounds__(kThreads) colpart_kernel(const void* __restrict__ m, float* __restrict__ part,
                                                          int64_t rows, int64_t cols, int64_t rows_per_blk) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= cols) return;
  const int64_t blk = blockIdx.y;
  const int64_t r0 = blk * rows_per_blk;
  const int64_t r1 = r0 + rows_per_blk < rows ? r0 + rows_per_blk : rows;
  constexpr int U = 8;
  float acc = 0.0f;
  int64_t r = r0;
  for (; r + U <= r1; r += U) {
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = IO<A>::ld(m, (r + k) * cols + j);
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  for (; r < r1; ++r) acc += IO<A>::ld(m, r * cols + j);
  part[blk * cols + j] = acc;
}

// out[j] += sum_{blk < nblk} part[blk, j], blocks in ascending order
__global__ void __launch_bounds__(kThreads) colsum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                         int64_t nblk, int64_t cols) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= cols) return;
  out[j] += mscan::ordered_sum(part + j, nblk, cols);
}

__global__ void __launch_bounds__(kThreads) zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e < n) p[e] = 0.0f;
}

dim3 grid1(int64_t n) { return dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)); }

// row-blocked elementwise launches: rows = n / cols, ceil(cols / 256) blocks per row
unsigned nchb(const Op& o) { return static_cast<unsigned>((o.cols + kThreads - 1) / kThreads); }
dim3 grid_rows(const Op& o) { return dim3(static_cast<unsigned>(o.n / o.cols) * nchb(o)); }

template <Act A>
hipError_t dispatch(const Op& o, hipStream_t st) {
  const dim3 blk(kThreads);
  switch (o.kind) {
    case OpKind::RmsnormFwd:
      hipLaunchKernelGGL(rmsnorm_fwd_kernel<A>, dim3(static_cast<unsigned>(o.rows)), blk, 0, st, o.f0, o.f1, o.v0,
                         o.f3, o.cols, o.eps);
      break;
    case OpKind::ConvSiluFwd:
      hipLaunchKernelGGL(conv_silu_fwd_kernel<A>, grid_rows(o), blk, 0, st, o.c0, o.f0, o.f1, o.v0, o.T, o.cols, o.K,
                         nchb(o));
      break;
    case OpKind::ConvSiluDp:
      hipLaunchKernelGGL(conv_silu_dp_kernel<A>, grid_rows(o), blk, 0, st, o.c0, o.f0, o.f1, o.c1, o.f2, o.f3, o.T,
                         o.cols, o.K, nchb(o));
      break;
    case OpKind::ConvDx:
      hipLaunchKernelGGL(conv_dx_kernel<A>, grid_rows(o), blk, 0, st, o.f0, o.f1, o.v0, o.T, o.cols, o.K, nchb(o));
      break;
    case OpKind::ConvWgradPart:
      hipLaunchKernelGGL(conv_wgrad_part_kernel<A>, dim3(grid1(o.cols).x, static_cast<unsigned>(o.nblk)), blk, 0, st,
                         o.f0, o.c0, o.f3, o.f6, o.T, o.cols, o.K, o.per_blk, o.nblk_t);
      break;
    case OpKind::BiasRound:
      hipLaunchKernelGGL(bias_round_kernel<A>, grid_rows(o), blk, 0, st, o.f0, o.f1, o.v0, o.T, o.cols, nchb(o));
      break;
    case OpKind::Cast:
      hipLaunchKernelGGL(cast_kernel<A>, grid1(o.n), blk, 0, st, o.f0, o.v0, o.n);
      break;
    case OpKind::ColPart:
      hipLaunchKernelGGL(colpart_kernel<A>, dim3(grid1(o.cols).x, static_cast<unsigned>(o.nblk)), blk, 0, st, o.c0,
                         o.f3, o.rows, o.cols, o.per_blk);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch(const Op& o, Act act, hipStream_t st) {
  const dim3 blk(kThreads);
  switch (o.kind) {   // dtype-free kernels
    case OpKind::RmsnormBwd:
      hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(static_cast<unsigned>(o.rows)), blk, 0, st, o.f0, o.f1, o.f2,
                         o.f4, o.f5, o.f3, o.cols);
      return hipGetLastError();
    case OpKind::RmsnormWgradPart:
      hipLaunchKernelGGL(rmsnorm_wgrad_part_kernel, dim3(grid1(o.cols).x, static_cast<unsigned>(o.nblk)), blk, 0, st,
                         o.f0, o.f1, o.f2, o.f3, o.rows, o.cols, o.per_blk);
      return hipGetLastError();
    case OpKind::ColSum:
      hipLaunchKernelGGL(colsum_kernel, grid1(o.cols), blk, 0, st, o.f0, o.f3, o.nblk, o.cols);
      return hipGetLastError();
    case OpKind::Zero:
      hipLaunchKernelGGL(zero_kernel, grid1(o.n), blk, 0, st, o.f3, o.n);
      return hipGetLastError();
    default:
      break;
  }
  switch (act) {
    case Act::F32: return dispatch<Act::F32>(o, st);
    case Act::BF16: return dispatch<Act::BF16>(o, st);
    case Act::F16: return dispatch<Act::F16>(o, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mlayer
