// Kernels of the Mamba-1 layer around the scan core (gfx950): RMSNorm, the
// causal conv + SiLU of the x branch, the dt bias, casts and the
// fixed-order column reductions of the layer's parameter gradients.  The
// steps are those of the per-layer forward on the mamba-rs 0.3.1
// forward_mixed.rs page (F1 RMSNorm, F4a conv + SiLU, F4c dt bias) and their
// adjoints.  All of them stream HBM once; none uses LDS beyond the 1 KB
// that the final column sums add their runs in.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layer_kernels.h"
#include "scan_common.h"

namespace mlayer {

using mscan::Act;
using mscan::IO;

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // row kernels: one wave per row
constexpr int kRowU = 4;                       // row kernels: loads in flight per lane and array

// sum over the 64 lanes of a wave; every lane gets the result
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Four f32 values to elements e .. e+3 of an activation (e % 4 == 0, the
// buffer 16-byte aligned), converted as IO<A>::st converts one.
template <Act A>
__device__ __forceinline__ void st4(void* p, int64_t e, float4 v);
template <>
__device__ __forceinline__ void st4<Act::F32>(void* p, int64_t e, float4 v) {
  *reinterpret_cast<float4*>(static_cast<float*>(p) + e) = v;
}
template <>
__device__ __forceinline__ void st4<Act::BF16>(void* p, int64_t e, float4 v) {
  struct alignas(8) H4 {
    __bf16 h[4];
  };
  const H4 q = {{static_cast<__bf16>(v.x), static_cast<__bf16>(v.y), static_cast<__bf16>(v.z), static_cast<__bf16>(v.w)}};
  *reinterpret_cast<H4*>(static_cast<__bf16*>(p) + e) = q;
}
template <>
__device__ __forceinline__ void st4<Act::F16>(void* p, int64_t e, float4 v) {
  struct alignas(8) H4 {
    _Float16 h[4];
  };
  const H4 q = {{static_cast<_Float16>(v.x), static_cast<_Float16>(v.y), static_cast<_Float16>(v.z),
                 static_cast<_Float16>(v.w)}};
  *reinterpret_cast<H4*>(static_cast<_Float16*>(p) + e) = q;
}

// F1: one wave per row (lane l takes columns l, l + 64, ...), kRowsPerBlock
// rows per workgroup; no workgroup barrier, so a wave past the last row
// simply exits
template <Act A>
__global__ void __launch_bounds__(kThreads) rmsnorm_fwd_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                              void* __restrict__ y, float* __restrict__ rstd,
                                                              int64_t rows, int64_t dm, float eps) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* xr = x + row * dm;
  float ss = 0.0f;
  for (int64_t j0 = lane; j0 < dm; j0 += kRowU * 64) {
    float xv[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) xv[k] = j0 + 64 * k < dm ? xr[j0 + 64 * k] : 0.0f;
#pragma unroll
    for (int k = 0; k < kRowU; ++k) ss = fmaf(xv[k], xv[k], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(dm) + eps);
  for (int64_t j0 = lane; j0 < dm; j0 += kRowU * 64) {
    float xv[kRowU], wv[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const bool in = j0 + 64 * k < dm;
      xv[k] = in ? xr[j0 + 64 * k] : 0.0f;
      wv[k] = in ? w[j0 + 64 * k] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kRowU; ++k)
      if (j0 + 64 * k < dm) IO<A>::st(y, row * dm + j0 + 64 * k, xv[k] * r * wv[k]);
  }
  if (lane == 0) rstd[row] = r;
}

// adjoint of F1 for one row: d_x = r w dy - x r^3 mean(dy w x);
// d_resid_in = d_resid_out + d_x (may alias: each element is read and then
// written by the same lane).  Rows are mapped as in the forward.
__global__ void __launch_bounds__(kThreads) rmsnorm_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ rstd, const float* dres_out,
                                                              float* dres_in, int64_t rows, int64_t dm) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* dyr = dy + row * dm;
  const float* xr = x + row * dm;
  float c = 0.0f;
  for (int64_t j0 = lane; j0 < dm; j0 += kRowU * 64) {
    float gv[kRowU], wv[kRowU], xv[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const bool in = j0 + 64 * k < dm;
      gv[k] = in ? dyr[j0 + 64 * k] : 0.0f;
      wv[k] = in ? w[j0 + 64 * k] : 0.0f;
      xv[k] = in ? xr[j0 + 64 * k] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kRowU; ++k) c = fmaf(gv[k] * wv[k], xv[k], c);
  }
  c = wave_sum(c) / static_cast<float>(dm);
  const float r = rstd[row];
  const float r3c = r * r * r * c;
  for (int64_t j0 = lane; j0 < dm; j0 += kRowU * 64) {
    float gv[kRowU], wv[kRowU], xv[kRowU], ov[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const bool in = j0 + 64 * k < dm;
      const int64_t e = row * dm + j0 + 64 * k;
      gv[k] = in ? dyr[j0 + 64 * k] : 0.0f;
      wv[k] = in ? w[j0 + 64 * k] : 0.0f;
      xv[k] = in ? xr[j0 + 64 * k] : 0.0f;
      ov[k] = in ? dres_out[e] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kRowU; ++k)
      if (j0 + 64 * k < dm) dres_in[row * dm + j0 + 64 * k] = ov[k] + (r * wv[k] * gv[k] - xv[k] * r3c);
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
  constexpr int U = 16;
  float acc = 0.0f;
  int64_t r = r0;
  for (; r + U <= r1; r += U) {   // sixteen rows' loads in flight, products added in row order
    float v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = dy[(r + k) * dm + j] * x[(r + k) * dm + j] * rstd[r + k];
#pragma unroll
    for (int k = 0; k < U; ++k) acc += v[k];
  }
  for (; r < r1; ++r) acc += dy[r * dm + j] * x[r * dm + j] * rstd[r];
  part[blk * dm + j] = acc;
}

// Tiles of the conv kernels: a workgroup walks kConvTT steps of one batch
// row for 256 channels, the conv window in registers, so each input is read
// once (plus a K-1 step halo).  Block id = (b * ntb + tb) * nchb + channel
// block, ntb = ceil(T / kConvTT).
constexpr int kConvTT = 64;
constexpr int kConvU = 8;   // steps whose inputs are loaded together

struct ConvTile {
  int64_t b, t0, t1, i;
};

__device__ __forceinline__ bool conv_tile(int64_t T, int64_t Di, unsigned nchb, unsigned ntb, ConvTile* c) {
  const unsigned cbk = blockIdx.x % nchb, rest = blockIdx.x / nchb;
  c->i = static_cast<int64_t>(cbk) * kThreads + threadIdx.x;
  if (c->i >= Di) return false;
  c->b = rest / ntb;
  c->t0 = static_cast<int64_t>(rest % ntb) * kConvTT;
  c->t1 = c->t0 + kConvTT < T ? c->t0 + kConvTT : T;
  return true;
}

// F4a: u_t = SiLU(b + sum_k w[i,k] x_{t-(K-1-k)}), zero history.  win[m] holds
// x_{t-1-m}; tap k < K-1 reads win[K-2-k], tap K-1 reads x_t.
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_silu_fwd_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ cw,
                                                                const float* __restrict__ cb, void* __restrict__ u,
                                                                int64_t T, int64_t Di, int K, unsigned nchb,
                                                                unsigned ntb) {
  ConvTile c;
  if (!conv_tile(T, Di, nchb, ntb, &c)) return;
  float w[4] = {0.0f, 0.0f, 0.0f, 0.0f}, win[3] = {0.0f, 0.0f, 0.0f};
  for (int k = 0; k < K; ++k) w[k] = cw[c.i * K + k];
  const float bias = cb[c.i];
  const int64_t base = c.b * T * Di + c.i;
  for (int m = 0; m < K - 1; ++m)
    if (c.t0 - 1 - m >= 0) win[m] = IO<A>::ld(x, base + (c.t0 - 1 - m) * Di);
  // kConvU steps' inputs are loaded before any is used (addresses clamped to
  // the tile, so every load is unconditional): several loads in flight per
  // thread instead of one round trip per step
  for (int64_t t0 = c.t0; t0 < c.t1; t0 += kConvU) {
    float xs[kConvU];
#pragma unroll
    for (int j = 0; j < kConvU; ++j) xs[j] = IO<A>::ld(x, base + (t0 + j < c.t1 ? t0 + j : c.t1 - 1) * Di);
#pragma unroll
    for (int j = 0; j < kConvU; ++j) {
      if (t0 + j < c.t1) {
        const float xt = xs[j];
        float p = fmaf(w[K - 1], xt, bias);
#pragma unroll
        for (int k = 0; k < 3; ++k)
          if (k < K - 1) p = fmaf(w[k], win[K - 2 - k], p);
        IO<A>::st(u, base + (t0 + j) * Di, p * mscan::sigmoid(p));
        win[2] = win[1];
        win[1] = win[0];
        win[0] = xt;
      }
    }
  }
}

// Adjoint of F4a in one pass over a tile, forward in time:
//   dp_t   = (d_u_t + d_u_extra_t) * silu'(p_t)          (p_t recomputed)
//   d_x_s  = sum_k w[i,k] dp_{s+K-1-k}, emitted at t = s + K-1 as
//            sum_k w[i,k] dp_{t-k} (dpw[k] holds dp_{t-k})
//   part_w[blk, i, k] = sum_t dp_t x_{t-(K-1-k)},  part_b[blk, i] = sum_t dp_t
// The K-1 steps after the tile are recomputed for the d_x of its last steps
// (they enter no weight partial); past the sequence end dp is zero.
template <Act A>
__global__ void __launch_bounds__(kThreads) conv_bwd_kernel(const void* __restrict__ x, const float* __restrict__ cw,
                                                           const float* __restrict__ cb, const void* __restrict__ du,
                                                           const float* __restrict__ du_extra,
                                                           void* __restrict__ dx, float* __restrict__ part_w,
                                                           float* __restrict__ part_b, int64_t T, int64_t Di, int K,
                                                           unsigned nchb, unsigned ntb) {
  ConvTile c;
  if (!conv_tile(T, Di, nchb, ntb, &c)) return;
  float w[4] = {0.0f, 0.0f, 0.0f, 0.0f}, win[3] = {0.0f, 0.0f, 0.0f}, dpw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, acc_b = 0.0f;
  for (int k = 0; k < K; ++k) w[k] = cw[c.i * K + k];
  const float bias = cb[c.i];
  const int64_t base = c.b * T * Di + c.i;
  for (int m = 0; m < K - 1; ++m)
    if (c.t0 - 1 - m >= 0) win[m] = IO<A>::ld(x, base + (c.t0 - 1 - m) * Di);
  const int64_t t_stop = c.t1 + (K - 1);                  // last emitted d_x is step t1 - 1
  const int64_t t_data = t_stop < T ? t_stop : T;          // steps with data
  for (int64_t t0 = c.t0; t0 < t_stop; t0 += kConvU) {
    // kConvU steps' inputs first (clamped to the data, so unconditional)
    float xs[kConvU], gs[kConvU];
#pragma unroll
    for (int j = 0; j < kConvU; ++j) {
      const int64_t e = base + (t0 + j < t_data ? t0 + j : t_data - 1) * Di;
      xs[j] = IO<A>::ld(x, e);
      gs[j] = IO<A>::ld(du, e) + du_extra[e];
    }
#pragma unroll
    for (int j = 0; j < kConvU; ++j) {
      const int64_t t = t0 + j;
      if (t >= t_stop) break;
      float g = 0.0f;
      if (t < t_data) {
        const float xt = xs[j];
        float p = fmaf(w[K - 1], xt, bias);
#pragma unroll
        for (int k = 0; k < 3; ++k)
          if (k < K - 1) p = fmaf(w[k], win[K - 2 - k], p);
        const float sg = mscan::sigmoid(p);
        g = gs[j] * (sg * (1.0f + p * (1.0f - sg)));
        if (t < c.t1) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (k < K) acc[k] = fmaf(g, k == K - 1 ? xt : win[K - 2 - k], acc[k]);
          acc_b += g;
        }
        win[2] = win[1];
        win[1] = win[0];
        win[0] = xt;
      }
      dpw[3] = dpw[2];
      dpw[2] = dpw[1];
      dpw[1] = dpw[0];
      dpw[0] = g;
      const int64_t s = t - (K - 1);
      if (s >= c.t0 && s < T) {
        float gx = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < K) gx = fmaf(w[k], dpw[k], gx);
        IO<A>::st(dx, base + s * Di, gx);
      }
    }
  }
  const int64_t blk = static_cast<int64_t>(blockIdx.x / nchb);   // b * ntb + tb
  for (int k = 0; k < K; ++k) part_w[(blk * Di + c.i) * K + k] = acc[k];
  part_b[blk * Di + c.i] = acc_b;
}

// F4c tail: delta_raw = round(dt + b_dt[i]), four channels per thread
// (d_inner % 4 == 0 and 16-byte aligned buffers); a grid of rows * nq4
// workgroups, nq4 = ceil(d_inner / 1024) blocks of four-channel groups per
// row, so the row comes from one 32-bit division per workgroup
template <Act A>
__global__ void __launch_bounds__(kThreads) bias_round_kernel(const float* __restrict__ dt,
                                                             const float* __restrict__ b, void* __restrict__ out,
                                                             int64_t Di, unsigned nq4) {
  const unsigned row = blockIdx.x / nq4;
  const int64_t i = (static_cast<int64_t>(blockIdx.x - row * nq4) * kThreads + threadIdx.x) * 4;
  if (i >= Di) return;
  const int64_t e = static_cast<int64_t>(row) * Di + i;
  const float4 d = *reinterpret_cast<const float4*>(dt + e);
  const float4 bb = *reinterpret_cast<const float4*>(b + i);
  st4<A>(out, e, make_float4(d.x + bb.x, d.y + bb.y, d.z + bb.z, d.w + bb.w));
}

// out = round(in), four elements per thread (16-byte aligned buffers); the
// thread at the end takes the n % 4 elements left one by one
template <Act A>
__global__ void __launch_bounds__(kThreads) cast_kernel(const float* __restrict__ in, void* __restrict__ out,
                                                       int64_t n) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
  if (e >= n) return;
  if (e + 4 <= n) {
    st4<A>(out, e, *reinterpret_cast<const float4*>(in + e));
  } else {
    for (int64_t k = e; k < n; ++k) IO<A>::st(out, k, in[k]);
  }
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
  constexpr int U = 16;
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

// out[j] += sum_{blk < nblk} part[blk, j] for the 64 columns of a
// workgroup: wave w sums the w-th of four contiguous runs of blocks in
// ascending order, then the four run sums are added in run order (a fixed
// order, so the result does not vary between runs)
constexpr int kFewBlocks = 8;   // colsum_few_kernel's most blocks

__global__ void __launch_bounds__(kThreads) colsum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                         int64_t nblk, int64_t cols) {
  constexpr int NW = kThreads / 64;
  __shared__ float run[NW][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const int64_t per = (nblk + NW - 1) / NW;
  const int64_t b0 = wave * per < nblk ? wave * per : nblk;
  const int64_t b1 = b0 + per < nblk ? b0 + per : nblk;
  run[wave][lane] = j < cols ? mscan::ordered_sum(part + b0 * cols + j, b1 - b0, cols) : 0.0f;
  __syncthreads();
  if (wave == 0 && j < cols) {
    float t = run[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += run[w][lane];
    out[j] += t;
  }
}

// The same sum for a few blocks over many columns (the K-split weight
// products' partials): one thread per 4 columns adds the blocks in
// ascending order, 16-byte accesses.
__global__ void __launch_bounds__(kThreads) colsum_few_kernel(const float4* __restrict__ part, float4* __restrict__ out,
                                                             int64_t nblk, int64_t cols4) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= cols4) return;
  float4 v[kFewBlocks];
#pragma unroll
  for (int b = 0; b < kFewBlocks; ++b)
    if (b < nblk) v[b] = part[b * cols4 + j];
  float4 t = v[0];
#pragma unroll
  for (int b = 1; b < kFewBlocks; ++b)
    if (b < nblk) {
      t.x += v[b].x;
      t.y += v[b].y;
      t.z += v[b].z;
      t.w += v[b].w;
    }
  float4 o = out[j];
  o.x += t.x;
  o.y += t.y;
  o.z += t.z;
  o.w += t.w;
  out[j] = o;
}

__global__ void __launch_bounds__(kThreads) zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e < n) p[e] = 0.0f;
}

dim3 grid1(int64_t n) { return dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)); }

// channel blocks of 256 threads per row (conv kernels)
unsigned nchb(const Op& o) { return static_cast<unsigned>((o.cols + kThreads - 1) / kThreads); }
// blocks of 256 four-channel groups per row (dt bias)
unsigned nq4(const Op& o) { return static_cast<unsigned>((o.cols + 4 * kThreads - 1) / (4 * kThreads)); }
// one wave per row (RMSNorm)
dim3 grid_wave_rows(int64_t rows) { return dim3(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }
// conv tiles: batch rows * step tiles * channel blocks
unsigned ntb(const Op& o) { return static_cast<unsigned>((o.T + kConvTT - 1) / kConvTT); }
dim3 grid_conv(const Op& o) { return dim3(static_cast<unsigned>(o.n / o.cols / o.T) * ntb(o) * nchb(o)); }

template <Act A>
hipError_t dispatch(const Op& o, hipStream_t st) {
  const dim3 blk(kThreads);
  switch (o.kind) {
    case OpKind::RmsnormFwd:
      hipLaunchKernelGGL(rmsnorm_fwd_kernel<A>, grid_wave_rows(o.rows), blk, 0, st, o.f0, o.f1, o.v0, o.f3, o.rows,
                         o.cols, o.eps);
      break;
    case OpKind::ConvSiluFwd:
      hipLaunchKernelGGL(conv_silu_fwd_kernel<A>, grid_conv(o), blk, 0, st, o.c0, o.f0, o.f1, o.v0, o.T, o.cols, o.K,
                         nchb(o), ntb(o));
      break;
    case OpKind::ConvBwd:
      hipLaunchKernelGGL(conv_bwd_kernel<A>, grid_conv(o), blk, 0, st, o.c0, o.f0, o.f1, o.c1, o.f2, o.v0, o.f3, o.f6,
                         o.T, o.cols, o.K, nchb(o), ntb(o));
      break;
    case OpKind::BiasRound:
      hipLaunchKernelGGL(bias_round_kernel<A>, dim3(static_cast<unsigned>(o.n / o.cols) * nq4(o)), blk, 0, st, o.f0,
                         o.f1, o.v0, o.cols, nq4(o));
      break;
    case OpKind::Cast:
      hipLaunchKernelGGL(cast_kernel<A>, grid1((o.n + 3) / 4), blk, 0, st, o.f0, o.v0, o.n);
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

int64_t conv_step_tiles(int64_t T) { return (T + kConvTT - 1) / kConvTT; }

hipError_t launch(const Op& o, Act act, hipStream_t st) {
  const dim3 blk(kThreads);
  switch (o.kind) {   // dtype-free kernels
    case OpKind::RmsnormBwd:
      hipLaunchKernelGGL(rmsnorm_bwd_kernel, grid_wave_rows(o.rows), blk, 0, st, o.f0, o.f1, o.f2, o.f4, o.f5, o.f3,
                         o.rows, o.cols);
      return hipGetLastError();
    case OpKind::RmsnormWgradPart:
      hipLaunchKernelGGL(rmsnorm_wgrad_part_kernel, dim3(grid1(o.cols).x, static_cast<unsigned>(o.nblk)), blk, 0, st,
                         o.f0, o.f1, o.f2, o.f3, o.rows, o.cols, o.per_blk);
      return hipGetLastError();
    case OpKind::ColSum:
      if (o.nblk >= 1 && o.nblk <= kFewBlocks && o.cols % 4 == 0 && reinterpret_cast<uintptr_t>(o.f0) % 16 == 0 &&
          reinterpret_cast<uintptr_t>(o.f3) % 16 == 0) {
        hipLaunchKernelGGL(colsum_few_kernel, grid1(o.cols / 4), blk, 0, st, reinterpret_cast<const float4*>(o.f0),
                           reinterpret_cast<float4*>(o.f3), o.nblk, o.cols / 4);
        return hipGetLastError();
      }
      hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>((o.cols + 63) / 64)), blk, 0, st, o.f0, o.f3,
                         o.nblk, o.cols);
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
