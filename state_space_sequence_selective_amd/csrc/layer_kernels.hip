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

// Four consecutive elements e .. e+3 of an activation as f32 (e % 4 == 0;
// the buffer 16-byte aligned, so the 8 or 16 bytes are aligned).
template <Act A>
__device__ __forceinline__ float4 ld4(const void* p, int64_t e);
template <>
__device__ __forceinline__ float4 ld4<Act::F32>(const void* p, int64_t e) {
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
}
template <>
__device__ __forceinline__ float4 ld4<Act::BF16>(const void* p, int64_t e) {
  const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + e);
  return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                     __uint_as_float(r.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ float4 ld4<Act::F16>(const void* p, int64_t e) {
  struct alignas(8) H4 {
    _Float16 h[4];
  };
  const H4 q = *reinterpret_cast<const H4*>(static_cast<const _Float16*>(p) + e);
  return make_float4(static_cast<float>(q.h[0]), static_cast<float>(q.h[1]), static_cast<float>(q.h[2]),
                     static_cast<float>(q.h[3]));
}

__device__ __forceinline__ float4 f4zero() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }

// Tiles of the conv kernels: the conv is a short stencil in time (K <= 4
// taps), so every output is computed independently from global memory (the
// K - 1 halo rows a neighbouring thread also reads come from the caches) and
// the kernels have no loop over time.  A thread takes 4 channels (8- or
// 16-byte accesses) x kConvS consecutive steps; a workgroup 64 channels x
// kConvTT steps of one batch row.  Block id = (b * ntb + tb) * ncb + channel
// block, ntb = ceil(T / kConvTT), ncb = ceil(d_inner / 64).
constexpr int kConvS = 8;                                 // steps per thread
constexpr int kConvCQ = 16;                               // channel quads per workgroup
constexpr int kConvTT = (kThreads / kConvCQ) * kConvS;   // steps per workgroup: 128

struct ConvTile {
  int64_t b, tb, s0, i0;   // batch row, step block, first step, first channel
  bool on;                 // the thread has channels and steps
};

__device__ __forceinline__ ConvTile conv_tile(int64_t T, int64_t Di, unsigned ncb, unsigned ntb) {
  ConvTile c;
  const unsigned cbk = blockIdx.x % ncb, rest = blockIdx.x / ncb;
  c.b = rest / ntb;
  c.tb = rest % ntb;
  const int cq = threadIdx.x % kConvCQ, tg = threadIdx.x / kConvCQ;
  c.i0 = static_cast<int64_t>(cbk) * (4 * kConvCQ) + 4 * cq;
  c.s0 = c.tb * kConvTT + tg * kConvS;
  c.on = c.i0 < Di && c.s0 < T;
  return c;
}

// the conv weights of channels i0 .. i0+3 per tap and their bias
template <int K>
__device__ __forceinline__ void conv_weights(const float* cw, const float* cb, int64_t i0, float4 (&w)[K],
                                             float4& bias) {
#pragma unroll
  for (int k = 0; k < K; ++k)
    w[k] = make_float4(cw[i0 * K + k], cw[(i0 + 1) * K + k], cw[(i0 + 2) * K + k], cw[(i0 + 3) * K + k]);
  bias = *reinterpret_cast<const float4*>(cb + i0);
}

// rows t0 .. t0 + R - 1 of 4 channels, rows `ld` elements apart (zero
// before the sequence start; rows past the end reload the last row: their
// values are not used)
template <Act A, int R>
__device__ __forceinline__ void conv_rows(const void* p, int64_t rb, int64_t t0, int64_t T, int64_t ld, int64_t i0,
                                          float4 (&r)[R]) {
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const int64_t t = t0 + m;
    const int64_t tc = t < 0 ? 0 : (t < T ? t : T - 1);
    r[m] = ld4<A>(p, (rb + tc) * ld + i0);
    if (t < 0) r[m] = f4zero();
  }
}

// conv pre-activation b + sum_k w[k] x_{t-(K-1)+k} of 4 channels, xw[k] =
// x_{t-(K-1)+k}
template <int K>
__device__ __forceinline__ float4 conv_pre(const float4 (&w)[K], const float4& bias, const float4* xw) {
  float4 p = bias;
#pragma unroll
  for (int k = K - 1; k >= 0; --k) {
    p.x = fmaf(w[k].x, xw[k].x, p.x);
    p.y = fmaf(w[k].y, xw[k].y, p.y);
    p.z = fmaf(w[k].z, xw[k].z, p.z);
    p.w = fmaf(w[k].w, xw[k].w, p.w);
  }
  return p;
}

// F4a: u_t = SiLU(b + sum_k w[i,k] x_{t-(K-1-k)}), zero history; x rows ldx
// elements apart, u rows Di.
template <Act A, int K>
__global__ void __launch_bounds__(kThreads) conv_silu_fwd_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ cw,
                                                                const float* __restrict__ cb, void* __restrict__ u,
                                                                int64_t T, int64_t Di, int64_t ldx, unsigned ncb,
                                                                unsigned ntb) {
  const ConvTile c = conv_tile(T, Di, ncb, ntb);
  if (!c.on) return;
  float4 w[K], bias;
  conv_weights<K>(cw, cb, c.i0, w, bias);
  const int64_t rb = c.b * T;
  float4 xr[kConvS + K - 1];   // x_{s0-(K-1)} .. x_{s0+kConvS-1}
  conv_rows<A>(x, rb, c.s0 - (K - 1), T, ldx, c.i0, xr);
#pragma unroll
  for (int j = 0; j < kConvS; ++j) {
    const int64_t t = c.s0 + j;
    if (t < T) {
      const float4 p = conv_pre<K>(w, bias, xr + j);
      st4<A>(u, (rb + t) * Di + c.i0,
             make_float4(p.x * mscan::sigmoid(p.x), p.y * mscan::sigmoid(p.y), p.z * mscan::sigmoid(p.z),
                         p.w * mscan::sigmoid(p.w)));
    }
  }
}

__device__ __forceinline__ float dsilu(float p, float g) {
  const float sg = mscan::sigmoid(p);
  return g * (sg * (1.0f + p * (1.0f - sg)));
}

// Adjoint of F4a for a thread's 4 channels x kConvS steps s:
//   dp_t  = (d_u_t + d_u_extra_t) * silu'(p_t)      (p_t recomputed; zero past T)
//   d_x_s = sum_k w[i,k] dp_{s+K-1-k}               (dp for t in [s0, s0+kConvS+K-2])
//   weight partials over the thread's own t = s: sum dp_t x_{t-(K-1-k)}, sum dp_t;
// the 16 step groups of a workgroup are added in order through LDS, one
// partial per (batch row, step block).  x and d_x rows ldx elements apart,
// d_u and d_u_extra rows Di.
template <Act A, int K>
__global__ void __launch_bounds__(kThreads) conv_bwd_kernel(const void* __restrict__ x, const float* __restrict__ cw,
                                                           const float* __restrict__ cb, const void* __restrict__ du,
                                                           const float* __restrict__ du_extra,
                                                           void* __restrict__ dx, float* __restrict__ part_w,
                                                           float* __restrict__ part_b, int64_t T, int64_t Di,
                                                           int64_t ldx, unsigned ncb, unsigned ntb) {
  __shared__ float4 s_red[K + 1][kThreads];   // [tap k | bias][thread]: the thread's partials of its 4 channels
  const ConvTile c = conv_tile(T, Di, ncb, ntb);
  float4 acc[K + 1];   // taps, then the bias
#pragma unroll
  for (int k = 0; k <= K; ++k) acc[k] = f4zero();
  if (c.on) {
    float4 w[K], bias;
    conv_weights<K>(cw, cb, c.i0, w, bias);
    const int64_t rb = c.b * T;
    constexpr int ND = kConvS + K - 1;   // dp_t for t = s0 .. s0 + ND - 1
    float4 xr[ND + K - 1];                // x_{s0-(K-1)} .. x_{s0+ND-1}
    conv_rows<A>(x, rb, c.s0 - (K - 1), T, ldx, c.i0, xr);
    float4 g0[ND];
    conv_rows<A>(du, rb, c.s0, T, Di, c.i0, g0);
    float4 dp[ND];
#pragma unroll
    for (int r = 0; r < ND; ++r) {
      const int64_t t = c.s0 + r;
      const int64_t tc = t < T ? t : T - 1;
      const float4 g1 = *reinterpret_cast<const float4*>(du_extra + (rb + tc) * Di + c.i0);
      const float4 p = conv_pre<K>(w, bias, xr + r);
      dp[r] = make_float4(dsilu(p.x, g0[r].x + g1.x), dsilu(p.y, g0[r].y + g1.y), dsilu(p.z, g0[r].z + g1.z),
                          dsilu(p.w, g0[r].w + g1.w));
      if (t >= T) dp[r] = f4zero();
    }
#pragma unroll
    for (int j = 0; j < kConvS; ++j) {
      const int64_t s = c.s0 + j;
      if (s < T) {
        float4 gx = f4zero();
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float4 dk = dp[j + K - 1 - k];
          gx.x = fmaf(w[k].x, dk.x, gx.x);
          gx.y = fmaf(w[k].y, dk.y, gx.y);
          gx.z = fmaf(w[k].z, dk.z, gx.z);
          gx.w = fmaf(w[k].w, dk.w, gx.w);
        }
        st4<A>(dx, (rb + s) * ldx + c.i0, gx);
        // step t = s: tap k saw x_{t-(K-1)+k} = xr[j + k]
        const float4 g = dp[j];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          acc[k].x = fmaf(g.x, xr[j + k].x, acc[k].x);
          acc[k].y = fmaf(g.y, xr[j + k].y, acc[k].y);
          acc[k].z = fmaf(g.z, xr[j + k].z, acc[k].z);
          acc[k].w = fmaf(g.w, xr[j + k].w, acc[k].w);
        }
        acc[K].x += g.x;
        acc[K].y += g.y;
        acc[K].z += g.z;
        acc[K].w += g.w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k <= K; ++k) s_red[k][threadIdx.x] = acc[k];
  __syncthreads();
  // 64 channels x (K taps + bias): the 16 step groups added in order
  const unsigned cbk = blockIdx.x % ncb;
  const int64_t blk = c.b * ntb + c.tb;
  const float* red = reinterpret_cast<const float*>(&s_red[0][0]);
  for (int e = threadIdx.x; e < (K + 1) * 4 * kConvCQ; e += kThreads) {
    const int k = e / (4 * kConvCQ), ch = e % (4 * kConvCQ);   // tap (K: bias), channel in the block
    const int64_t i = static_cast<int64_t>(cbk) * (4 * kConvCQ) + ch;
    if (i >= Di) continue;
    // thread tg * kConvCQ + ch / 4 holds channel ch as component ch % 4
    float t = 0.0f;
    for (int tg = 0; tg < kThreads / kConvCQ; ++tg) t += red[(k * kThreads + tg * kConvCQ) * 4 + ch];
    if (k < K) part_w[(blk * Di + i) * K + k] = t;
    else part_b[blk * Di + i] = t;
  }
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
constexpr int kFewBlocks = 16;   // colsum_few_kernel's most blocks

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

// channel blocks of 64 per row (conv kernels)
unsigned nchb(const Op& o) { return static_cast<unsigned>((o.cols + 4 * kConvCQ - 1) / (4 * kConvCQ)); }
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
      switch (o.K) {
#define CONV_FWD(KK)                                                                                                \
  case KK:                                                                                                          \
    hipLaunchKernelGGL((conv_silu_fwd_kernel<A, KK>), grid_conv(o), blk, 0, st, o.c0, o.f0, o.f1, o.v0, o.T, o.cols, \
                       o.ld ? o.ld : o.cols, nchb(o), ntb(o));                                                      \
    break;
        CONV_FWD(1) CONV_FWD(2) CONV_FWD(3) CONV_FWD(4)
#undef CONV_FWD
        default:
          return hipErrorInvalidValue;
      }
      break;
    case OpKind::ConvBwd:
      switch (o.K) {
#define CONV_BWD(KK)                                                                                                \
  case KK:                                                                                                          \
    hipLaunchKernelGGL((conv_bwd_kernel<A, KK>), grid_conv(o), blk, 0, st, o.c0, o.f0, o.f1, o.c1, o.f2, o.v0, o.f3, \
                       o.f6, o.T, o.cols, o.ld ? o.ld : o.cols, nchb(o), ntb(o));                                    \
    break;
        CONV_BWD(1) CONV_BWD(2) CONV_BWD(3) CONV_BWD(4)
#undef CONV_BWD
        default:
          return hipErrorInvalidValue;
      }
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
