// Matrix-core (MFMA) versions of the Mamba-3 chunk kernels for bf16
// activations (gfx950, v_mfma_f32_16x16x32_bf16).  Included by m3.hip after
// the VALU versions, whose argument structs and chunk algebra they share.
//
// Every contraction of a chunk (64 steps, headdim 64, d_state N) is a sum of
// 16 x 16 tiles.  One instruction multiplies a 16 x 32 A block by a 32 x 16
// B block into a 16 x 16 f32 accumulator; lane l holds
//   A[l % 16][8 (l / 16) .. + 7],  B[8 (l / 16) .. + 7][l % 16]  (bf16 x 8)
//   D[4 (l / 16) + e][l % 16], e < 4                              (f32 x 4)
// (checked on the device).  So each operand is read as 8 consecutive
// elements along the contracted index: the LDS copies are laid out with the
// contracted index fastest, transposed where a product needs it.  bf16
// operands (the turned Q and K, x, dy) are exact; an f32 operand (masked
// pair weights, weighted rows, chunk states) is split into a bf16 high part
// and the bf16 rounding of the remainder, two instructions whose sum keeps
// about 16 significant bits (the f32 accumulation is unchanged).
#pragma once

namespace m3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// 8 consecutive f32 (16-byte aligned) as high and low bf16 parts
__device__ __forceinline__ void ld8_split(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(v[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
  }
}

__device__ __forceinline__ __bf16 raw_bf16(const void* p, int64_t i) { return static_cast<const __bf16*>(p)[i]; }

// 8 consecutive bf16 of a global row (16-byte aligned), or zeros
__device__ __forceinline__ bf16x8 g8(const void* p, int64_t i, bool ok) {
  if (!ok) return bf16x8{};
  return *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p) + i);
}

__device__ __forceinline__ void st8(__bf16* p, const bf16x8& v) { *reinterpret_cast<bf16x8*>(p) = v; }

__device__ __forceinline__ float sum16(float v) {   // over the 16 lanes of one l / 16 group
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

__device__ __forceinline__ float sum_groups(float v) {   // over the four l / 16 groups
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// ------------------------------------------------------- chunk state
// out[p][n] = sum_s w_s X[s][p] Y[s][n]: A = (w X)^T [p][s] (f32, split),
// B = Y^T [n][s] (bf16).  Wave w computes p rows 16w .. 16w + 15.
template <int N, bool BWD>
__global__ void __launch_bounds__(kThreads) m3_chunk_state_mfma(const ChunkStateArgs p) {
  constexpr int XS = kL + 4, YS = kL + 8;
  __shared__ __attribute__((aligned(16))) float sXT[kP * XS];
  __shared__ __attribute__((aligned(16))) __bf16 sYT[N * YS];
  __shared__ float sW[kL];
  const Dims d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  if (tid < 64) {
    const ChunkScalars s = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    float wt = 0.0f;
    if (s.valid) wt = BWD ? expf_fast(s.cum) : expf_fast(s.tot - s.cum) * p.sc[bh * d.T + t0 + tid];
    sW[tid] = wt;
    if (tid == 0) p.tot[bh * d.nc + c] = s.tot;
  }
  __syncthreads();
  for (int e = tid; e < kL * kP / 8; e += kThreads) {
    const int s = e / (kP / 8), q = (e % (kP / 8)) * 8;
    const bf16x8 v = g8(p.X, ((b * d.T + t0 + s) * d.H + h) * kP + q, t0 + s < d.T);
#pragma unroll
    for (int k = 0; k < 8; ++k) sXT[(q + k) * XS + s] = sW[s] * static_cast<float>(v[k]);
  }
  for (int e = tid; e < kL * N / 8; e += kThreads) {
    const int s = e / (N / 8), n = (e % (N / 8)) * 8;
    const bf16x8 v = g8(p.Y, (bh * d.T + t0 + s) * N + n, t0 + s < d.T);
#pragma unroll
    for (int k = 0; k < 8; ++k) sYT[(n + k) * YS + s] = v[k];
  }
  __syncthreads();
  const int r = lane & 15, g = lane >> 4;
  bf16x8 ahi[2], alo[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) ld8_split(&sXT[(16 * w + r) * XS + 32 * k + 8 * g], ahi[k], alo[k]);
  float* out = p.out + (bh * d.nc + c) * kP * N;
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bf16x8 bv = ld8(&sYT[(16 * nt + r) * YS + 32 * k + 8 * g]);
      acc = mma(ahi[k], bv, acc);
      acc = mma(alo[k], bv, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(16 * w + 4 * g + e) * N + 16 * nt + r] = acc[e];
  }
}

// ---------------------------------------------------------- chunk output
// Wave w owns the steps t = 16w .. 16w + 15: G = Q K^T for the key blocks
// s <= t, masked into GM (f32, LDS), then y = GM V + e^{cum} Q St_in^T + the
// diagonal and D terms.
template <int N>
struct OutLdsM {
  static constexpr int QS = N + 8, VS = kL + 8, GS = kL + 4;
  __bf16 q[kL * QS];
  __bf16 k[kL * QS];
  __bf16 vT[kP * VS];     // [p][s]
  float gm[kL * GS];      // [t][s]
  float cum[kL], sc[kL], gam[kL], qk[kL];
};

template <int N>
__global__ void __launch_bounds__(kThreads) m3_chunk_out_mfma(const OutArgs p) {
  using L = OutLdsM<N>;
  constexpr int QS = L::QS, VS = L::VS, GS = L::GS;
  __shared__ __attribute__((aligned(16))) L s;
  const Dims d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  if (tid < 64) {
    const ChunkScalars cs = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    s.cum[tid] = cs.cum;
    s.sc[tid] = cs.valid ? p.sc[bh * d.T + t0 + tid] : 0.0f;
    s.gam[tid] = cs.valid ? p.gam[bh * d.T + t0 + tid] : 0.0f;
  }
  for (int e = tid; e < kL * N / 8; e += kThreads) {
    const int row = e / (N / 8), n = (e % (N / 8)) * 8;
    const bool ok = t0 + row < d.T;
    const int64_t gi = (bh * d.T + t0 + row) * N + n;
    st8(&s.q[row * QS + n], g8(p.Qr, gi, ok));
    st8(&s.k[row * QS + n], g8(p.Kr, gi, ok));
  }
  for (int e = tid; e < kL * kP / 8; e += kThreads) {
    const int row = e / (kP / 8), q = (e % (kP / 8)) * 8;
    const bf16x8 v = g8(p.x, ((b * d.T + t0 + row) * d.H + h) * kP + q, t0 + row < d.T);
#pragma unroll
    for (int k = 0; k < 8; ++k) s.vT[(q + k) * VS + row] = v[k];
  }
  __syncthreads();
  bf16x8 qa[N / 32];
#pragma unroll
  for (int k = 0; k < N / 32; ++k) qa[k] = ld8(&s.q[(16 * w + r) * QS + 32 * k + 8 * g]);
  // masked G for the key blocks sb <= w; zeros for the blocks after
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (sb <= w) {
#pragma unroll
      for (int k = 0; k < N / 32; ++k) acc = mma(qa[k], ld8(&s.k[(16 * sb + r) * QS + 32 * k + 8 * g]), acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g + e, sv = 16 * sb + r;
      const float m = sv <= t ? expf_fast(s.cum[t] - s.cum[sv]) * s.sc[sv] : 0.0f;
      s.gm[t * GS + sv] = acc[e] * m;
      if (sv == t) s.qk[t] = acc[e];
    }
  }
  __syncthreads();
  const float* st = p.st + (bh * d.nc + c) * kP * N;
  const int kmax = (16 * (w + 1) + 31) / 32;   // 32-step blocks of s that reach t <= 16w + 15
  bf16x8 ghi[2], glo[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (k < kmax) ld8_split(&s.gm[(16 * w + r) * GS + 32 * k + 8 * g], ghi[k], glo[k]);
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    f32x4 yi = {0.0f, 0.0f, 0.0f, 0.0f}, ys = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k < kmax) {
        const bf16x8 vv = ld8(&s.vT[(16 * pb + r) * VS + 32 * k + 8 * g]);
        yi = mma(ghi[k], vv, yi);
        yi = mma(glo[k], vv, yi);
      }
    }
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
      bf16x8 shi, slo;
      ld8_split(st + (16 * pb + r) * N + 32 * k + 8 * g, shi, slo);
      ys = mma(qa[k], shi, ys);
      ys = mma(qa[k], slo, ys);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g + e, q = 16 * pb + r;
      if (t0 + t >= d.T) continue;
      const float vt = static_cast<float>(s.vT[q * VS + t]);
      const float yv = fmaf(expf_fast(s.cum[t]), ys[e], yi[e]) + ((s.gam[t] - s.sc[t]) * s.qk[t] + Dh) * vt;
      IO<Act::BF16>::st(p.y, ((b * d.T + t0 + t) * d.H + h) * kP + q, yv);
    }
  }
}

// -------------------------------------------------------- chunk backward
// Eight waves: wave w handles block tb = w % 4 of 16 steps, in half hf = w / 4
// of the tiles: the key blocks sb = hf, hf + 2 of its G / DV row, the p tiles
// 2 hf, 2 hf + 1 of dV and half of the d_state tiles of dQ and dK (two waves
// per SIMD hide the LDS and memory latency a single one waits on).  Phase 1:
// G and DV tiles, their masked forms and per-step sums; phase 2: the
// products inside the chunk; phase 3 (with the entering state and the
// outgoing state's gradient in LDS): the products across chunks; then the
// outputs.
constexpr int kThreadsB = 512;

template <int N>
struct BwdLdsM {
  static constexpr int QS = N + 8, VS = kL + 8, FS = kL + 4, TS = kP + 4;
  __bf16 q[kL * QS];       // [t][n]
  __bf16 k[kL * QS];       // [s][n]
  __bf16 v[kL * VS];       // [s][p]
  __bf16 dy[kL * VS];      // [t][p]
  // phase 1-2 arrays, then (phase 3) the two states as [n][p] f32
  union {
    struct {
      __bf16 qT[N * VS];     // [n][t]
      __bf16 kT[N * VS];     // [n][s]
      __bf16 dyT[kP * VS];   // [p][t]
      float gmT[kL * FS];    // [s][t]
      float dvm[kL * FS];    // [t][s]
      float dvmT[kL * FS];   // [s][t]
    } a;
    struct {
      float stT[N * TS];     // St_in  [n][p]
      float dsT[N * TS];     // dSt_out [n][p]
    } c;
  } u;
  float cum[kL], sc[kL], gam[kL], qk[kL], dvd[kL];
  float rrow[2][kL], dcq[2][kL], dus[2][kL];
  float colR[4][kL], colE[4][kL];
  float red[kThreadsB];
  float tot;
};

template <int N>
__global__ void __launch_bounds__(kThreadsB) m3_chunk_bwd_mfma(const BwdArgs p) {
  using L = BwdLdsM<N>;
  constexpr int QS = L::QS, VS = L::VS, FS = L::FS, TS = L::TS;
  constexpr int NT = N / 16, NH = NT / 2;   // d_state tiles, per half
  __shared__ __attribute__((aligned(16))) L s;
  const Dims d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tb = wv & 3, hf = wv >> 2;
  const int r = lane & 15, g = lane >> 4;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  if (tid < 64) {
    const ChunkScalars cs = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    s.cum[tid] = cs.cum;
    s.sc[tid] = cs.valid ? p.sc[bh * d.T + t0 + tid] : 0.0f;
    s.gam[tid] = cs.valid ? p.gam[bh * d.T + t0 + tid] : 0.0f;
    if (tid == 0) s.tot = cs.tot;
  }
  for (int e = tid; e < kL * N / 8; e += kThreadsB) {
    const int row = e / (N / 8), n = (e % (N / 8)) * 8;
    const bool ok = t0 + row < d.T;
    const int64_t gi = (bh * d.T + t0 + row) * N + n;
    const bf16x8 qv = g8(p.Qr, gi, ok), kv = g8(p.Kr, gi, ok);
    st8(&s.q[row * QS + n], qv);
    st8(&s.k[row * QS + n], kv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s.u.a.qT[(n + k) * VS + row] = qv[k];
      s.u.a.kT[(n + k) * VS + row] = kv[k];
    }
  }
  for (int e = tid; e < kL * kP / 8; e += kThreadsB) {
    const int row = e / (kP / 8), q = (e % (kP / 8)) * 8;
    const bool ok = t0 + row < d.T;
    const int64_t gi = ((b * d.T + t0 + row) * d.H + h) * kP + q;
    const bf16x8 vv = g8(p.x, gi, ok), yv = g8(p.dy, gi, ok);
    st8(&s.v[row * VS + q], vv);
    st8(&s.dy[row * VS + q], yv);
#pragma unroll
    for (int k = 0; k < 8; ++k) s.u.a.dyT[(q + k) * VS + row] = yv[k];
  }
  __syncthreads();

  // ---- phase 1: G = Q K^T and DV = dY V^T on the tiles (block tb, key blocks sb = hf, hf + 2)
  {
    bf16x8 qa[N / 32], ya[2];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) qa[k] = ld8(&s.q[(16 * tb + r) * QS + 32 * k + 8 * g]);
#pragma unroll
    for (int k = 0; k < 2; ++k) ya[k] = ld8(&s.dy[(16 * tb + r) * VS + 32 * k + 8 * g]);
    float rrow[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sb = hf + 2 * j;
      f32x4 gt = {0.0f, 0.0f, 0.0f, 0.0f}, dv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (sb <= tb) {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) gt = mma(qa[k], ld8(&s.k[(16 * sb + r) * QS + 32 * k + 8 * g]), gt);
#pragma unroll
        for (int k = 0; k < 2; ++k) dv = mma(ya[k], ld8(&s.v[(16 * sb + r) * VS + 32 * k + 8 * g]), dv);
      }
      float cr = 0.0f, ce = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e, sv = 16 * sb + r;
        const float ee = sv <= t ? expf_fast(s.cum[t] - s.cum[sv]) : 0.0f;
        const float m = ee * s.sc[sv];
        s.u.a.gmT[sv * FS + t] = gt[e] * m;
        s.u.a.dvm[t * FS + sv] = dv[e] * m;
        s.u.a.dvmT[sv * FS + t] = dv[e] * m;
        const float gd = gt[e] * dv[e];
        rrow[e] = fmaf(gd, m, rrow[e]);
        cr = fmaf(gd, m, cr);
        ce = fmaf(gd, ee, ce);
        if (sv == t) {
          s.qk[t] = gt[e];
          s.dvd[t] = dv[e];
        }
      }
      cr = sum_groups(cr);
      ce = sum_groups(ce);
      if (g == 0) {
        s.colR[tb][16 * sb + r] = cr;
        s.colE[tb][16 * sb + r] = ce;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = sum16(rrow[e]);
      if (r == 0) s.rrow[hf][16 * tb + 4 * g + e] = v;
    }
  }
  __syncthreads();

  // ---- phase 2: products inside the chunk
  //   dV[s][p] = sum_{t>=s} GM[t][s] dY[t][p]   (A = GM^T [s][t], B = dY^T [p][t])
  //   dQ[t][n] = sum_{s<=t} DVM[t][s] K[s][n]    (A = DVM [t][s],  B = K^T [n][s])
  //   dK[s][n] = sum_{t>=s} DVM[t][s] Q[t][n]    (A = DVM^T [s][t], B = Q^T [n][t])
  f32x4 dV[2], dQ[NH], dK[NH];
  const int klo = (16 * tb) / 32;              // first 32-step block of t that reaches t >= 16 tb
  const int khi = (16 * (tb + 1) + 31) / 32;   // 32-step blocks of s that reach s <= 16 tb + 15
  {
    bf16x8 ghi[2], glo[2], dhi[2], dlo[2], thi[2], tlo[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ld8_split(&s.u.a.gmT[(16 * tb + r) * FS + 32 * k + 8 * g], ghi[k], glo[k]);
      ld8_split(&s.u.a.dvm[(16 * tb + r) * FS + 32 * k + 8 * g], dhi[k], dlo[k]);
      ld8_split(&s.u.a.dvmT[(16 * tb + r) * FS + 32 * k + 8 * g], thi[k], tlo[k]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pb = 2 * hf + j;
      dV[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (k >= klo) {
          const bf16x8 bv = ld8(&s.u.a.dyT[(16 * pb + r) * VS + 32 * k + 8 * g]);
          dV[j] = mma(ghi[k], bv, dV[j]);
          dV[j] = mma(glo[k], bv, dV[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int nt = hf * NH + j;
      dQ[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      dK[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k < khi) {
          const bf16x8 bk = ld8(&s.u.a.kT[(16 * nt + r) * VS + 32 * k + 8 * g]);
          dQ[j] = mma(dhi[k], bk, dQ[j]);
          dQ[j] = mma(dlo[k], bk, dQ[j]);
        }
        if (k >= klo) {
          const bf16x8 bq = ld8(&s.u.a.qT[(16 * nt + r) * VS + 32 * k + 8 * g]);
          dK[j] = mma(thi[k], bq, dK[j]);
          dK[j] = mma(tlo[k], bq, dK[j]);
        }
      }
    }
  }
  __syncthreads();   // the phase 1-2 arrays are free from here

  // ---- phase 3: products across chunks
  const float* stin = p.st + (bh * d.nc + c) * kP * N;
  const float* dsout = p.dst + (bh * d.nc + c) * kP * N;
  float dtot_part = 0.0f;
  for (int e = tid; e < kP * N / 4; e += kThreadsB) {
    const int q = e / (N / 4), n = (e % (N / 4)) * 4;
    const float4 a = *reinterpret_cast<const float4*>(stin + q * N + n);
    const float4 bb = *reinterpret_cast<const float4*>(dsout + q * N + n);
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s.u.c.stT[(n + k) * TS + q] = av[k];
      s.u.c.dsT[(n + k) * TS + q] = bv[k];
      dtot_part = fmaf(av[k], bv[k], dtot_part);
    }
  }
  s.red[tid] = dtot_part;
  __syncthreads();
  const float totv = s.tot;
  {
    bf16x8 ya[2], va[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ya[k] = ld8(&s.dy[(16 * tb + r) * VS + 32 * k + 8 * g]);
      va[k] = ld8(&s.v[(16 * tb + r) * VS + 32 * k + 8 * g]);
    }
    float ec[4], uc[4], dcq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dus[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tb + 4 * g + e;
      ec[e] = expf_fast(s.cum[t]);
      uc[e] = expf_fast(totv - s.cum[t]) * s.sc[t];
    }
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int nt = hf * NH + j;
      f32x4 zq = {0.0f, 0.0f, 0.0f, 0.0f}, zk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        bf16x8 hi, lo;
        ld8_split(&s.u.c.stT[(16 * nt + r) * TS + 32 * k + 8 * g], hi, lo);
        zq = mma(ya[k], hi, zq);
        zq = mma(ya[k], lo, zq);
        ld8_split(&s.u.c.dsT[(16 * nt + r) * TS + 32 * k + 8 * g], hi, lo);
        zk = mma(va[k], hi, zk);
        zk = mma(va[k], lo, zk);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tb + 4 * g + e, n = 16 * nt + r;
        const float qz = ec[e] * zq[e];
        dQ[j][e] += qz;
        dcq[e] = fmaf(static_cast<float>(s.q[t * QS + n]), qz, dcq[e]);
        dK[j][e] = fmaf(uc[e], zk[e], dK[j][e]);
        dus[e] = fmaf(static_cast<float>(s.k[t * QS + n]), zk[e], dus[e]);
      }
    }
    // dV[s][p] += u_s sum_n K[s][n] dSt[p][n]   (A = K [s][n], B = dSt [p][n] from global)
    bf16x8 ka[N / 32];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) ka[k] = ld8(&s.k[(16 * tb + r) * QS + 32 * k + 8 * g]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pb = 2 * hf + j;
      f32x4 wacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < N / 32; ++k) {
        bf16x8 hi, lo;
        ld8_split(dsout + (16 * pb + r) * N + 32 * k + 8 * g, hi, lo);
        wacc = mma(ka[k], hi, wacc);
        wacc = mma(ka[k], lo, wacc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dV[j][e] = fmaf(uc[e], wacc[e], dV[j][e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = sum16(dcq[e]), bq = sum16(dus[e]);
      if (r == 0) {
        s.dcq[hf][16 * tb + 4 * g + e] = a;
        s.dus[hf][16 * tb + 4 * g + e] = bq;
      }
    }
  }

  // ---- outputs of the tiles (rows 16 tb + 4g + e)
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 16 * tb + 4 * g + e;
    if (t0 + t >= d.T) continue;
    const float dg = s.gam[t] - s.sc[t];
    const float dq_c = dg * s.dvd[t];
    const float dv_c = dg * s.qk[t] + Dh;
    const int64_t xrow = ((b * d.T + t0 + t) * d.H + h) * kP;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = 16 * (2 * hf + j) + r;
      IO<Act::BF16>::st(p.d_x, xrow + q, fmaf(dv_c, static_cast<float>(s.dy[t * VS + q]), dV[j][e]));
    }
    const int64_t qrow = (bh * d.T + t0 + t) * N;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int n = 16 * (hf * NH + j) + r;
      p.dQ[qrow + n] = fmaf(dq_c, static_cast<float>(s.k[t * QS + n]), dQ[j][e]);
      p.dK[qrow + n] = fmaf(dq_c, static_cast<float>(s.q[t * QS + n]), dK[j][e]);
    }
  }
  __syncthreads();
  // ---- per-step scalars (wave 0, lane = step); partial sums added in a fixed order
  if (tid < 64) {
    float cr = 0.0f, ce = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cr += s.colR[k][tid];
      ce += s.colE[k][tid];
    }
    float dsum = 0.0f;
    for (int k = 0; k < kThreadsB; k += 64) dsum += s.red[k + tid];
    const float dotSS = wave_sum(dsum);
    const float tot = s.tot;
    const float us = s.dus[0][tid] + s.dus[1][tid];
    const float u = expf_fast(tot - s.cum[tid]) * s.sc[tid];
    const float dcum_t = (s.rrow[0][tid] + s.rrow[1][tid]) - cr + (s.dcq[0][tid] + s.dcq[1][tid]) - u * us;
    const float dsc_t = ce - s.qk[tid] * s.dvd[tid] + expf_fast(tot - s.cum[tid]) * us;
    const float dtot = wave_sum(u * us) + expf_fast(tot) * dotSS;
    const float dda = wave_suffix_scan(dcum_t, tid) + dtot;
    const bool ok = t0 + tid < d.T;
    if (ok) {
      const int64_t i = bh * d.T + t0 + tid;
      p.d_da[i] = dda;
      p.d_sc[i] = dsc_t;
      p.d_gam[i] = s.qk[tid] * s.dvd[tid];
    }
    const float dD = wave_sum(ok ? s.dvd[tid] : 0.0f);
    if (tid == 0) p.dD_part[bh * d.nc + c] = dD;
  }
}

}  // namespace m3
