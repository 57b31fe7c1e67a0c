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
  for (int e = tid; e < kL * kP; e += kThreads) {
    const int s = e / kP, q = e % kP;
    const bool ok = t0 + s < d.T;
    sXT[q * XS + s] = ok ? sW[s] * IO<Act::BF16>::ld(p.X, ((b * d.T + t0 + s) * d.H + h) * kP + q) : 0.0f;
  }
  for (int e = tid; e < kL * N; e += kThreads) {
    const int s = e / N, n = e % N;
    sYT[n * YS + s] = t0 + s < d.T ? raw_bf16(p.Y, (bh * d.T + t0 + s) * N + n) : static_cast<__bf16>(0.0f);
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
  for (int e = tid; e < kL * N; e += kThreads) {
    const int row = e / N, n = e % N;
    const bool ok = t0 + row < d.T;
    const int64_t gi = (bh * d.T + t0 + row) * N + n;
    s.q[row * QS + n] = ok ? raw_bf16(p.Qr, gi) : static_cast<__bf16>(0.0f);
    s.k[row * QS + n] = ok ? raw_bf16(p.Kr, gi) : static_cast<__bf16>(0.0f);
  }
  for (int e = tid; e < kL * kP; e += kThreads) {
    const int row = e / kP, q = e % kP;
    s.vT[q * VS + row] =
        t0 + row < d.T ? raw_bf16(p.x, ((b * d.T + t0 + row) * d.H + h) * kP + q) : static_cast<__bf16>(0.0f);
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
// Wave w owns the query steps t = 16w .. +15 (rows of G, DV, dQ) and the key
// steps s = 16w .. +15 (rows of dV, dK).  Phase 1: G and DV tiles, their
// masked forms and per-step sums; phase 2: the products inside the chunk;
// phase 3 (with the entering state and the outgoing state's gradient in
// LDS): the products across chunks; then the outputs.
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
  float cum[kL], sc[kL], gam[kL], qk[kL], dvd[kL], rrow[kL], dcq[kL], dus[kL];
  float colR[4][kL], colE[4][kL];
  float red[kThreads];
};

template <int N>
__global__ void __launch_bounds__(kThreads) m3_chunk_bwd_mfma(const BwdArgs p) {
  using L = BwdLdsM<N>;
  constexpr int QS = L::QS, VS = L::VS, FS = L::FS, TS = L::TS;
  constexpr int NT = N / 16;
  __shared__ __attribute__((aligned(16))) L s;
  const Dims d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t c = blockIdx.x % d.nc, bh = blockIdx.x / d.nc, h = bh % d.H, b = bh / d.H;
  const int64_t t0 = c * kL;
  const __bf16 z16 = static_cast<__bf16>(0.0f);
  float tot = 0.0f;
  if (tid < 64) {
    const ChunkScalars cs = chunk_cum(p.da + bh * d.T, t0, d.T, tid);
    s.cum[tid] = cs.cum;
    s.sc[tid] = cs.valid ? p.sc[bh * d.T + t0 + tid] : 0.0f;
    s.gam[tid] = cs.valid ? p.gam[bh * d.T + t0 + tid] : 0.0f;
    tot = cs.tot;
  }
  for (int e = tid; e < kL * N; e += kThreads) {
    const int row = e / N, n = e % N;
    const bool ok = t0 + row < d.T;
    const int64_t gi = (bh * d.T + t0 + row) * N + n;
    const __bf16 qv = ok ? raw_bf16(p.Qr, gi) : z16, kv = ok ? raw_bf16(p.Kr, gi) : z16;
    s.q[row * QS + n] = qv;
    s.k[row * QS + n] = kv;
    s.u.a.qT[n * VS + row] = qv;
    s.u.a.kT[n * VS + row] = kv;
  }
  for (int e = tid; e < kL * kP; e += kThreads) {
    const int row = e / kP, q = e % kP;
    const bool ok = t0 + row < d.T;
    const int64_t gi = ((b * d.T + t0 + row) * d.H + h) * kP + q;
    const __bf16 vv = ok ? raw_bf16(p.x, gi) : z16, yv = ok ? raw_bf16(p.dy, gi) : z16;
    s.v[row * VS + q] = vv;
    s.dy[row * VS + q] = yv;
    s.u.a.dyT[q * VS + row] = yv;
  }
  __syncthreads();

  // ---- phase 1: G = Q K^T and DV = dY V^T on the tiles (t-block w, s-block sb)
  {
    bf16x8 qa[N / 32], ya[2];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) qa[k] = ld8(&s.q[(16 * w + r) * QS + 32 * k + 8 * g]);
#pragma unroll
    for (int k = 0; k < 2; ++k) ya[k] = ld8(&s.dy[(16 * w + r) * VS + 32 * k + 8 * g]);
    float rrow[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4 gt = {0.0f, 0.0f, 0.0f, 0.0f}, dv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (sb <= w) {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) gt = mma(qa[k], ld8(&s.k[(16 * sb + r) * QS + 32 * k + 8 * g]), gt);
#pragma unroll
        for (int k = 0; k < 2; ++k) dv = mma(ya[k], ld8(&s.v[(16 * sb + r) * VS + 32 * k + 8 * g]), dv);
      }
      float cr = 0.0f, ce = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + 4 * g + e, sv = 16 * sb + r;
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
        s.colR[w][16 * sb + r] = cr;
        s.colE[w][16 * sb + r] = ce;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = sum16(rrow[e]);
      if (r == 0) s.rrow[16 * w + 4 * g + e] = v;
    }
  }
  __syncthreads();

  // ---- phase 2: products inside the chunk
  //   dV[s][p] = sum_{t>=s} GM[t][s] dY[t][p]   (A = GM^T [s][t], B = dY^T [p][t])
  //   dQ[t][n] = sum_{s<=t} DVM[t][s] K[s][n]    (A = DVM [t][s],  B = K^T [n][s])
  //   dK[s][n] = sum_{t>=s} DVM[t][s] Q[t][n]    (A = DVM^T [s][t], B = Q^T [n][t])
  f32x4 dV[4], dQ[NT], dK[NT];
  const int klo = (16 * w) / 32;              // first 32-step block of t that reaches t >= 16w
  const int khi = (16 * (w + 1) + 31) / 32;   // 32-step blocks of s that reach s <= 16w + 15
  {
    bf16x8 ghi[2], glo[2], dhi[2], dlo[2], thi[2], tlo[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ld8_split(&s.u.a.gmT[(16 * w + r) * FS + 32 * k + 8 * g], ghi[k], glo[k]);
      ld8_split(&s.u.a.dvm[(16 * w + r) * FS + 32 * k + 8 * g], dhi[k], dlo[k]);
      ld8_split(&s.u.a.dvmT[(16 * w + r) * FS + 32 * k + 8 * g], thi[k], tlo[k]);
    }
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      dV[pb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (k >= klo) {
          const bf16x8 bv = ld8(&s.u.a.dyT[(16 * pb + r) * VS + 32 * k + 8 * g]);
          dV[pb] = mma(ghi[k], bv, dV[pb]);
          dV[pb] = mma(glo[k], bv, dV[pb]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      dQ[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      dK[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k < khi) {
          const bf16x8 bk = ld8(&s.u.a.kT[(16 * nt + r) * VS + 32 * k + 8 * g]);
          dQ[nt] = mma(dhi[k], bk, dQ[nt]);
          dQ[nt] = mma(dlo[k], bk, dQ[nt]);
        }
        if (k >= klo) {
          const bf16x8 bq = ld8(&s.u.a.qT[(16 * nt + r) * VS + 32 * k + 8 * g]);
          dK[nt] = mma(thi[k], bq, dK[nt]);
          dK[nt] = mma(tlo[k], bq, dK[nt]);
        }
      }
    }
  }
  __syncthreads();   // the phase 1-2 arrays are free from here

  // ---- phase 3: products across chunks
  const float* stin = p.st + (bh * d.nc + c) * kP * N;
  const float* dsout = p.dst + (bh * d.nc + c) * kP * N;
  float dtot_part = 0.0f;
  for (int e = tid; e < kP * N; e += kThreads) {
    const int q = e / N, n = e % N;
    const float a = stin[e], bb = dsout[e];
    s.u.c.stT[n * TS + q] = a;
    s.u.c.dsT[n * TS + q] = bb;
    dtot_part = fmaf(a, bb, dtot_part);
  }
  s.red[tid] = dtot_part;
  __shared__ float s_tot;
  if (tid == 0) s_tot = tot;
  __syncthreads();
  const float totv = s_tot;
  {
    bf16x8 ya[2], va[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ya[k] = ld8(&s.dy[(16 * w + r) * VS + 32 * k + 8 * g]);
      va[k] = ld8(&s.v[(16 * w + r) * VS + 32 * k + 8 * g]);
    }
    float ec[4], uc[4], dcq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dus[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g + e;
      ec[e] = expf_fast(s.cum[t]);
      uc[e] = expf_fast(totv - s.cum[t]) * s.sc[t];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
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
        const int t = 16 * w + 4 * g + e, n = 16 * nt + r;
        const float qz = ec[e] * zq[e];
        dQ[nt][e] += qz;
        dcq[e] = fmaf(static_cast<float>(s.q[t * QS + n]), qz, dcq[e]);
        dK[nt][e] = fmaf(uc[e], zk[e], dK[nt][e]);
        dus[e] = fmaf(static_cast<float>(s.k[t * QS + n]), zk[e], dus[e]);
      }
    }
    // dV[s][p] += u_s sum_n K[s][n] dSt[p][n]   (A = K [s][n], B = dSt [p][n] from global)
    bf16x8 ka[N / 32];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) ka[k] = ld8(&s.k[(16 * w + r) * QS + 32 * k + 8 * g]);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      f32x4 wv = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < N / 32; ++k) {
        bf16x8 hi, lo;
        ld8_split(dsout + (16 * pb + r) * N + 32 * k + 8 * g, hi, lo);
        wv = mma(ka[k], hi, wv);
        wv = mma(ka[k], lo, wv);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dV[pb][e] = fmaf(uc[e], wv[e], dV[pb][e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = sum16(dcq[e]), bq = sum16(dus[e]);
      if (r == 0) {
        s.dcq[16 * w + 4 * g + e] = a;
        s.dus[16 * w + 4 * g + e] = bq;
      }
    }
  }

  // ---- outputs of the tiles (rows 16w + 4g + e)
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 16 * w + 4 * g + e;
    if (t0 + t >= d.T) continue;
    const float dg = s.gam[t] - s.sc[t];
    const float dq_c = dg * s.dvd[t];
    const float dv_c = dg * s.qk[t] + Dh;
    const int64_t xrow = ((b * d.T + t0 + t) * d.H + h) * kP;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const int q = 16 * pb + r;
      IO<Act::BF16>::st(p.d_x, xrow + q, fmaf(dv_c, static_cast<float>(s.dy[t * VS + q]), dV[pb][e]));
    }
    const int64_t qrow = (bh * d.T + t0 + t) * N;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = 16 * nt + r;
      p.dQ[qrow + n] = fmaf(dq_c, static_cast<float>(s.k[t * QS + n]), dQ[nt][e]);
      p.dK[qrow + n] = fmaf(dq_c, static_cast<float>(s.q[t * QS + n]), dK[nt][e]);
    }
  }
  __syncthreads();
  // ---- per-step scalars (wave 0, lane = step)
  if (tid < 64) {
    float cr = 0.0f, ce = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cr += s.colR[k][tid];
      ce += s.colE[k][tid];
    }
    float dsum = 0.0f;
    for (int k = 0; k < kThreads; k += 64) dsum += s.red[k + tid];
    const float dotSS = wave_sum(dsum);
    const float us = s.dus[tid];
    const float u = expf_fast(tot - s.cum[tid]) * s.sc[tid];
    const float dcum_t = s.rrow[tid] - cr + s.dcq[tid] - u * us;
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
