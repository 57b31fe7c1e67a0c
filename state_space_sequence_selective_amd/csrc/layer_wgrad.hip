// Weight gradients of the layer's skinny projections on the matrix cores
// (gfx950, v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit activations.
//
// Backward of steps F4b and F4c of the per-layer forward (mamba-rs 0.3.1
// src/mamba_ssm/gpu/forward_mixed.rs): the dt_proj weight gradient
// d_W_dt[c][j] = sum_n d_delta_raw[n][c] xdbl[n][j] (j < dt_rank) and the
// x_proj one d_W_x[j][c] = sum_n d_xdbl[n][j] u[n][c] (j < X).  Both contract
// over the N = batch * seqlen tokens a wide [N, d_inner] operand (BIG) with a
// narrow [N, J] one (SMALL, J = 48 .. 256): bound by reading BIG once.
//
// A workgroup owns 64 channels x 64 columns of the result and one chunk of
// the tokens; its 4 waves take the chunk's 32-token steps in turn.  The
// matrix cores contract over k = tokens, so a lane needs 8 consecutive tokens
// of one channel (column): it loads 4 neighbouring channels (8 bytes) of each
// of its 8 tokens, coalesced along the row (16 lanes cover 128 bytes of one
// token), and packs them into 4 operands, one per channel of the 4.  Operand
// q of the A side then holds channels c0 + 4 i + q (i = lane % 16) and of the
// B side columns j0 + 4 i + q; the 16 products of the 4 x 4 operands cover
// the 64 x 64 tile.  The 4 waves' tiles meet in LDS and are added in a
// fixed order, (w0 + w2) + (w1 + w3), through a buffer of two tiles (so
// three workgroups fit a CU), and each chunk writes its own partial (f32, in
// the gradient's layout); a column sum adds the chunks in order onto the gradient, so no
// result depends on timing.  With part_b, column J of SMALL is taken as all
// ones: its products are the column sums of BIG (the dt bias gradient beside
// the dt_proj weight gradient), written to part_b[P][Di].
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layer_kernels.h"
#include "scan_common.h"

namespace mlayer {
namespace {

using mscan::Act;

constexpr int kWw = 4;            // waves per workgroup
constexpr int kTw = 64 * kWw;
constexpr int kLs = 65;           // LDS row stride (floats): the 4 lane groups of a store land on distinct banks

template <Act A>
struct Mma;

template <>
struct Mma<Act::BF16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 mma(const v8& a, const v8& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<Act::F16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f4 mma(const v8& a, const v8& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// 8 tokens x 4 neighbouring 16-bit elements (d[t].x: elements 0, 1; d[t].y:
// 2, 3; the lower address in the low half) -> 4 operands of 8 tokens each
template <class V8>
__device__ __forceinline__ void pack4(const uint2 (&d)[8], V8 (&out)[4]) {
  union U {
    V8 v;
    uint32_t w[4];
  };
  U o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t x0 = d[2 * m].x, x1 = d[2 * m + 1].x, y0 = d[2 * m].y, y1 = d[2 * m + 1].y;
    o[0].w[m] = (x0 & 0xffffu) | (x1 << 16);
    o[1].w[m] = (x0 >> 16) | (x1 & 0xffff0000u);
    o[2].w[m] = (y0 & 0xffffu) | (y1 << 16);
    o[3].w[m] = (y0 >> 16) | (y1 & 0xffff0000u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = o[q].v;
}

template <Act A, bool JMajor>
__global__ void __launch_bounds__(kTw) skinny_wgrad_kernel(const SkinnyWgradArgs p) {
  using M = Mma<A>;
  typedef typename M::v8 v8;
  typedef typename M::f4 f4;
  __shared__ float red[kWw / 2][64 * kLs];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int i = lane & 15, g = lane >> 4;
  const int64_t Jt = p.J + (p.part_b ? 1 : 0);   // columns computed
  const int G = static_cast<int>((Jt + 63) / 64);
  const int64_t CB = p.Di / 64, T = CB * p.P;   // (channel block, token chunk) tiles
  // The G column groups of a tile read the same BIG slice: give them ids 8
  // apart (consecutive ids go to the 8 XCDs in turn) so they run on one XCD
  // and the later ones find the slice in its L2.
  const int64_t bid = blockIdx.x;
  const int64_t tile = (bid / (8 * G)) * 8 + bid % 8;
  const int grp = static_cast<int>((bid / 8) % G);
  if (tile >= T) return;
  const int64_t c0 = (tile % CB) * 64, pc = tile / CB;
  const int j0 = 64 * grp;
  const int64_t KS = (p.N + 31) / 32;
  const int64_t ks0 = pc * p.chunk;
  const int64_t ks1 = ks0 + p.chunk < KS ? ks0 + p.chunk : KS;
  const uint16_t* big = static_cast<const uint16_t*>(p.big) + c0 + 4 * i;
  const bool jok = j0 + 4 * i < p.J;
  // the lane whose 4 columns start at J, when J is the ones column
  const bool jone = p.part_b != nullptr && j0 + 4 * i == p.J;
  const uint32_t one = A == Act::BF16 ? 0x3f80u : 0x3c00u;   // 1.0
  const uint16_t* small = static_cast<const uint16_t*>(p.small) + (jok ? j0 + 4 * i : 0);
  f4 acc[4][4];
#pragma unroll
  for (int qa = 0; qa < 4; ++qa)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) acc[qa][qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // One step's loads run ahead of the products.  The loads are unconditional
  // (tokens past N reload token N - 1, the last step reloads itself); the
  // narrow side is zeroed where it is used for tokens past N and columns past
  // J, so no load waits on a select.
  uint2 db[8], ds[8], dbn[8], dsn[8];
  auto fetch = [&](int64_t ks, uint2(&b)[8], uint2(&sm)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      int64_t n = 32 * ks + 8 * g + t;
      n = n < p.N ? n : p.N - 1;
      b[t] = *reinterpret_cast<const uint2*>(big + n * p.Di);
      sm[t] = *reinterpret_cast<const uint2*>(small + n * p.lds);
    }
  };
  if (ks0 + w < ks1) fetch(ks0 + w, db, ds);
  for (int64_t ks = ks0 + w; ks < ks1; ks += kWw) {
    fetch(ks + kWw < ks1 ? ks + kWw : ks, dbn, dsn);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (!jok) ds[t] = make_uint2(jone ? one : 0u, 0u);
      if (32 * ks + 8 * g + t >= p.N) ds[t] = make_uint2(0u, 0u);
    }
    v8 a[4], b[4];
    pack4(db, a);
    pack4(ds, b);
#pragma unroll
    for (int qa = 0; qa < 4; ++qa)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) acc[qa][qb] = M::mma(a[qa], b[qb], acc[qa][qb]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      db[t] = dbn[t];
      ds[t] = dsn[t];
    }
  }
  // accumulator lane (i, g), element e of product (qa, qb): channel
  // c0 + 4 (4 g + e) + qa, column j0 + 4 i + qb; kept at LDS row
  // 16 g + 4 e + qa, word 16 qb + i.  Waves 2 and 3 store their tiles,
  // waves 0 and 1 add theirs to them (each lane to the words it stored).
  float* mine = red[w & 1];
  if (w >= 2) {
#pragma unroll
    for (int qa = 0; qa < 4; ++qa)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[(16 * g + 4 * e + qa) * kLs + 16 * qb + i] = acc[qa][qb][e];
  }
  __syncthreads();
  if (w < 2) {
#pragma unroll
    for (int qa = 0; qa < 4; ++qa)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float& r = mine[(16 * g + 4 * e + qa) * kLs + 16 * qb + i];
          r = acc[qa][qb][e] + r;
        }
  }
  __syncthreads();
  float* part = p.part + pc * p.Di * p.J;
  for (int e = threadIdx.x; e < 64 * 64; e += kTw) {
    const int cl = JMajor ? e % 64 : e / 64, jl = JMajor ? e / 64 : e % 64;
    if (j0 + jl >= Jt) continue;
    const int at = cl * kLs + 16 * (jl & 3) + (jl >> 2);
    const float s = red[0][at] + red[1][at];
    if (j0 + jl == p.J) p.part_b[pc * p.Di + c0 + cl] = s;
    else if (JMajor) part[static_cast<int64_t>(j0 + jl) * p.Di + c0 + cl] = s;
    else part[(c0 + cl) * p.J + j0 + jl] = s;
  }
}

}  // namespace

bool skinny_wgrad_supported(Act act, int64_t N, int64_t Di, int64_t J, int64_t lds) {
  return (act == Act::BF16 || act == Act::F16) && N >= 1 && Di >= 64 && Di % 64 == 0 && J >= 4 && J % 4 == 0 &&
         J <= lds && lds % 4 == 0;
}

int64_t skinny_wgrad_chunks(int64_t N, int64_t Di, int64_t J, int64_t* chunk) {
  // (the launch rounds the tiles up to a multiple of 8 per column group)
  const int64_t KS = (N + 31) / 32, tiles = (Di / 64) * ((J + 64) / 64);
  int64_t P = (768 + tiles - 1) / tiles;   // about three workgroups per CU
  const int64_t by_steps = KS / 8;   // at least 8 token steps (2 per wave) per chunk
  P = P < by_steps ? P : by_steps;
  P = P < 1 ? 1 : P;
  const int64_t c = (KS + P - 1) / P;
  if (chunk) *chunk = c;
  return (KS + c - 1) / c;
}

hipError_t launch_skinny_wgrad(const SkinnyWgradArgs& p, Act act, bool j_major, hipStream_t st) {
  const int64_t T = (p.Di / 64) * p.P, Jt = p.J + (p.part_b ? 1 : 0);
  const dim3 grid(static_cast<unsigned>((T + 7) / 8 * 8 * ((Jt + 63) / 64))), blk(kTw);
  if (act == Act::BF16) {
    if (j_major) hipLaunchKernelGGL((skinny_wgrad_kernel<Act::BF16, true>), grid, blk, 0, st, p);
    else hipLaunchKernelGGL((skinny_wgrad_kernel<Act::BF16, false>), grid, blk, 0, st, p);
  } else {
    if (j_major) hipLaunchKernelGGL((skinny_wgrad_kernel<Act::F16, true>), grid, blk, 0, st, p);
    else hipLaunchKernelGGL((skinny_wgrad_kernel<Act::F16, false>), grid, blk, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mlayer
