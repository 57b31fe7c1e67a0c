// Launch descriptions of the layer kernels (layer_kernels.hip), used by the
// layer entry points (layer_abi.hip).  One plain struct per launch; the
// fields each kind reads are listed beside it.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "scan_common.h"

namespace mlayer {

enum class OpKind {
  RmsnormFwd,        // x f0, w f1 -> y v0 (act), rstd f3; rows, cols = d_model, eps
  RmsnormBwd,        // dy f0, x f1, w f2, rstd f4, d_out f5 -> d_in f3; rows, cols
  RmsnormWgradPart,  // dy f0, x f1, rstd f2 -> part f3 [nblk, cols]; rows, cols, per_blk, nblk
  ConvSiluFwd,       // x c0 (rows ld apart), conv_w f0, conv_b f1 -> u v0; T, cols = d_inner, ld, K, n
  ConvBwd,           // x c0 (rows ld apart), conv_w f0, conv_b f1, d_u c1 (act), d_u_extra f2 -> d_x v0 (act,
                     // rows ld apart),
                     // part_w f3 [batch * ntiles, cols, K], part_b f6 [batch * ntiles, cols]; T, cols, K, n
                     // (ntiles = conv_step_tiles(T))
  BiasRound,         // dt f0, b f1 -> out v0 (act); cols = d_inner (% 4 == 0), n
  Cast,              // f0 -> v0 (act); n
  ColPart,           // m c0 (act) -> part f3 [nblk, cols]; rows, cols, per_blk, nblk
  ColSum,            // part f0 -> out f3 (+=); nblk, cols
  Zero,              // f3 = 0; n
};

struct Op {
  OpKind kind;
  const float* f0 = nullptr;
  const float* f1 = nullptr;
  const float* f2 = nullptr;
  float* f3 = nullptr;
  const float* f4 = nullptr;
  const float* f5 = nullptr;
  float* f6 = nullptr;
  const void* c0 = nullptr;
  const void* c1 = nullptr;
  void* v0 = nullptr;
  int64_t rows = 0, cols = 0, n = 0, T = 0, nblk = 0, per_blk = 0, nblk_t = 0;
  int64_t ld = 0;   // elements between rows of the conv kernels' x and d_x (0: cols)
  int K = 0;
  float eps = 0.0f;
};

hipError_t launch(const Op& o, mscan::Act act, hipStream_t st);

// The fused x_proj -> dt_proj products (layer_mfma.hip), 16-bit activations.
// Forward: xdbl [N, X] = round(u W_x^T), delta_raw [N, Di] = round(xdbl[:, :R]
// W_dt^T + b_dt).  Backward: d_xdbl_a [N, X] = round([d_delta_raw W_dt |
// the B / C columns of d_xdbl]), d_uex [N, Di] = d_xdbl_a W_x (f32), with
// W_dt and W_x transposed into w_dtT [R, Di] and w_xT [Di, X] first.
struct XdtArgs {
  const void* u = nullptr;        // fwd [N, Di]
  const void* w_x = nullptr;      // [X, Di]
  const void* w_dt = nullptr;     // [Di, R]
  const float* b_dt = nullptr;    // fwd [Di]
  void* xdbl = nullptr;           // fwd out [N, X]
  void* dr = nullptr;             // fwd out [N, Di]
  const void* d_dr = nullptr;     // bwd [N, Di]
  const float* d_xdbl = nullptr;  // bwd [N, X] f32 (its B / C columns)
  void* d_xdbl_a = nullptr;       // bwd out [N, X]
  float* d_uex = nullptr;         // bwd out [N, Di]
  void* w_dtT = nullptr;          // bwd scratch [R, Di]
  void* w_xT = nullptr;           // bwd scratch [Di, xdt_xT_stride(X)], zero padded
  float* part = nullptr;          // scratch: xdt_groups(N, Di) x N x (fwd X, bwd R) f32
  int64_t N = 0, Di = 0;
  int X = 0, R = 0;
};

// row stride (elements) of the transposed x_proj weight the backward keeps
__host__ __device__ inline int64_t xdt_xT_stride(int64_t X) { return (X + 7) / 8 * 8; }

// The long product over d_inner: part[g][n][c] = sum over the 32-wide k
// steps [g kchunk, (g + 1) kchunk) of a[n][k] b[c][k]; a [N][K], b [C][K]
// (16-bit, rows 16-byte aligned), part f32.
struct ContractArgs {
  const void* a = nullptr;
  const void* b = nullptr;
  float* part = nullptr;
  int64_t N = 0, K = 0;
  int C = 0;
  int64_t G = 1, kchunk = 1;
};

// The short product into the wide output: out[n][c] = sum_{k < kmax} x[n][k]
// w[c][k] (+ bias[c], rounded, forward; f32, backward); x [N][ldx], w
// [Di][ldw], out [N][Di].
struct ExpandArgs {
  const void* x = nullptr;
  const void* w = nullptr;
  const float* bias = nullptr;
  void* out = nullptr;
  int64_t ldx = 0, ldw = 0, N = 0, Di = 0;
  int kmax = 0;
  int64_t cpb = 1;   // 256-channel blocks per workgroup
};

// K groups of the long product (and its 32-wide k steps per group)
int64_t xdt_groups(int64_t N, int64_t K, int64_t* kchunk);

bool xdt_supported(const XdtArgs& p, mscan::Act act);
hipError_t launch_xdt_fwd(const XdtArgs& p, mscan::Act act, hipStream_t st);
// the backward's transposed weights (w_dtT, w_xT) from w_dt and w_x; before
// launch_xdt_bwd
hipError_t launch_xdt_bwd_prep(const XdtArgs& p, mscan::Act act, hipStream_t st);
hipError_t launch_xdt_bwd(const XdtArgs& p, mscan::Act act, hipStream_t st);

// part[P][...] (f32) = per-chunk token sums of BIG[n][c] SMALL[n][j] (c <
// Di, j < J): the gradient layout [Di][J], or [J][Di] when j_major.  BIG is
// [N, Di], SMALL [N, lds] (its first J columns), both 16-bit; P chunks of
// `chunk` 32-token steps.  With part_b (not j_major): part_b[P][Di] = the
// per-chunk token sums of BIG[n][c] (a column of ones past SMALL's J).
struct SkinnyWgradArgs {
  const void* big = nullptr;
  const void* small = nullptr;
  float* part = nullptr;
  float* part_b = nullptr;
  int64_t N = 0, Di = 0, J = 0, lds = 0, chunk = 1;
  int64_t P = 1;   // token chunks: ceil(ceil(N / 32) / chunk)
};

bool skinny_wgrad_supported(mscan::Act act, int64_t N, int64_t Di, int64_t J, int64_t lds);
// the chunk count P (and the 32-token steps per chunk)
int64_t skinny_wgrad_chunks(int64_t N, int64_t Di, int64_t J, int64_t* chunk);
hipError_t launch_skinny_wgrad(const SkinnyWgradArgs& p, mscan::Act act, bool j_major, hipStream_t st);

// step tiles per batch row of the conv kernels (their weight partials come
// one per batch row and tile)
int64_t conv_step_tiles(int64_t T);

}  // namespace mlayer
