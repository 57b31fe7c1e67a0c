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
  ConvSiluFwd,       // x c0, conv_w f0, conv_b f1 -> u v0; T, cols = d_inner, K, n
  ConvBwd,           // x c0, conv_w f0, conv_b f1, d_u c1 (act), d_u_extra f2 -> d_x v0 (act),
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
  int K = 0;
  float eps = 0.0f;
};

hipError_t launch(const Op& o, mscan::Act act, hipStream_t st);

// step tiles per batch row of the conv kernels (their weight partials come
// one per batch row and tile)
int64_t conv_step_tiles(int64_t T);

}  // namespace mlayer
