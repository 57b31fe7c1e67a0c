/*
 * One whole Mamba-1 layer around the selective-scan core, forward and
 * backward, on MI355X (gfx950).  Part of libmamba_scan.so; the core entry
 * points are in mamba_scan.h.
 *
 * The steps are those of the per-layer forward on the mamba-rs 0.3.1
 * "src/mamba_ssm/gpu/forward_mixed.rs" page (its F1..F6 list and the
 * launches behind them):
 *   F1  xn = RMSNorm(resid_in) * norm_w, eps 1e-5, over d_model; the f32
 *       residual stream in, a typed output (act dtype)
 *   F2  in_proj: [x | z] = xn W_in^T, W_in [2*d_inner, d_model]; rows
 *       0 .. d_inner-1 of W_in give the x branch, the rest the gate input z
 *   F4a u = SiLU(causal depthwise conv1d(x) + conv_b), zero history
 *   F4b xdbl = u W_x^T, W_x [dt_rank + 2*d_state, d_inner] (dt | B | C)
 *   F4c delta_raw = xdbl[:, :dt_rank] W_dt^T + b_dt, W_dt [d_inner, dt_rank]
 *   F4d/e the selective-scan core (mamba_scan_fwd, gate z)
 *   F5  out_proj: o = gated W_out^T, W_out [d_model, d_inner]
 *   F6  resid_out = resid_in + o (f32)
 * The backward is the adjoint of each step in reverse order.  It ends in
 * d_resid_in = d_resid_out + the RMSNorm adjoint.
 *
 * Precision.  The projections take the activation-dtype weights (the
 * compute copies of f32 masters, which the caller keeps) and accumulate in
 * f32.  xn, x, z, u, xdbl, delta_raw and the gated scan output are stored in
 * the activation dtype (rounded to nearest even); so are the activation
 * gradients that feed a projection.  The residual stream, the RMSNorm
 * statistics and every parameter gradient are f32.
 *
 * Projections.  The dense products go through rocBLAS (gemm_ex, f32
 * compute, atomics disabled so that every result is reproducible run to
 * run).  One rocBLAS handle is created per device on the first layer call
 * (that call allocates the handle's own memory); later calls allocate
 * nothing.  Layer calls on one device from several host threads at once
 * are serialised.
 *
 * Streams.  The forward runs on `stream`.  The backward runs its weight-
 * gradient products on a second stream of the device (created, with its
 * own rocBLAS handle and events, on the first backward call; default
 * priority), each forked from `stream` once its operands are final, and
 * joins that stream back into `stream` before returning, also when it
 * fails: work enqueued on `stream` afterwards sees every result.  The
 * fork and join are event records and waits; the host never blocks.
 *
 * Buffers.  All pointers are caller-owned device memory, row-major:
 *   resid_in, resid_out, d_resid_out, d_resid_in: f32 [batch, seqlen, d_model]
 *   saved: mamba_layer_saved_bytes(dims) bytes; written by the forward,
 *          read by the backward of the same inputs and weights
 *   workspace: mamba_layer_workspace_bytes(dims) bytes; scratch of either
 *          call (one buffer can serve both, not at the same time)
 * Every pointer needs 16-byte alignment; saved and workspace 256.  All
 * weights are required.  Gradients are accumulated (+=) into the caller's
 * f32 buffers, which the caller zeroes once per step (the convention of
 * the mamba-rs 0.4.0 "src/mamba3_siso/gpu/backward_mixed.rs" page's
 * backbone backward).  Errors follow mamba_scan.h: a status code, nothing
 * enqueued on an argument error, and mamba_last_error() naming the entry
 * point.
 */
#ifndef MAMBA_LAYER_H
#define MAMBA_LAYER_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mamba_layer_dims {
  mamba_dims_t core; /* batch, seqlen, d_inner, d_state, dt_rank (>= 1),
                        d_conv (1 .. 4), chunk, act, segments of the core */
  int64_t d_model;   /* width of the residual stream, 1 .. 2^24 */
} mamba_layer_dims_t;

/* Device pointers; "act" = the activation dtype of dims.core.act. */
typedef struct mamba_layer_weights {
  const float* norm_w; /* [d_model] f32 */
  const void* w_in;    /* [2*d_inner, d_model] act */
  const float* conv_w; /* [d_inner, d_conv] f32 */
  const float* conv_b; /* [d_inner] f32 */
  const void* w_x;     /* [dt_rank + 2*d_state, d_inner] act */
  const void* w_dt;    /* [d_inner, dt_rank] act */
  const float* b_dt;   /* [d_inner] f32 */
  const float* a_log;  /* [d_inner, d_state] f32 */
  const float* D;      /* [d_inner] f32 */
  const void* w_out;   /* [d_model, d_inner] act */
} mamba_layer_weights_t;

/* f32 gradients of the weights above, same shapes, accumulated (+=). */
typedef struct mamba_layer_grads {
  float* norm_w;
  float* w_in;
  float* conv_w;
  float* conv_b;
  float* w_x;
  float* w_dt;
  float* b_dt;
  float* a_log;
  float* D;
  float* w_out;
} mamba_layer_grads_t;

/* Bytes of the saved-activation buffer and of the workspace. */
int mamba_layer_saved_bytes(const mamba_layer_dims_t* dims, size_t* bytes);
int mamba_layer_workspace_bytes(const mamba_layer_dims_t* dims, size_t* bytes);

/* Forward of one layer: resid_out = resid_in + out_proj(core(...)).  Fills
 * `saved` for the backward.  resid_out must not alias resid_in. */
int mamba_layer_fwd(const mamba_layer_dims_t* dims, const mamba_layer_weights_t* w, const float* resid_in,
                    float* resid_out, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Backward of one layer for the loss sum(d_resid_out * resid_out): writes
 * d_resid_in (may alias d_resid_out) and adds every weight gradient into
 * `grads`.  resid_in and saved must be those of the matching forward. */
int mamba_layer_bwd(const mamba_layer_dims_t* dims, const mamba_layer_weights_t* w, const float* resid_in,
                    const void* saved, size_t saved_bytes, const float* d_resid_out, float* d_resid_in,
                    const mamba_layer_grads_t* grads, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_LAYER_H */
