/* C ABI of the Mamba-3 SISO state-space core on MI355X (gfx950).
 *
 * What is computed.  The mamba-rs 0.4.0 page
 * "src/mamba3_siso/gpu/backward_mixed.rs" shows the chunked state-space
 * block of a Mamba-3 SISO layer's backward (m3_extract_da_cs_sum,
 * m3_dqkv_typed, m3_dqktheta_typed, m3_ddt_dtrap, m3_angle_dt_bwd_seq,
 * m3_final_grads, bc_bias_add_bwd and the bias / dt-bias column sums) as
 * launches and arguments only.  These entry points compute that block's
 * forward and backward under the following reading of those names, per
 * batch row b and head h (x split into heads of `headdim` channels; head h
 * uses B/C group h / (heads / groups)):
 *   dt_t    = softplus(dd_dt_raw_t + dt_bias_h)
 *   A_t     = -max(softplus(dd_a_raw_t), a_floor)
 *   lam_t   = sigmoid(trap_raw_t)
 *   theta_t = sum_{s<=t} dt_s angles_raw_s                  (per head)
 *   K_t = rot(theta_t)(B_t + b_bias_h),  Q_t = rot(theta_t)(C_t + c_bias_h)
 *         (state pairs (a, a + n_angles), a < n_angles, turned by theta_t[a])
 *   S_t = exp(dt_t A_t) S_{t-1} + (1 - lam_t) dt_t exp(dt_t A_t) V_{t-1} K_{t-1}^T
 *         + lam_t dt_t V_t K_t^T,          S_{-1} = 0, S_t [headdim, d_state]
 *   y_t = S_t Q_t + D_h V_t
 * The kernels evaluate it in 64-step chunks (the state entering each chunk
 * is kept, in f32, in `states`); the result equals the step-by-step
 * definition up to rounding.
 *
 * Layouts (row-major, channels fastest): x, y, d_x [B, T, heads*headdim];
 * b_in, c_in, d_b_in, d_c_in [B, T, groups, d_state] (activation dtype);
 * dd_dt_raw, dd_a_raw, trap_raw and their gradients [B, T, heads] f32;
 * angles_raw, d_angles_raw [B, T, n_angles] f32; b_bias, c_bias and grads
 * [heads, d_state] f32; dt_bias, D and grads [heads] f32; states
 * [B, heads, ceil(T/64), headdim, d_state] f32.
 *
 * Ownership and errors: every pointer is caller-owned device memory; the
 * library allocates nothing and enqueues on `stream` (a hipStream_t, NULL
 * for the default stream).  Arguments are checked before anything is
 * enqueued; a failure returns a mamba_status_t code and mamba_last_error()
 * names the entry point.  Parameter gradients (d_b_bias, d_c_bias,
 * d_dt_bias, d_D) accumulate (+=); every other gradient is overwritten.
 * Activation pointers must be 16-byte aligned.
 */
#ifndef MAMBA3_H
#define MAMBA3_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t batch;      /* >= 1 */
  int64_t seqlen;     /* >= 1 */
  int64_t heads;      /* >= 1, a multiple of groups */
  int64_t headdim;    /* 64 */
  int64_t d_state;    /* 32, 64 or 128 (f32 activations: 32 or 64) */
  int64_t groups;     /* >= 1 */
  int64_t n_angles;   /* 0 .. d_state / 2 */
  int32_t chunk;      /* 0 or 64: steps per chunk */
  int32_t act;        /* mamba_dtype_t of x, b_in, c_in, y and their gradients */
  float a_floor;      /* >= 0: smallest decay rate |A| */
} mamba3_dims_t;

/* Bytes of the f32 chunk states the forward writes and the backward reads. */
int mamba3_states_bytes(const mamba3_dims_t* dims, size_t* bytes);

/* Bytes of device workspace one forward or backward call needs (the
 * backward's is the larger; one buffer of this size serves both).  A call
 * given fewer bytes than it needs returns MAMBA_ERR_CAPACITY. */
int mamba3_workspace_bytes(const mamba3_dims_t* dims, size_t* bytes);

/* Forward: y, and the state entering every chunk (for the backward). */
int mamba3_siso_fwd(const mamba3_dims_t* dims, const void* x, const void* b_in, const void* c_in,
                    const float* dd_dt_raw, const float* dd_a_raw, const float* trap_raw,
                    const float* angles_raw, const float* b_bias, const float* c_bias, const float* dt_bias,
                    const float* D, void* y, float* states, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Backward of sum(dy * y): every input's gradient.  `states` is what the
 * forward wrote for the same inputs. */
int mamba3_siso_bwd(const mamba3_dims_t* dims, const void* x, const void* b_in, const void* c_in,
                    const float* dd_dt_raw, const float* dd_a_raw, const float* trap_raw,
                    const float* angles_raw, const float* b_bias, const float* c_bias, const float* dt_bias,
                    const float* D, const float* states, const void* dy, void* d_x, void* d_b_in,
                    void* d_c_in, float* d_dd_dt_raw, float* d_dd_a_raw, float* d_trap_raw,
                    float* d_angles_raw, float* d_b_bias, float* d_c_bias, float* d_dt_bias, float* d_D,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA3_H */
