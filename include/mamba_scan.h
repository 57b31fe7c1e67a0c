/*
 * mamba_scan.h: C ABI of the MI355X (gfx950) selective-scan layer core.
 *
 * Computes the Mamba-1 selective-scan layer core for training, as laid out
 * on the mamba-rs pages:
 *   - "mamba-rs 0.3.1 src/mamba_ssm/gpu/forward_mixed.rs": the per-layer
 *     forward steps F4a (causal depthwise conv1d with carried f32 state,
 *     then SiLU), F4c (softplus of delta_raw), F4d (the SSM scan over
 *     u, delta, B, C with a_neg and the D skip term, f32 state) and F4e
 *     (gating y * silu(gate)); the GpuMambaLayerMixedActs struct (tensor
 *     shapes; f32 state; typed activations; y saved for the backward);
 *     and the GpuMambaMixedTrainScratch struct (the backward's outputs:
 *     d_y, d_gate, d_delta / d_delta_raw, d_u, d_B / d_C reduced over
 *     channels, per-sample d_D and d_a_log, conv weight and bias grads).
 *   - "mamba-rs 0.7.3 src/mamba_ssm/gpu/trainer.rs": A = -exp(a_log)
 *     (recompute_a_neg_all) and the recurrent state kept across calls
 *     (conv state [B, d_inner, d_conv], ssm state [B, d_inner, d_state]).
 *
 * Per channel i of batch row b (n runs over the d_state states):
 *   u_t     = silu(conv_b[i] + sum_k conv_w[i,k] x_{t-K+1+k})  (fused entry)
 *           = u given directly                                  (scan entry)
 *   delta_t = softplus(delta_raw_t),        A[i,n] = -exp(a_log[i,n])
 *   h_t[n]  = exp(delta_t A[i,n]) h_{t-1}[n] + delta_t B_t[n] u_t    (f32)
 *   y_t     = sum_n C_t[n] h_t[n] + D[i] u_t
 *   out_t   = y_t * silu(z_t)   (y_t when z is NULL)
 * B_t and C_t are columns [R, R+Ds) and [R+Ds, R+2Ds) of the xdbl row.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and completes
 *     asynchronously.  A kernel fault surfaces at the caller's next
 *     synchronisation.
 *   - Layouts are dense row-major with channels fastest:
 *       activations (u, x, delta_raw, z, out, y, dout and their grads):
 *                         [B, T, Di] of dims->act
 *       xdbl, d_xdbl:     [B, T, R + 2 Ds]   (xdbl of dims->act, d_xdbl f32)
 *       a_log, d_a_log:   [Di, Ds] f32        D, d_D, conv_b, d_conv_b: [Di] f32
 *       conv_w, d_conv_w: [Di, K] f32
 *       h0, h_last:       [B, Di, Ds] f32
 *       conv_state0, conv_state_last: [B, Di, K] f32, the K most recent
 *                         inputs, oldest first (only the last K-1 entries of
 *                         an incoming state reach the output)
 *       ckpt:             [B, ceil(T/L), Ds, Di] f32; ckpt[b, c] is the
 *                         state entering step c*L (ckpt[b, 0] = h0)
 *   - The activation inputs read in bulk (u or x, delta_raw, z, dout,
 *     y_saved) must be 4-byte aligned for 16-bit types and 16-byte aligned
 *     for f32; every other activation pointer needs its element alignment,
 *     every f32 pointer 4 bytes.  Inputs and outputs must not overlap.
 *   - Parameter gradients (d_a_log, d_D, d_conv_w, d_conv_b) and the B/C
 *     columns of d_xdbl are ACCUMULATED (+=): zero them once per training
 *     step.  The dt columns [0, R) of d_xdbl are never touched.
 *     Activation gradients are overwritten.  No gradient flows into h0 or
 *     conv_state0 (truncated backpropagation through time).
 *   - Every argument is checked before anything is enqueued.  A failed call
 *     returns a non-zero mamba_status_t, enqueues nothing (or, for
 *     MAMBA_ERR_HIP, stops at the failing launch) and leaves a message
 *     naming the entry point in mamba_last_error().
 *   - Half-precision outputs are rounded to nearest even.
 *
 * Segmented schedule.  When too few (batch row, channel group) pairs would
 * fill the GPU, the sequence is cut into segments that are scanned in
 * parallel, in the spirit of the parallel prefix scan the forward_mixed
 * page's F4d step switches to for long sequences.  The
 * recurrence is affine in the state, so a segment started from zero yields
 * its end state H_s, and the product of its dA is exp(A * sum of delta):
 *   forward : an aggregate pass gives (H_s, sum delta) per segment; the main
 *             pass starts segment s from the fold of the earlier pairs
 *             (h <- exp(A sum delta) h + H), starting at h0.
 *   backward: an aggregate pass runs each segment's adjoint of h from a zero
 *             carry, giving the carry it hands to the earlier steps; the main
 *             pass starts segment s from the fold of the later segments'
 *             pairs.
 * The schedule changes only the order of floating-point operations.  The
 * fused backward always sweeps whole sequences (its conv tail would cross
 * segment borders).  The pairs live in the workspace.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 3

typedef enum mamba_dtype { MAMBA_F32 = 0, MAMBA_BF16 = 1, MAMBA_F16 = 2 } mamba_dtype_t;

typedef enum mamba_status {
  MAMBA_OK = 0,
  MAMBA_ERR_INVALID = 1,     /* bad dimension, NULL required pointer, misalignment */
  MAMBA_ERR_UNSUPPORTED = 2, /* valid but not compiled: d_state / chunk / d_conv combination */
  MAMBA_ERR_CAPACITY = 3,    /* sizes beyond the launch limits, or workspace too small */
  MAMBA_ERR_HIP = 4          /* a HIP launch failed */
} mamba_status_t;

typedef struct mamba_dims {
  int64_t batch;    /* B, 1 .. 65535 */
  int64_t seqlen;   /* T >= 1 */
  int64_t d_inner;  /* Di >= 4, a multiple of 4 (the pages' MambaConfig rule), <= 2^24 */
  int64_t d_state;  /* Ds in {4, 8, 16, 32, 64} */
  int64_t dt_rank;  /* R in 0 .. 2^24: xdbl row = [dt (R) | B (Ds) | C (Ds)] */
  int32_t d_conv;   /* K in 1..4 for the fused entry points; ignored by mamba_scan_* */
  int32_t chunk;    /* checkpoint interval L: a multiple of 16 up to 4096;
                       0 = 64.  The backward re-runs the recurrence over
                       tiles of 16 (or, where compiled, 32) steps held in
                       registers; for a longer L it first regenerates the
                       states at every 16th step from the checkpoints
                       (into its workspace), trading one more forward pass
                       for L/16 times less checkpoint memory */
  int32_t act;      /* mamba_dtype_t of every activation tensor (and xdbl) */
  int32_t segments; /* sequence segments scanned in parallel (see below):
                       0 = chosen from the sizes; n in 1 .. 4096 = n
                       segments in both passes, fewer only when the
                       sequence has fewer tiles (1 = one sweep per channel
                       group); the fused backward always uses 1 */
} mamba_dims_t;

/* Version of this ABI (MAMBA_SCAN_ABI_VERSION of the built library). */
int mamba_abi_version(void);

/* Message of the calling thread's last failed call; "" after a success.
   Valid until the thread's next call into the library. */
const char* mamba_last_error(void);

/* Bytes of the f32 checkpoint buffer: B * ceil(T/L) * Ds * Di * 4. */
int mamba_ckpt_bytes(const mamba_dims_t* dims, size_t* bytes);

/* Bytes of device scratch the entry points need: an f32 copy of the B / C
   columns (forward for T > 16; backward when it regenerates checkpoints),
   the backward's per-group partial sums (reduced in a fixed order, so the
   result is run-to-run reproducible), the segment pairs of the segmented
   schedule and the regenerated 16-step checkpoints.  One buffer of this
   size serves the forward and the backward of these dims. */
int mamba_workspace_bytes(const mamba_dims_t* dims, size_t* bytes);

/*
 * Forward of the scan (steps F4c, F4d and F4e on the forward_mixed page).
 *   u, delta_raw, xdbl [act]; a_log f32; D f32 or NULL (= 0);
 *   z [act] or NULL (no gate); h0 f32 or NULL (= zeros).
 * Outputs: out [act]; y_save [act] or NULL: the pre-gate y (saved
 *   activation for the backward; required later when z is given);
 *   h_last f32 or NULL; ckpt f32 or NULL (needed by the backward).
 * workspace: device scratch of at least mamba_workspace_bytes(dims) bytes
 *   (NULL allowed when T <= 16: the short-sequence path needs none),
 *   contents irrelevant on entry.
 */
int mamba_scan_fwd(const mamba_dims_t* dims, const void* u, const void* delta_raw,
                   const float* a_log, const void* xdbl, const float* D, const void* z,
                   const float* h0, void* out, void* y_save, float* h_last, float* ckpt,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of mamba_scan_fwd (the reverse-time adjoint) for a given dout.
 * Inputs as in the forward, plus y_saved [act] (required when z is given),
 * ckpt from the forward with the same dims, and dout [act].
 * Outputs: d_u, d_delta_raw [act] (overwritten); d_z [act] (required
 *   when z is given, overwritten); d_xdbl f32 (B/C columns +=);
 *   d_a_log, d_D f32 (+=).  workspace: device scratch of at least
 *   mamba_workspace_bytes(dims) bytes, contents irrelevant on entry.
 */
int mamba_scan_bwd(const mamba_dims_t* dims, const void* u, const void* delta_raw,
                   const float* a_log, const void* xdbl, const float* D, const void* z,
                   const void* y_saved, const float* ckpt, const void* dout, void* d_u,
                   void* d_delta_raw, void* d_z, float* d_xdbl, float* d_a_log, float* d_D,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mamba_scan_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc).  Same arguments,
 * outputs and accumulation as mamba_scan_bwd; its scratch (the per-group
 * partial sums and segment pairs) lives in a static device array of
 * MAMBA_STATIC_SCRATCH_BYTES per GPU, set up on the first call on a device
 * (with that device current) and held until the process ends.  The call
 * allocates and frees nothing.  Dims whose scratch (mamba_workspace_bytes)
 * exceeds the array return MAMBA_ERR_CAPACITY before anything is enqueued.
 * All calls on one GPU share its array: calls that may overlap on that GPU
 * (other streams, other threads) race and must be serialised by the
 * caller.  `stream` must belong to the current device.
 */
#define MAMBA_STATIC_SCRATCH_BYTES (64u << 20)

int mamba_scan_bwd_static(const mamba_dims_t* dims, const void* u, const void* delta_raw,
                          const float* a_log, const void* xdbl, const float* D, const void* z,
                          const void* y_saved, const float* ckpt, const void* dout, void* d_u,
                          void* d_delta_raw, void* d_z, float* d_xdbl, float* d_a_log, float* d_D,
                          void* stream);

/*
 * Fused forward: causal depthwise conv1d (dims->d_conv taps) + SiLU, then
 * the scan and the gate (steps F4a..F4e on the forward_mixed page).
 *   x [act]: conv input; conv_w f32; conv_b f32 or NULL (= 0);
 *   conv_state0 f32 or NULL (= zeros); the rest as in mamba_scan_fwd.
 * Outputs: out [act]; u_out [act] or NULL: the conv+SiLU output;
 *   y_save, h_last, ckpt as in mamba_scan_fwd; conv_state_last f32 or NULL.
 * workspace: as in mamba_scan_fwd.
 */
int mamba_conv_scan_gate_fwd(const mamba_dims_t* dims, const void* x, const float* conv_w,
                             const float* conv_b, const float* conv_state0, const void* delta_raw,
                             const float* a_log, const void* xdbl, const float* D, const void* z,
                             const float* h0, void* out, void* u_out, void* y_save,
                             float* h_last, float* conv_state_last, float* ckpt,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of mamba_conv_scan_gate_fwd.  d_u_extra [act] or NULL: an extra
 * gradient on the conv+SiLU output u (from the x_proj path of a full layer),
 * added before the SiLU and conv backward.
 * Outputs: d_x, d_delta_raw [act] (overwritten); d_z [act] (required when z
 *   is given); d_xdbl, d_a_log, d_D, d_conv_w, d_conv_b f32 (+=).
 */
int mamba_conv_scan_gate_bwd(const mamba_dims_t* dims, const void* x, const float* conv_w,
                             const float* conv_b, const float* conv_state0, const void* delta_raw,
                             const float* a_log, const void* xdbl, const float* D, const void* z,
                             const void* y_saved, const float* ckpt, const void* dout,
                             const void* d_u_extra, void* d_x, void* d_delta_raw, void* d_z,
                             float* d_xdbl, float* d_a_log, float* d_D, float* d_conv_w,
                             float* d_conv_b, void* workspace, size_t workspace_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
