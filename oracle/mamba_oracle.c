/*
 * Plain CPU oracle for the Mamba-1 selective-scan layer core (training
 * forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP path is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may build,
 * load or call it; the product path never does.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * Sources (the mamba-rs pages):
 *  - "mamba-rs 0.3.1 src/mamba_ssm/gpu/forward_mixed.rs", the saved
 *    activation struct GpuMambaLayerMixedActs (conv state, post_conv, u,
 *    delta_raw, delta, h_saved = state BEFORE each step, da_exp =
 *    exp(delta*A), y, gated = y * silu(gate)) and the per-layer forward
 *    steps F4a (causal conv + state), F4c (softplus on delta_raw),
 *    F4d (SSM scan with a_neg and d_param) and F4e (gating).
 *  - "mamba-rs 0.7.3 src/mamba_ssm/gpu/trainer.rs", recompute_a_neg_all:
 *    A = -exp(a_log).
 *  - "mamba-rs 0.3.1 ... forward_mixed.rs", GpuMambaMixedTrainScratch:
 *    the backward produces d_y, d_gate, d_B/d_C (reduced over channels),
 *    d_delta, d_u, d_D and d_a_log per sample, d_delta_raw (softplus
 *    backward) and conv weight/bias grads.
 *
 * Everything is double precision (the type `real` below) and sequential in
 * time.  Per (b, i)
 * channel the forward is
 *     u_t      = silu(conv_b[i] + sum_k conv_w[i,k] x_{t-K+1+k})   (fused)
 *              = x_t                                               (no conv)
 *     delta_t  = softplus(delta_raw_t)
 *     A_n      = -exp(a_log[i,n])
 *     h_t[n]   = exp(delta_t A_n) h_{t-1}[n] + delta_t B_t[n] u_t
 *     y_t      = sum_n C_t[n] h_t[n] + D_i u_t
 *     out_t    = y_t * silu(z_t)   (or y_t without a gate)
 * and the backward is the exact reverse-time adjoint of those lines.
 * Readings taken where the pages are silent are listed next to the code.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <tgmath.h>

/* The parity build is double precision (the default).  Building with
 * -DORA_REAL=float gives the same code in single precision; that build
 * only times the oracle on the host and never serves as a reference. */
#ifndef ORA_REAL
#define ORA_REAL double
#endif
typedef ORA_REAL real;
#define RC(c) ((real)(c))

typedef struct {
  int64_t batch;    /* B */
  int64_t seqlen;   /* T */
  int64_t d_inner;  /* Di: channels */
  int64_t d_state;  /* Ds: states per channel */
  int64_t dt_rank;  /* R: xdbl row = [dt (R) | B (Ds) | C (Ds)] */
  int64_t d_conv;   /* K taps; 0 = no convolution, x is u */
  int64_t chunk;    /* checkpoint interval L (>= 1) */
} ora_dims;

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static real ora_softplus(real x) {
  return (x > RC(0) ? x : RC(0)) + log1p(exp(-fabs(x)));
}

/* logistic sigmoid, evaluated on the side where exp() cannot overflow. */
static real ora_sigmoid(real x) {
  if (x >= RC(0)) return RC(1) / (RC(1) + exp(-x));
  real e = exp(x);
  return e / (RC(1) + e);
}

static real ora_silu(real x) { return x * ora_sigmoid(x); }

/* d silu / dx = s (1 + x (1 - s)), s = sigmoid(x) */
static real ora_dsilu(real x) {
  real s = ora_sigmoid(x);
  return s * (RC(1) + x * (RC(1) - s));
}

static int ora_check(const ora_dims* d) {
  if (!d) return 1;
  if (d->batch < 1 || d->seqlen < 1 || d->d_inner < 1 || d->d_state < 1) return 1;
  if (d->dt_rank < 0 || d->d_conv < 0 || d->chunk < 1) return 1;
  return 0;
}

/* Input of the causal convolution at time s for channel i of batch b.
 * Reading (the pages give only the [B*d_inner*d_conv] state shape):
 * the state holds the K most recent inputs, oldest first; positions s < 0
 * read state[K + s], so only its last K-1 entries are ever used. */
static real ora_conv_in(const ora_dims* d, const real* x, const real* conv_state0,
                          int64_t b, int64_t i, int64_t s) {
  const int64_t T = d->seqlen, Di = d->d_inner, K = d->d_conv;
  if (s >= 0) return x[(b * T + s) * Di + i];
  if (!conv_state0) return RC(0);
  return conv_state0[(b * Di + i) * K + (K + s)];
}

/* Pre-activation of the convolution at time t: conv_b[i] + sum_k w[i,k] x_{t-K+1+k}. */
static real ora_conv_pre(const ora_dims* d, const real* x, const real* conv_w,
                           const real* conv_b, const real* conv_state0,
                           int64_t b, int64_t i, int64_t t) {
  const int64_t K = d->d_conv;
  real p = conv_b ? conv_b[i] : RC(0);
  for (int64_t k = 0; k < K; ++k)
    p += conv_w[i * K + k] * ora_conv_in(d, x, conv_state0, b, i, t - K + 1 + k);
  return p;
}

/*
 * One channel's forward pass.  Fills u[T], delta[T], the state history
 * hist[(T+1)*Ds] (hist[t+1] = h_t, hist[0] = h_{-1} = h0) and y[T].
 */
static void ora_channel_forward(const ora_dims* d, int64_t b, int64_t i,
                                const real* x, const real* conv_w, const real* conv_b,
                                const real* conv_state0, const real* delta_raw,
                                const real* a_log, const real* xdbl, const real* D,
                                const real* h0, real* u, real* delta, real* hist,
                                real* y) {
  const int64_t T = d->seqlen, Di = d->d_inner, Ds = d->d_state, R = d->dt_rank;
  const int64_t X = R + 2 * Ds;
  for (int64_t n = 0; n < Ds; ++n) hist[n] = h0 ? h0[(b * Di + i) * Ds + n] : RC(0);
  for (int64_t t = 0; t < T; ++t) {
    const int64_t row = b * T + t;
    real ut;
    if (d->d_conv > 0)
      ut = ora_silu(ora_conv_pre(d, x, conv_w, conv_b, conv_state0, b, i, t));
    else
      ut = x[row * Di + i];
    const real dt = ora_softplus(delta_raw[row * Di + i]);
    u[t] = ut;
    delta[t] = dt;
    real yt = RC(0);
    for (int64_t n = 0; n < Ds; ++n) {
      const real A = -exp(a_log[i * Ds + n]);
      const real Bn = xdbl[row * X + R + n];
      const real Cn = xdbl[row * X + R + Ds + n];
      const real hprev = hist[t * Ds + n];
      const real h = exp(dt * A) * hprev + dt * Bn * ut;
      hist[(t + 1) * Ds + n] = h;
      yt += Cn * h;
    }
    y[t] = yt + (D ? D[i] : RC(0)) * ut;
  }
}

/*
 * Forward over batch rows [b_begin, b_end) and channels [i_begin, i_end).
 * Channels never interact in the forward, so any split of them gives the
 * same values.  Output pointers other than `out` may be NULL.  Layouts (row-major):
 *   x, delta_raw, z, out, y_out, u_out : [B, T, Di]
 *   xdbl                               : [B, T, R + 2 Ds]
 *   a_log                              : [Di, Ds]
 *   D, conv_b                          : [Di]
 *   conv_w                             : [Di, K]
 *   h0, h_last                         : [B, Di, Ds]
 *   conv_state0, conv_state_last       : [B, Di, K]
 *   ckpt                               : [B, ceil(T/L), Ds, Di],
 *                                        ckpt[b, c, n, i] = state entering
 *                                        step c*L (so ckpt[b, 0] = h0).
 * Returns 0, or 1 on bad arguments, 2 on allocation failure.
 */
int ora_forward(const ora_dims* d, int64_t b_begin, int64_t b_end, int64_t i_begin,
                int64_t i_end, const real* x,
                const real* conv_w, const real* conv_b, const real* conv_state0,
                const real* delta_raw, const real* a_log, const real* xdbl,
                const real* D, const real* z, const real* h0, real* out,
                real* y_out, real* u_out, real* h_last, real* conv_state_last,
                real* ckpt) {
  if (ora_check(d) || !x || !delta_raw || !a_log || !xdbl || !out) return 1;
  if (d->d_conv > 0 && !conv_w) return 1;
  if (b_begin < 0 || b_end > d->batch || b_begin > b_end) return 1;
  if (i_begin < 0 || i_end > d->d_inner || i_begin > i_end) return 1;
  const int64_t T = d->seqlen, Di = d->d_inner, Ds = d->d_state, K = d->d_conv;
  const int64_t L = d->chunk, nC = (T + L - 1) / L;
  real* u = malloc(sizeof(real) * T);
  real* delta = malloc(sizeof(real) * T);
  real* y = malloc(sizeof(real) * T);
  real* hist = malloc(sizeof(real) * (T + 1) * Ds);
  if (!u || !delta || !y || !hist) {
    free(u); free(delta); free(y); free(hist);
    return 2;
  }
  for (int64_t b = b_begin; b < b_end; ++b) {
    for (int64_t i = i_begin; i < i_end; ++i) {
      ora_channel_forward(d, b, i, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D,
                          h0, u, delta, hist, y);
      for (int64_t t = 0; t < T; ++t) {
        const int64_t e = (b * T + t) * Di + i;
        out[e] = z ? y[t] * ora_silu(z[e]) : y[t];
        if (y_out) y_out[e] = y[t];
        if (u_out) u_out[e] = u[t];
      }
      if (h_last)
        for (int64_t n = 0; n < Ds; ++n) h_last[(b * Di + i) * Ds + n] = hist[T * Ds + n];
      if (ckpt)
        for (int64_t c = 0; c < nC; ++c)
          for (int64_t n = 0; n < Ds; ++n)
            ckpt[((b * nC + c) * Ds + n) * Di + i] = hist[(c * L) * Ds + n];
      if (conv_state_last && K > 0)
        /* the K most recent inputs, oldest first (taken from the incoming
           state when T < K) */
        for (int64_t k = 0; k < K; ++k)
          conv_state_last[(b * Di + i) * K + k] = ora_conv_in(d, x, conv_state0, b, i, T - K + k);
    }
  }
  free(u); free(delta); free(y); free(hist);
  return 0;
}

/*
 * Backward over batch rows [b_begin, b_end) and channels [i_begin, i_end):
 * the reverse-time adjoint of ora_forward for the loss
 * sum(dout * out) + sum(d_u_extra * u).
 *
 * Outputs (all written, none accumulated):
 *   d_x         [B,T,Di]  gradient w.r.t. x (w.r.t. u when d_conv == 0)
 *   d_delta_raw [B,T,Di]  gradient w.r.t. delta_raw (softplus backward)
 *   d_delta     [B,T,Di]  gradient w.r.t. delta = softplus(delta_raw); may be NULL
 *   d_z         [B,T,Di]  may be NULL when z is NULL
 *   d_xdbl      [B,T,X]   only the B and C columns of the rows
 *                         [b_begin, b_end) are written (zeroed, then the
 *                         channels [i_begin, i_end) summed in); the dt
 *                         columns are left untouched
 *   d_a_log     [Di,Ds], d_D [Di], d_conv_w [Di,K], d_conv_b [Di]:
 *                         channels [i_begin, i_end) only, summed over the
 *                         rows [b_begin, b_end)
 * No gradient is returned for h0 or conv_state0 (truncated BPTT).
 */
int ora_backward(const ora_dims* d, int64_t b_begin, int64_t b_end, int64_t i_begin,
                 int64_t i_end, const real* x,
                 const real* conv_w, const real* conv_b, const real* conv_state0,
                 const real* delta_raw, const real* a_log, const real* xdbl,
                 const real* D, const real* z, const real* h0, const real* dout,
                 const real* d_u_extra, real* d_x, real* d_delta_raw, real* d_delta,
                 real* d_z, real* d_xdbl, real* d_a_log, real* d_D, real* d_conv_w,
                 real* d_conv_b) {
  if (ora_check(d) || !x || !delta_raw || !a_log || !xdbl || !dout) return 1;
  if (!d_x || !d_delta_raw || !d_xdbl || !d_a_log || !d_D) return 1;
  if (z && !d_z) return 1;
  if (d->d_conv > 0 && (!conv_w || !d_conv_w || !d_conv_b)) return 1;
  if (b_begin < 0 || b_end > d->batch || b_begin > b_end) return 1;
  if (i_begin < 0 || i_end > d->d_inner || i_begin > i_end) return 1;
  const int64_t T = d->seqlen, Di = d->d_inner, Ds = d->d_state, R = d->dt_rank;
  const int64_t K = d->d_conv, X = R + 2 * Ds;

  real* u = malloc(sizeof(real) * T);
  real* delta = malloc(sizeof(real) * T);
  real* y = malloc(sizeof(real) * T);
  real* hist = malloc(sizeof(real) * (T + 1) * Ds);
  real* dy = malloc(sizeof(real) * T);
  real* du = malloc(sizeof(real) * T);
  real* dh = malloc(sizeof(real) * Ds);
  real* dA = malloc(sizeof(real) * Ds);
  real* dp = malloc(sizeof(real) * T);
  if (!u || !delta || !y || !hist || !dy || !du || !dh || !dA || !dp) {
    free(u); free(delta); free(y); free(hist); free(dy); free(du); free(dh); free(dA); free(dp);
    return 2;
  }

  for (int64_t i = i_begin; i < i_end; ++i) {
    for (int64_t n = 0; n < Ds; ++n) d_a_log[i * Ds + n] = RC(0);
    d_D[i] = RC(0);
    if (K > 0) {
      for (int64_t k = 0; k < K; ++k) d_conv_w[i * K + k] = RC(0);
      d_conv_b[i] = RC(0);
    }
  }
  for (int64_t b = b_begin; b < b_end; ++b)
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = R; j < X; ++j) d_xdbl[(b * T + t) * X + j] = RC(0);

  for (int64_t b = b_begin; b < b_end; ++b) {
    for (int64_t i = i_begin; i < i_end; ++i) {
      ora_channel_forward(d, b, i, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D,
                          h0, u, delta, hist, y);
      const real Di_ = D ? D[i] : RC(0);

      /* gating backward: out = y * silu(z) */
      for (int64_t t = 0; t < T; ++t) {
        const int64_t e = (b * T + t) * Di + i;
        if (z) {
          dy[t] = dout[e] * ora_silu(z[e]);
          d_z[e] = dout[e] * y[t] * ora_dsilu(z[e]);
        } else {
          dy[t] = dout[e];
        }
      }

      /* reverse-time pass through the recurrence */
      for (int64_t n = 0; n < Ds; ++n) { dh[n] = RC(0); dA[n] = RC(0); }
      for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = b * T + t;
        const int64_t e = row * Di + i;
        const real dt = delta[t], ut = u[t];
        real du_t = Di_ * dy[t];   /* y = ... + D u */
        real ddelta_t = RC(0);
        d_D[i] += dy[t] * ut;
        for (int64_t n = 0; n < Ds; ++n) {
          const real A = -exp(a_log[i * Ds + n]);
          const real Bn = xdbl[row * X + R + n];
          const real Cn = xdbl[row * X + R + Ds + n];
          const real hprev = hist[t * Ds + n];
          const real h = hist[(t + 1) * Ds + n];
          const real decay = exp(dt * A);
          /* y_t = sum_n C_t[n] h_t[n] + ... */
          dh[n] += dy[t] * Cn;
          d_xdbl[row * X + R + Ds + n] += dy[t] * h;
          /* h_t = decay * h_{t-1} + delta_t B_t u_t */
          d_xdbl[row * X + R + n] += dh[n] * dt * ut;
          du_t += dh[n] * dt * Bn;
          ddelta_t += dh[n] * (Bn * ut + A * decay * hprev);
          dA[n] += dh[n] * dt * decay * hprev;
          dh[n] *= decay; /* now the part of dL/dh_{t-1} coming from step t */
        }
        du[t] = du_t;
        if (d_delta) d_delta[e] = ddelta_t;
        /* delta = softplus(delta_raw): d softplus / dx = sigmoid(x) */
        d_delta_raw[e] = ddelta_t * ora_sigmoid(delta_raw[e]);
      }
      /* A = -exp(a_log): dA/da_log = -exp(a_log) = A */
      for (int64_t n = 0; n < Ds; ++n) d_a_log[i * Ds + n] += dA[n] * (-exp(a_log[i * Ds + n]));

      if (d_u_extra)
        for (int64_t t = 0; t < T; ++t) du[t] += d_u_extra[(b * T + t) * Di + i];

      if (K > 0) {
        /* u = silu(p), p = conv_b + sum_k w_k x_{t-K+1+k} */
        for (int64_t t = 0; t < T; ++t) {
          const real p = ora_conv_pre(d, x, conv_w, conv_b, conv_state0, b, i, t);
          dp[t] = du[t] * ora_dsilu(p);
          d_conv_b[i] += dp[t];
          for (int64_t k = 0; k < K; ++k)
            d_conv_w[i * K + k] += dp[t] * ora_conv_in(d, x, conv_state0, b, i, t - K + 1 + k);
        }
        for (int64_t s = 0; s < T; ++s) {
          real g = RC(0);
          for (int64_t k = 0; k < K; ++k) {
            const int64_t t = s + K - 1 - k; /* output step that reads x_s through tap k */
            if (t < T) g += conv_w[i * K + k] * dp[t];
          }
          d_x[(b * T + s) * Di + i] = g;
        }
      } else {
        for (int64_t t = 0; t < T; ++t) d_x[(b * T + t) * Di + i] = du[t];
      }
    }
  }
  free(u); free(delta); free(y); free(hist); free(dy); free(du); free(dh); free(dA); free(dp);
  return 0;
}
