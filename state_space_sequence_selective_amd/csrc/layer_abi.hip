// C ABI of one whole Mamba-1 layer around the scan core (declared in
// include/mamba_layer.h): argument checks, the saved / workspace layouts,
// and the sequence of launches.  The per-layer forward follows the F1..F6
// steps of the mamba-rs 0.3.1 forward_mixed.rs page; the backward is their
// adjoint in reverse order.  Dense projections go to rocBLAS (gemm_ex, f32
// compute); every other step is a kernel of this library.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <climits>
#include <cstdint>
#include <mutex>
#include <string>

#include "layer_kernels.h"
#include "mamba_layer.h"
#include "mamba_scan.h"
#include "scan_strided.h"

namespace mscan {
void set_last_error(const std::string& msg);   // abi.hip
}

namespace {

using mlayer::Op;
using mlayer::OpKind;

constexpr float kNormEps = 1e-5f;   // the forward_mixed page's RMSNorm epsilon
constexpr size_t kAlign = 256;
constexpr int64_t kMaxModel = int64_t(1) << 24;
constexpr int64_t kPartBlocks = 128;   // row blocks of the fixed-order column reductions

int fail(int code, const char* fn, const std::string& msg) {
  mscan::set_last_error(std::string(fn) + ": " + msg);
  return code;
}

#define LAYER_TRY(expr)          \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != MAMBA_OK) return rc_; \
  } while (0)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct LPlan {
  mamba_dims_t core;
  int64_t B, T, N, Di, Ds, R, X, K, dm, es;
  mscan::Act act;
  size_t ckpt_bytes, core_ws;
  // saved
  size_t s_xn, s_rstd, s_x, s_z, s_u, s_xdbl, s_dr, s_gated, s_y, s_ckpt, s_total;
  // workspace: forward
  size_t w_dt, w_core_f, w_xpart, wf_total;
  // workspace: backward
  size_t w_dy, w_dgated, w_du, w_ddr, w_dz, w_dxdbl, w_dxdbl_a, w_duex, w_dx, w_dxn, w_pnorm, w_pbdt, w_pconv_w,
      w_pconv_b, w_pwg, w_core_b, w_dtT, w_xT, w_xpart_b, w_pskb, wb_total;
  int64_t norm_per, norm_nblk, bdt_per, bdt_nblk, conv_nblk;
  int64_t P_dt, P_x, P_wide;   // K chunks of the dt_proj / x_proj / in_proj and out_proj weight products
  // token chunks of the matrix-core dt_proj / x_proj weight products (0: the
  // library products) and their 32-token steps per chunk
  int64_t S_dt, S_x, S_dt_chunk, S_x_chunk;
  bool xdt;   // x_proj -> dt_proj (and the adjoint) on the matrix-core kernels
};

// K chunks for a weight product grad[M, N] += A^T B over K token rows.  Its
// output is small next to K, so a single product covers the chip with few
// tiles, each looping over all of K; P chunks run as one batched product
// into P partials that a fixed-order sum adds (no atomics).  P aims at
// about 512 tiles of 64 x 64 and keeps at least 256 rows per chunk.
int64_t wgrad_chunks(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t P = (512 + tiles - 1) / tiles;
  P = P < 16 ? P : 16;
  const int64_t by_rows = K / 256;
  P = P < by_rows ? P : by_rows;
  return P < 1 ? 1 : P;
}

// The same for the wide weight products (in_proj, out_proj: d_model x
// d_inner outputs): the library tiles them 128 x 64, so P aims at about 1024
// tiles of 64 x 64 and keeps at least 512 rows per chunk.
int64_t wgrad_chunks_wide(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t P = (1024 + tiles - 1) / tiles;
  P = P < 8 ? P : 8;
  const int64_t by_rows = K / 512;
  P = P < by_rows ? P : by_rows;
  return P < 1 ? 1 : P;
}

// Lays out consecutive 256-byte-aligned regions.
struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  }
};

int plan_layer(const mamba_layer_dims_t* d, const char* fn, LPlan* pl) {
  if (!d) return fail(MAMBA_ERR_INVALID, fn, "dims is NULL");
  if (d->d_model < 1) return fail(MAMBA_ERR_INVALID, fn, "d_model must be >= 1");
  if (d->d_model > kMaxModel) return fail(MAMBA_ERR_CAPACITY, fn, "d_model must be <= 2^24");
  if (d->core.d_conv < 1) return fail(MAMBA_ERR_INVALID, fn, "a layer has a conv: core.d_conv must be >= 1");
  if (d->core.dt_rank < 1) return fail(MAMBA_ERR_INVALID, fn, "a layer has a dt projection: core.dt_rank must be >= 1");
  size_t ck = 0, ws = 0;
  int rc = mamba_ckpt_bytes(&d->core, &ck);
  if (rc == MAMBA_OK) rc = mamba_workspace_bytes(&d->core, &ws);
  if (rc != MAMBA_OK) return fail(rc, fn, std::string("core dims: ") + mamba_last_error());
  pl->core = d->core;
  pl->B = d->core.batch;
  pl->T = d->core.seqlen;
  pl->N = pl->B * pl->T;
  pl->Di = d->core.d_inner;
  pl->Ds = d->core.d_state;
  pl->R = d->core.dt_rank;
  pl->X = pl->R + 2 * pl->Ds;
  pl->K = d->core.d_conv;
  pl->dm = d->d_model;
  pl->act = static_cast<mscan::Act>(d->core.act);
  pl->es = d->core.act == MAMBA_F32 ? 4 : 2;
  pl->ckpt_bytes = ck;
  pl->core_ws = ws;
  // rocBLAS takes 32-bit sizes and leading dimensions
  const int64_t big = pl->N > pl->dm ? pl->N : pl->dm;
  if (big > INT_MAX || 2 * pl->Di > INT_MAX)
    return fail(MAMBA_ERR_CAPACITY, fn, "batch * seqlen, d_model and 2 * d_inner must be < 2^31");
  if (pl->N * pl->dm > (int64_t(1) << 46))
    return fail(MAMBA_ERR_CAPACITY, fn, "batch * seqlen * d_model exceeds 2^46 elements");
  if (pl->K > 4) return fail(MAMBA_ERR_UNSUPPORTED, fn, "core.d_conv must be <= 4");

  const size_t es = static_cast<size_t>(pl->es), f = sizeof(float);
  const size_t N = static_cast<size_t>(pl->N), Di = static_cast<size_t>(pl->Di), dm = static_cast<size_t>(pl->dm),
               X = static_cast<size_t>(pl->X);
  Layout s;
  pl->s_xn = s.take(N * dm * es);
  pl->s_rstd = s.take(N * f);
  // x | z interleaved, rows of 2 d_inner: the one in_proj product's output
  pl->s_x = s.take(2 * N * Di * es);
  pl->s_z = pl->s_x + Di * es;
  pl->s_u = s.take(N * Di * es);
  pl->s_xdbl = s.take(N * X * es);
  pl->s_dr = s.take(N * Di * es);
  pl->s_gated = s.take(N * Di * es);
  pl->s_y = s.take(N * Di * es);
  pl->s_ckpt = s.take(ck);
  pl->s_total = s.off;

  Layout wf;
  pl->w_dt = wf.take(N * Di * f);
  {
    mlayer::XdtArgs q;
    q.N = pl->N;
    q.Di = pl->Di;
    q.X = static_cast<int>(pl->X);
    q.R = static_cast<int>(pl->R);
    pl->xdt = mlayer::xdt_supported(q, pl->act);
  }
  // partial sums of the matrix-core x_proj (K groups x N x X)
  const size_t xdt_G = pl->xdt ? static_cast<size_t>(mlayer::xdt_groups(pl->N, pl->Di, nullptr)) : 0;
  pl->w_xpart = wf.take(xdt_G * N * X * f);
  pl->w_core_f = wf.take(ws);
  pl->wf_total = wf.off;

  pl->norm_nblk = pl->N < kPartBlocks ? pl->N : kPartBlocks;
  pl->norm_per = (pl->N + pl->norm_nblk - 1) / pl->norm_nblk;
  pl->norm_nblk = (pl->N + pl->norm_per - 1) / pl->norm_per;
  pl->bdt_nblk = pl->norm_nblk;
  pl->bdt_per = pl->norm_per;
  // conv weight partials: one per (batch row, step tile)
  pl->conv_nblk = pl->B * mlayer::conv_step_tiles(pl->T);
  // row-blocked elementwise launches: rows * ceil(d_inner / 256) workgroups
  if (pl->N * ((pl->Di + 255) / 256) > static_cast<int64_t>(UINT_MAX))
    return fail(MAMBA_ERR_CAPACITY, fn, "batch * seqlen * ceil(d_inner / 256) must be < 2^32");
  const size_t nconv = static_cast<size_t>(pl->conv_nblk);
  Layout wb;
  pl->w_dy = wb.take(N * dm * es);
  pl->w_dgated = wb.take(N * Di * es);
  pl->w_du = wb.take(N * Di * es);
  pl->w_ddr = wb.take(N * Di * es);
  // d_x | d_z interleaved like x | z: the one in_proj input-gradient product's operand
  pl->w_dx = wb.take(2 * N * Di * es);
  pl->w_dz = pl->w_dx + Di * es;
  pl->w_dxdbl = wb.take(N * X * f);
  pl->w_dxdbl_a = wb.take(N * X * es);
  pl->w_duex = wb.take(N * Di * f);
  pl->w_dxn = wb.take(N * dm * f);
  pl->w_pnorm = wb.take(static_cast<size_t>(pl->norm_nblk) * dm * f);
  pl->w_pbdt = wb.take(static_cast<size_t>(pl->bdt_nblk) * Di * f);
  pl->w_pconv_w = wb.take(nconv * Di * static_cast<size_t>(pl->K) * f);
  pl->w_pconv_b = wb.take(nconv * Di * f);
  // partials of the split weight products (one region: they run in turn on
  // one stream): P chunks plus a tail chunk when P does not divide N
  pl->P_dt = wgrad_chunks(pl->Di, pl->R, pl->N);
  pl->P_x = wgrad_chunks(pl->X, pl->Di, pl->N);
  const size_t pdt = pl->P_dt > 1 ? static_cast<size_t>(pl->P_dt + 1) * Di * static_cast<size_t>(pl->R) : 0;
  const size_t px = pl->P_x > 1 ? static_cast<size_t>(pl->P_x + 1) * X * Di : 0;
  pl->P_wide = wgrad_chunks_wide(pl->Di, pl->dm, pl->N);
  const size_t pw = pl->P_wide > 1 ? static_cast<size_t>(pl->P_wide + 1) * Di * dm : 0;
  pl->S_dt = pl->S_x = 0;
  if (mlayer::skinny_wgrad_supported(pl->act, pl->N, pl->Di, pl->R, pl->X))
    pl->S_dt = mlayer::skinny_wgrad_chunks(pl->N, pl->Di, pl->R, &pl->S_dt_chunk);
  if (mlayer::skinny_wgrad_supported(pl->act, pl->N, pl->Di, pl->X, pl->X))
    pl->S_x = mlayer::skinny_wgrad_chunks(pl->N, pl->Di, pl->X, &pl->S_x_chunk);
  const size_t sdt = static_cast<size_t>(pl->S_dt) * Di * static_cast<size_t>(pl->R);
  const size_t sx = static_cast<size_t>(pl->S_x) * Di * X;
  size_t pmax = pdt > px ? pdt : px;
  pmax = pmax > pw ? pmax : pw;
  pmax = pmax > sdt ? pmax : sdt;
  pmax = pmax > sx ? pmax : sx;
  pl->w_pwg = wb.take(pmax * f);
  pl->w_core_b = wb.take(ws);
  // the fused x_proj / dt_proj adjoint reads W_dt and W_x transposed
  pl->w_dtT = wb.take(static_cast<size_t>(pl->R) * Di * es);
  pl->w_xT = wb.take(Di * mlayer::xdt_xT_stride(X) * es);
  pl->w_xpart_b = wb.take(xdt_G * N * static_cast<size_t>(pl->R) * f);
  // the dt bias partials beside the matrix-core dt_proj weight gradient
  pl->w_pskb = wb.take(static_cast<size_t>(pl->S_dt) * Di * f);
  pl->wb_total = wb.off;
  return MAMBA_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, size_t align) {
  if (!p) return fail(MAMBA_ERR_INVALID, fn, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(MAMBA_ERR_INVALID, fn, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return MAMBA_OK;
}

int check_weights(const char* fn, const mamba_layer_weights_t* w) {
  if (!w) return fail(MAMBA_ERR_INVALID, fn, "weights is NULL");
  LAYER_TRY(check_ptr(fn, "w.norm_w", w->norm_w, 16));
  LAYER_TRY(check_ptr(fn, "w.w_in", w->w_in, 16));
  LAYER_TRY(check_ptr(fn, "w.conv_w", w->conv_w, 16));
  LAYER_TRY(check_ptr(fn, "w.conv_b", w->conv_b, 16));
  LAYER_TRY(check_ptr(fn, "w.w_x", w->w_x, 16));
  LAYER_TRY(check_ptr(fn, "w.w_dt", w->w_dt, 16));
  LAYER_TRY(check_ptr(fn, "w.b_dt", w->b_dt, 16));
  LAYER_TRY(check_ptr(fn, "w.a_log", w->a_log, 16));
  LAYER_TRY(check_ptr(fn, "w.D", w->D, 16));
  LAYER_TRY(check_ptr(fn, "w.w_out", w->w_out, 16));
  return MAMBA_OK;
}

int check_buffer(const char* fn, const char* name, const void* p, size_t have, size_t need) {
  LAYER_TRY(check_ptr(fn, name, p, kAlign));
  if (have < need)
    return fail(MAMBA_ERR_CAPACITY, fn,
                std::string(name) + " holds " + std::to_string(have) + " bytes < required " + std::to_string(need));
  return MAMBA_OK;
}

// ------------------------------------------------------------- rocBLAS

std::mutex g_blas_mu;   // held for a whole layer call
rocblas_handle g_blas[64] = {};

int blas_handle(const char* fn, hipStream_t st, rocblas_handle* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MAMBA_ERR_HIP, fn, "no usable current device");
  if (!g_blas[dev]) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return fail(MAMBA_ERR_HIP, fn, "rocblas_create_handle failed");
    // no atomics: every product is reproducible run to run
    rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
    g_blas[dev] = h;
  }
  if (rocblas_set_stream(g_blas[dev], st) != rocblas_status_success)
    return fail(MAMBA_ERR_HIP, fn, "rocblas_set_stream failed");
  *out = g_blas[dev];
  return MAMBA_OK;
}

// The backward's weight-gradient products run on a second stream of the
// same device (default priority), forked from the caller's stream once
// their operands are final and joined back before the call returns.
struct Side {
  hipStream_t s = nullptr;
  rocblas_handle h = nullptr;
  hipEvent_t ev[7] = {};   // four forks and the join of one backward call; the weight transposes' fork and end
};
Side g_side[64];

// The device's side resources, created on first use; published only when
// every part was created, so a failed creation is retried by the next call
// (what it did create is released).
int side_res(const char* fn, Side** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MAMBA_ERR_HIP, fn, "no usable current device");
  if (!g_side[dev].s) {
    Side n;
    const char* what = nullptr;
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess) {
      n.s = nullptr;
      what = "hipStreamCreateWithFlags failed";
    }
    for (auto& e : n.ev)
      if (!what && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
        e = nullptr;
        what = "hipEventCreateWithFlags failed";
      }
    if (!what && rocblas_create_handle(&n.h) != rocblas_status_success) {
      n.h = nullptr;
      what = "rocblas_create_handle failed";
    }
    if (!what) {
      rocblas_set_atomics_mode(n.h, rocblas_atomics_not_allowed);
      if (rocblas_set_stream(n.h, n.s) != rocblas_status_success) what = "rocblas_set_stream failed";
    }
    if (what) {
      if (n.h) rocblas_destroy_handle(n.h);
      for (auto& e : n.ev)
        if (e) (void)hipEventDestroy(e);
      if (n.s) (void)hipStreamDestroy(n.s);
      return fail(MAMBA_ERR_HIP, fn, what);
    }
    g_side[dev] = n;
  }
  *out = &g_side[dev];
  return MAMBA_OK;
}

// work on `to` after what is enqueued on `from` so far
int fork_wait(const char* fn, hipStream_t from, hipStream_t to, hipEvent_t e) {
  if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess)
    return fail(MAMBA_ERR_HIP, fn, "stream fork / join failed");
  return MAMBA_OK;
}

rocblas_datatype blas_type(mscan::Act a) {
  switch (a) {
    case mscan::Act::F32: return rocblas_datatype_f32_r;
    case mscan::Act::BF16: return rocblas_datatype_bf16_r;
    case mscan::Act::F16: return rocblas_datatype_f16_r;
  }
  return rocblas_datatype_f32_r;
}

// Row-major D[M, N] = op(A) op(B) + beta C, op(A) [M, K], op(B) [K, N]; A is
// stored [M, K] (or [K, M] when ta), B [K, N] (or [N, K] when tb), with row
// strides lda / ldb / ldc.  Column-major rocBLAS computes D^T = op(B)^T op(A)^T.
int gemm(const char* fn, const char* what, rocblas_handle h, bool ta, bool tb, int64_t M, int64_t N, int64_t K,
         const void* A, rocblas_datatype at, int64_t lda, const void* B, rocblas_datatype bt, int64_t ldb, float beta,
         const void* C, void* D, rocblas_datatype ct, int64_t ldc) {
  const float alpha = 1.0f;
  const rocblas_status s = rocblas_gemm_ex(
      h, tb ? rocblas_operation_transpose : rocblas_operation_none,
      ta ? rocblas_operation_transpose : rocblas_operation_none, static_cast<rocblas_int>(N),
      static_cast<rocblas_int>(M), static_cast<rocblas_int>(K), &alpha, B, bt, static_cast<rocblas_int>(ldb), A, at,
      static_cast<rocblas_int>(lda), &beta, C, ct, static_cast<rocblas_int>(ldc), D, ct,
      static_cast<rocblas_int>(ldc), rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (s != rocblas_status_success)
    return fail(MAMBA_ERR_HIP, fn, std::string(what) + ": rocblas_gemm_ex: " + rocblas_status_to_string(s));
  return MAMBA_OK;
}

int run(const char* fn, const char* what, const Op& o, mscan::Act act, hipStream_t st) {
  const hipError_t e = mlayer::launch(o, act, st);
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string(what) + " launch: " + hipGetErrorString(e));
  return MAMBA_OK;
}

// grad[M, N] (f32, row-major, contiguous) += A^T B, A [K, M] and B [K, N]
// row-major typed (es bytes per element), on stream s with handle h.  With
// P > 1: P chunks of K / P rows as one strided-batched product into part
// [P, M, N], the K % P rows left as one more product into part[P], then the
// partials added in chunk order onto grad.
int wgrad(const char* fn, const char* what, rocblas_handle h, hipStream_t s, mscan::Act act, int64_t M, int64_t N,
          int64_t K, const void* A, rocblas_datatype at, int64_t lda, const void* B, rocblas_datatype bt, int64_t ldb,
          int64_t es, float* grad, float* part, int64_t P) {
  const rocblas_datatype f32 = rocblas_datatype_f32_r;
  if (P <= 1) return gemm(fn, what, h, true, false, M, N, K, A, at, lda, B, bt, ldb, 1.0f, grad, grad, f32, N);
  const int64_t Kc = K / P, Kt = K - P * Kc;
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st = rocblas_gemm_strided_batched_ex(
      h, rocblas_operation_none, rocblas_operation_transpose, static_cast<rocblas_int>(N), static_cast<rocblas_int>(M),
      static_cast<rocblas_int>(Kc), &alpha, B, bt, static_cast<rocblas_int>(ldb), Kc * ldb, A, at,
      static_cast<rocblas_int>(lda), Kc * lda, &beta, part, f32, static_cast<rocblas_int>(N), M * N, part, f32,
      static_cast<rocblas_int>(N), M * N, static_cast<rocblas_int>(P), f32, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success)
    return fail(MAMBA_ERR_HIP, fn, std::string(what) + ": rocblas_gemm_strided_batched_ex: " +
                                       rocblas_status_to_string(st));
  int64_t nparts = P;
  if (Kt > 0) {
    const char* a_t = static_cast<const char*>(A) + P * Kc * lda * es;
    const char* b_t = static_cast<const char*>(B) + P * Kc * ldb * es;
    float* p_t = part + P * M * N;
    LAYER_TRY(gemm(fn, what, h, true, false, M, N, Kt, a_t, at, lda, b_t, bt, ldb, 0.0f, p_t, p_t, f32, N));
    ++nparts;
  }
  Op o{OpKind::ColSum};
  o.f0 = part;
  o.f3 = grad;
  o.nblk = nparts;
  o.cols = M * N;
  return run(fn, what, o, act, s);
}

// grad (f32, += ) from the matrix-core skinny weight product: P chunk
// partials into a.part, then their column sum in chunk order, on stream s
int skinny_wgrad(const char* fn, const char* what, const mlayer::SkinnyWgradArgs& a, mscan::Act act, bool j_major,
                 hipStream_t s, float* grad, int64_t P, float* grad_b = nullptr) {
  const hipError_t e = mlayer::launch_skinny_wgrad(a, act, j_major, s);
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string(what) + " launch: " + hipGetErrorString(e));
  Op o{OpKind::ColSum};
  o.f0 = a.part;
  o.f3 = grad;
  o.nblk = P;
  o.cols = a.Di * a.J;
  LAYER_TRY(run(fn, what, o, act, s));
  if (!a.part_b) return MAMBA_OK;
  o.f0 = a.part_b;
  o.f3 = grad_b;
  o.cols = a.Di;
  return run(fn, what, o, act, s);
}

int core_call(const char* fn, const char* what, int rc) {
  if (rc == MAMBA_OK) return rc;
  return fail(rc, fn, std::string(what) + ": " + mamba_last_error());
}

}  // namespace

extern "C" {

int mamba_layer_saved_bytes(const mamba_layer_dims_t* dims, size_t* bytes) {
  const char* fn = "mamba_layer_saved_bytes";
  LPlan pl;
  LAYER_TRY(plan_layer(dims, fn, &pl));
  if (!bytes) return fail(MAMBA_ERR_INVALID, fn, "bytes is NULL");
  *bytes = pl.s_total;
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba_layer_workspace_bytes(const mamba_layer_dims_t* dims, size_t* bytes) {
  const char* fn = "mamba_layer_workspace_bytes";
  LPlan pl;
  LAYER_TRY(plan_layer(dims, fn, &pl));
  if (!bytes) return fail(MAMBA_ERR_INVALID, fn, "bytes is NULL");
  *bytes = pl.wf_total > pl.wb_total ? pl.wf_total : pl.wb_total;
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba_layer_fwd(const mamba_layer_dims_t* dims, const mamba_layer_weights_t* w, const float* resid_in,
                    float* resid_out, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "mamba_layer_fwd";
  LPlan pl;
  LAYER_TRY(plan_layer(dims, fn, &pl));
  LAYER_TRY(check_weights(fn, w));
  LAYER_TRY(check_ptr(fn, "resid_in", resid_in, 16));
  LAYER_TRY(check_ptr(fn, "resid_out", resid_out, 16));
  if (resid_out == resid_in) return fail(MAMBA_ERR_INVALID, fn, "resid_out must not alias resid_in");
  LAYER_TRY(check_buffer(fn, "saved", saved, saved_bytes, pl.s_total));
  LAYER_TRY(check_buffer(fn, "workspace", workspace, workspace_bytes, pl.wf_total));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle h = nullptr;
  LAYER_TRY(blas_handle(fn, st, &h));

  char* S = static_cast<char*>(saved);
  char* W = static_cast<char*>(workspace);
  const mscan::Act act = pl.act;
  const rocblas_datatype at = blas_type(act), f32 = rocblas_datatype_f32_r;
  void* xn = S + pl.s_xn;
  float* rstd = reinterpret_cast<float*>(S + pl.s_rstd);
  void* x = S + pl.s_x;
  void* z = S + pl.s_z;
  void* u = S + pl.s_u;
  void* xdbl = S + pl.s_xdbl;
  void* dr = S + pl.s_dr;
  void* gated = S + pl.s_gated;
  void* y = S + pl.s_y;
  float* ckpt = reinterpret_cast<float*>(S + pl.s_ckpt);
  float* dt = reinterpret_cast<float*>(W + pl.w_dt);
  const int64_t N = pl.N, Di = pl.Di, dm = pl.dm, X = pl.X, R = pl.R;

  Op o{OpKind::RmsnormFwd};   // F1
  o.f0 = resid_in;
  o.f1 = w->norm_w;
  o.v0 = xn;
  o.f3 = rstd;
  o.rows = N;
  o.cols = dm;
  o.eps = kNormEps;
  LAYER_TRY(run(fn, "rmsnorm", o, act, st));
  // F2: x = xn W_in[:Di]^T, z = xn W_in[Di:]^T into the halves of rows of 2 d_inner
  const char* w_in_z = static_cast<const char*>(w->w_in) + Di * dm * pl.es;
  LAYER_TRY(gemm(fn, "in_proj x", h, false, true, N, Di, dm, xn, at, dm, w->w_in, at, dm, 0.0f, x, x, at, 2 * Di));
  LAYER_TRY(gemm(fn, "in_proj z", h, false, true, N, Di, dm, xn, at, dm, w_in_z, at, dm, 0.0f, z, z, at, 2 * Di));
  o = Op{OpKind::ConvSiluFwd};   // F4a
  o.c0 = x;
  o.ld = 2 * Di;
  o.f0 = w->conv_w;
  o.f1 = w->conv_b;
  o.v0 = u;
  o.T = pl.T;
  o.cols = Di;
  o.K = static_cast<int>(pl.K);
  o.n = N * Di;
  LAYER_TRY(run(fn, "conv", o, act, st));
  // F4b, F4c: fused on the matrix cores for 16-bit activations, else two
  // library products and the bias pass
  mlayer::XdtArgs xa;
  xa.u = u;
  xa.w_x = w->w_x;
  xa.w_dt = w->w_dt;
  xa.b_dt = w->b_dt;
  xa.xdbl = xdbl;
  xa.dr = dr;
  xa.part = reinterpret_cast<float*>(W + pl.w_xpart);
  xa.N = N;
  xa.Di = Di;
  xa.X = static_cast<int>(X);
  xa.R = static_cast<int>(R);
  if (pl.xdt) {
    const hipError_t e = mlayer::launch_xdt_fwd(xa, act, st);
    if (e != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("x_proj / dt_proj launch: ") + hipGetErrorString(e));
  } else {
    LAYER_TRY(gemm(fn, "x_proj", h, false, true, N, X, Di, u, at, Di, w->w_x, at, Di, 0.0f, xdbl, xdbl, at, X));
    LAYER_TRY(gemm(fn, "dt_proj", h, false, true, N, Di, R, xdbl, at, X, w->w_dt, at, R, 0.0f, dt, dt, f32, Di));
    o = Op{OpKind::BiasRound};
    o.f0 = dt;
    o.f1 = w->b_dt;
    o.v0 = dr;
    o.T = pl.T;
    o.cols = Di;
    o.n = N * Di;
    LAYER_TRY(run(fn, "dt bias", o, act, st));
  }
  // F4d/e
  LAYER_TRY(core_call(fn, "scan", mscan::scan_fwd_ldz(&pl.core, u, dr, w->a_log, xdbl, w->D, z, 2 * Di, nullptr,
                                                      gated, y, nullptr, ckpt, W + pl.w_core_f, pl.core_ws,
                                                      stream)));
  // F5 + F6: resid_out = resid_in + gated W_out^T
  LAYER_TRY(gemm(fn, "out_proj", h, false, true, N, dm, Di, gated, at, Di, w->w_out, at, Di, 1.0f, resid_in, resid_out,
                 f32, dm));
  mscan::set_last_error("");
  return MAMBA_OK;
}

int mamba_layer_bwd(const mamba_layer_dims_t* dims, const mamba_layer_weights_t* w, const float* resid_in,
                    const void* saved, size_t saved_bytes, const float* d_resid_out, float* d_resid_in,
                    const mamba_layer_grads_t* g, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mamba_layer_bwd";
  LPlan pl;
  LAYER_TRY(plan_layer(dims, fn, &pl));
  LAYER_TRY(check_weights(fn, w));
  LAYER_TRY(check_ptr(fn, "resid_in", resid_in, 16));
  LAYER_TRY(check_ptr(fn, "d_resid_out", d_resid_out, 16));
  LAYER_TRY(check_ptr(fn, "d_resid_in", d_resid_in, 16));
  if (d_resid_in == resid_in) return fail(MAMBA_ERR_INVALID, fn, "d_resid_in must not alias resid_in");
  if (!g) return fail(MAMBA_ERR_INVALID, fn, "grads is NULL");
  LAYER_TRY(check_ptr(fn, "grads.norm_w", g->norm_w, 16));
  LAYER_TRY(check_ptr(fn, "grads.w_in", g->w_in, 16));
  LAYER_TRY(check_ptr(fn, "grads.conv_w", g->conv_w, 16));
  LAYER_TRY(check_ptr(fn, "grads.conv_b", g->conv_b, 16));
  LAYER_TRY(check_ptr(fn, "grads.w_x", g->w_x, 16));
  LAYER_TRY(check_ptr(fn, "grads.w_dt", g->w_dt, 16));
  LAYER_TRY(check_ptr(fn, "grads.b_dt", g->b_dt, 16));
  LAYER_TRY(check_ptr(fn, "grads.a_log", g->a_log, 16));
  LAYER_TRY(check_ptr(fn, "grads.D", g->D, 16));
  LAYER_TRY(check_ptr(fn, "grads.w_out", g->w_out, 16));
  LAYER_TRY(check_buffer(fn, "saved", saved, saved_bytes, pl.s_total));
  LAYER_TRY(check_buffer(fn, "workspace", workspace, workspace_bytes, pl.wb_total));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle h = nullptr;
  LAYER_TRY(blas_handle(fn, st, &h));
  Side* sd = nullptr;
  LAYER_TRY(side_res(fn, &sd));
  const rocblas_handle hw = sd->h;
  // Everything below runs in `body`; the join that follows it runs on every
  // path, so a call that fails part-way still leaves no product of this call
  // unordered with the caller's later work.
  auto body = [&]() -> int {
    const char* S = static_cast<const char*>(saved);
    char* W = static_cast<char*>(workspace);
    const mscan::Act act = pl.act;
    const rocblas_datatype at = blas_type(act), f32 = rocblas_datatype_f32_r;
    const void* xn = S + pl.s_xn;
    const float* rstd = reinterpret_cast<const float*>(S + pl.s_rstd);
    const void* x = S + pl.s_x;
    const void* z = S + pl.s_z;
    const void* u = S + pl.s_u;
    const void* xdbl = S + pl.s_xdbl;
    const void* dr = S + pl.s_dr;
    const void* gated = S + pl.s_gated;
    const void* y = S + pl.s_y;
    const float* ckpt = reinterpret_cast<const float*>(S + pl.s_ckpt);
    void* dy = W + pl.w_dy;
    void* d_gated = W + pl.w_dgated;
    void* d_u = W + pl.w_du;
    void* d_dr = W + pl.w_ddr;
    void* d_z = W + pl.w_dz;
    float* d_xdbl = reinterpret_cast<float*>(W + pl.w_dxdbl);
    void* d_xdbl_a = W + pl.w_dxdbl_a;
    float* d_uex = reinterpret_cast<float*>(W + pl.w_duex);
    void* d_x = W + pl.w_dx;
    float* d_xn = reinterpret_cast<float*>(W + pl.w_dxn);
    float* pnorm = reinterpret_cast<float*>(W + pl.w_pnorm);
    float* pbdt = reinterpret_cast<float*>(W + pl.w_pbdt);
    float* pcw = reinterpret_cast<float*>(W + pl.w_pconv_w);
    float* pcb = reinterpret_cast<float*>(W + pl.w_pconv_b);
    float* pwg = reinterpret_cast<float*>(W + pl.w_pwg);
    const int64_t N = pl.N, Di = pl.Di, dm = pl.dm, X = pl.X, R = pl.R;
    mlayer::XdtArgs xa;
    xa.w_x = w->w_x;
    xa.w_dt = w->w_dt;
    xa.d_dr = d_dr;
    xa.d_xdbl = d_xdbl;
    xa.d_xdbl_a = d_xdbl_a;
    xa.d_uex = d_uex;
    xa.w_dtT = W + pl.w_dtT;
    xa.w_xT = W + pl.w_xT;
    xa.part = reinterpret_cast<float*>(W + pl.w_xpart_b);
    xa.N = N;
    xa.Di = Di;
    xa.X = static_cast<int>(X);
    xa.R = static_cast<int>(R);
    const bool fused_xdt = pl.xdt;
    if (fused_xdt) {
      // the transposed weights the x_proj / dt_proj adjoint reads depend on
      // the weights alone: they are made on the second stream while this one
      // runs the out_proj adjoint
      LAYER_TRY(fork_wait(fn, st, sd->s, sd->ev[5]));
      const hipError_t e = mlayer::launch_xdt_bwd_prep(xa, act, sd->s);
      if (e != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("weight transposes launch: ") + hipGetErrorString(e));
      if (hipEventRecord(sd->ev[6], sd->s) != hipSuccess) return fail(MAMBA_ERR_HIP, fn, "stream fork / join failed");
    }

    // out_proj adjoint (the products take typed operands)
    Op o{OpKind::Cast};
    o.f0 = d_resid_out;
    o.v0 = dy;
    o.n = N * dm;
    LAYER_TRY(run(fn, "cast d_resid_out", o, act, st));
    LAYER_TRY(gemm(fn, "out_proj dgrad", h, false, false, N, Di, dm, dy, at, dm, w->w_out, at, Di, 0.0f, d_gated, d_gated,
                   at, Di));
    // the core; it adds into the B/C columns of d_xdbl, which start at zero.
    // No product runs beside it: its kernels are sized to fill every SIMD in
    // one round, and workgroups that a concurrent product keeps off some
    // compute units spill into a second round (a third slower at 130M
    // widths).
    o = Op{OpKind::Zero};
    o.f3 = d_xdbl;
    o.n = N * X;
    LAYER_TRY(run(fn, "zero d_xdbl", o, act, st));
    LAYER_TRY(core_call(fn, "scan backward",
                        mscan::scan_bwd_ldz(&pl.core, u, dr, w->a_log, xdbl, w->D, z, 2 * Di, y, ckpt, d_gated,
                                            d_u, d_dr, d_z, d_xdbl, g->a_log, g->D, W + pl.w_core_b, pl.core_ws,
                                            stream)));
    // the out_proj weight product, and d_z being final, its in_proj one,
    // start beside the rest of the adjoint
    float* gw_in_z = g->w_in + Di * dm;
    LAYER_TRY(fork_wait(fn, st, sd->s, sd->ev[0]));
    LAYER_TRY(wgrad(fn, "out_proj wgrad", hw, sd->s, act, dm, Di, N, dy, at, dm, gated, at, Di, pl.es, g->w_out, pwg,
                    pl.P_wide));
    LAYER_TRY(wgrad(fn, "in_proj wgrad z", hw, sd->s, act, Di, dm, N, d_z, at, 2 * Di, xn, at, dm, pl.es, gw_in_z, pwg,
                    pl.P_wide));
    // dt_proj adjoint: W_dt and b_dt here; the dt columns of d_xdbl with the
    // x_proj adjoint below
    if (!fused_xdt)
      LAYER_TRY(gemm(fn, "dt_proj dgrad", h, false, false, N, R, Di, d_dr, at, Di, w->w_dt, at, R, 0.0f, d_xdbl,
                     d_xdbl, f32, X));
    LAYER_TRY(fork_wait(fn, st, sd->s, sd->ev[1]));
    if (pl.S_dt > 0) {
      mlayer::SkinnyWgradArgs sw;
      sw.big = d_dr;
      sw.small = xdbl;
      sw.part = pwg;
      sw.N = N;
      sw.Di = Di;
      sw.J = R;
      sw.lds = X;
      sw.chunk = pl.S_dt_chunk;
      sw.P = pl.S_dt;
      sw.part_b = reinterpret_cast<float*>(W + pl.w_pskb);   // and the dt bias
      LAYER_TRY(skinny_wgrad(fn, "dt_proj wgrad", sw, act, false, sd->s, g->w_dt, pl.S_dt, g->b_dt));
    } else {
      LAYER_TRY(wgrad(fn, "dt_proj wgrad", hw, sd->s, act, Di, R, N, d_dr, at, Di, xdbl, at, X, pl.es, g->w_dt, pwg,
                      pl.P_dt));
    }
    if (pl.S_dt == 0) {   // the dt bias (the matrix-core dt_proj weight gradient takes it beside itself)
      o = Op{OpKind::ColPart};
      o.c0 = d_dr;
      o.f3 = pbdt;
      o.rows = N;
      o.cols = Di;
      o.per_blk = pl.bdt_per;
      o.nblk = pl.bdt_nblk;
      LAYER_TRY(run(fn, "b_dt partials", o, act, st));
      o = Op{OpKind::ColSum};
      o.f0 = pbdt;
      o.f3 = g->b_dt;
      o.nblk = pl.bdt_nblk;
      o.cols = Di;
      LAYER_TRY(run(fn, "b_dt sum", o, act, st));
    }
    // x_proj adjoint (with the dt columns of d_xdbl when fused)
    if (fused_xdt) {
      if (hipStreamWaitEvent(st, sd->ev[6], 0) != hipSuccess) return fail(MAMBA_ERR_HIP, fn, "stream fork / join failed");
      const hipError_t e = mlayer::launch_xdt_bwd(xa, act, st);
      if (e != hipSuccess)
        return fail(MAMBA_ERR_HIP, fn, std::string("dt_proj / x_proj adjoint launch: ") + hipGetErrorString(e));
    } else {
      o = Op{OpKind::Cast};
      o.f0 = d_xdbl;
      o.v0 = d_xdbl_a;
      o.n = N * X;
      LAYER_TRY(run(fn, "cast d_xdbl", o, act, st));
      LAYER_TRY(gemm(fn, "x_proj dgrad", h, false, false, N, Di, X, d_xdbl_a, at, X, w->w_x, at, Di, 0.0f, d_uex, d_uex,
                     f32, Di));
    }
    LAYER_TRY(fork_wait(fn, st, sd->s, sd->ev[2]));
    if (pl.S_x > 0) {
      mlayer::SkinnyWgradArgs sw;
      sw.big = u;
      sw.small = d_xdbl_a;
      sw.part = pwg;
      sw.N = N;
      sw.Di = Di;
      sw.J = X;
      sw.lds = X;
      sw.chunk = pl.S_x_chunk;
      sw.P = pl.S_x;
      LAYER_TRY(skinny_wgrad(fn, "x_proj wgrad", sw, act, true, sd->s, g->w_x, pl.S_x));
    } else {
      LAYER_TRY(wgrad(fn, "x_proj wgrad", hw, sd->s, act, X, Di, N, d_xdbl_a, at, X, u, at, Di, pl.es, g->w_x, pwg,
                      pl.P_x));
    }
    // conv + SiLU adjoint: d_x and the weight / bias partials in one pass
    o = Op{OpKind::ConvBwd};
    o.c0 = x;
    o.f0 = w->conv_w;
    o.f1 = w->conv_b;
    o.c1 = d_u;
    o.f2 = d_uex;
    o.v0 = d_x;
    o.f3 = pcw;
    o.f6 = pcb;
    o.T = pl.T;
    o.cols = Di;
    o.ld = 2 * Di;   // x and d_x: rows of x | z and of d_x | d_z
    o.K = static_cast<int>(pl.K);
    o.n = N * Di;
    LAYER_TRY(run(fn, "conv adjoint", o, act, st));
    // d_x is final here: its in_proj weight product starts beside the rest
    LAYER_TRY(fork_wait(fn, st, sd->s, sd->ev[3]));
    LAYER_TRY(wgrad(fn, "in_proj wgrad x", hw, sd->s, act, Di, dm, N, d_x, at, 2 * Di, xn, at, dm, pl.es, g->w_in, pwg,
                    pl.P_wide));
    o = Op{OpKind::ColSum};
    o.f0 = pcw;
    o.f3 = g->conv_w;
    o.nblk = pl.conv_nblk;
    o.cols = Di * pl.K;
    LAYER_TRY(run(fn, "conv_w sum", o, act, st));
    o.f0 = pcb;
    o.f3 = g->conv_b;
    o.cols = Di;
    LAYER_TRY(run(fn, "conv_b sum", o, act, st));
    // in_proj adjoint: d_xn = [d_x | d_z] W_in, one product over K = 2 d_inner
    LAYER_TRY(gemm(fn, "in_proj dgrad", h, false, false, N, dm, 2 * Di, d_x, at, 2 * Di, w->w_in, at, dm, 0.0f, d_xn,
                   d_xn, f32, dm));
    // RMSNorm adjoint and the residual
    o = Op{OpKind::RmsnormBwd};
    o.f0 = d_xn;
    o.f1 = resid_in;
    o.f2 = w->norm_w;
    o.f4 = rstd;
    o.f5 = d_resid_out;
    o.f3 = d_resid_in;
    o.rows = N;
    o.cols = dm;
    LAYER_TRY(run(fn, "rmsnorm adjoint", o, act, st));
    o = Op{OpKind::RmsnormWgradPart};
    o.f0 = d_xn;
    o.f1 = resid_in;
    o.f2 = rstd;
    o.f3 = pnorm;
    o.rows = N;
    o.cols = dm;
    o.per_blk = pl.norm_per;
    o.nblk = pl.norm_nblk;
    LAYER_TRY(run(fn, "norm_w partials", o, act, st));
    o = Op{OpKind::ColSum};
    o.f0 = pnorm;
    o.f3 = g->norm_w;
    o.nblk = pl.norm_nblk;
    o.cols = dm;
    LAYER_TRY(run(fn, "norm_w sum", o, act, st));
    return MAMBA_OK;
  };
  const int rc = body();
  const int rj = fork_wait(fn, sd->s, st, sd->ev[4]);   // join: the caller's stream covers every product
  if (rc != MAMBA_OK) return rc;
  if (rj != MAMBA_OK) return rj;
  mscan::set_last_error("");
  return MAMBA_OK;
}

}  // extern "C"
