// C ABI of the selective-scan layer core: argument checks, workspace
// layout and kernel dispatch.  Declared in include/mamba_scan.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "bwd_table.h"
#include "mamba_scan.h"
#include "scan_common.h"
#include "scan_conv.h"
#include "scan_fwd2.h"

namespace mscan {
hipError_t launch_bwd_f32(const BwdArgs& p, int ds, int L, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& p, int ds, int L, hipStream_t st);
hipError_t launch_bwd_f16(const BwdArgs& p, int ds, int L, hipStream_t st);
hipError_t launch_step_f32(const FwdArgs& p, int ds, hipStream_t st);
hipError_t launch_step_bf16(const FwdArgs& p, int ds, hipStream_t st);
hipError_t launch_step_f16(const FwdArgs& p, int ds, hipStream_t st);
hipError_t launch_carry_f32(const CarryArgs& p, int ds, hipStream_t st);
hipError_t launch_carry_bf16(const CarryArgs& p, int ds, hipStream_t st);
hipError_t launch_carry_f16(const CarryArgs& p, int ds, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& p, hipStream_t st);
hipError_t launch_carry_fold(const CarryFoldArgs& p, hipStream_t st);
hipError_t launch_conv_bwd_f32(const ConvBwdArgs& p, hipStream_t st);
hipError_t launch_conv_bwd_bf16(const ConvBwdArgs& p, hipStream_t st);
hipError_t launch_conv_bwd_f16(const ConvBwdArgs& p, hipStream_t st);

static hipError_t launch_conv_bwd(const ConvBwdArgs& p, Act act, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_conv_bwd_f32(p, st);
    case Act::BF16: return launch_conv_bwd_bf16(p, st);
    case Act::F16: return launch_conv_bwd_f16(p, st);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_fwd2_f32(const Fwd2Args& p, int ds, bool regen, hipStream_t st);
hipError_t launch_fwd2_bf16(const Fwd2Args& p, int ds, bool regen, hipStream_t st);
hipError_t launch_fwd2_f16(const Fwd2Args& p, int ds, bool regen, hipStream_t st);
hipError_t launch_bc_f32_f32(const BcArgs& p, hipStream_t st);
hipError_t launch_bc_f32_bf16(const BcArgs& p, hipStream_t st);
hipError_t launch_bc_f32_f16(const BcArgs& p, hipStream_t st);

static hipError_t launch_fwd2(const Fwd2Args& p, Act act, int ds, bool regen, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_fwd2_f32(p, ds, regen, st);
    case Act::BF16: return launch_fwd2_bf16(p, ds, regen, st);
    case Act::F16: return launch_fwd2_f16(p, ds, regen, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_bc(const BcArgs& p, Act act, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_bc_f32_f32(p, st);
    case Act::BF16: return launch_bc_f32_bf16(p, st);
    case Act::F16: return launch_bc_f32_f16(p, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_bwd(const BwdArgs& p, Act act, int ds, int L, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_bwd_f32(p, ds, L, st);
    case Act::BF16: return launch_bwd_bf16(p, ds, L, st);
    case Act::F16: return launch_bwd_f16(p, ds, L, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_step(const FwdArgs& p, Act act, int ds, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_step_f32(p, ds, st);
    case Act::BF16: return launch_step_bf16(p, ds, st);
    case Act::F16: return launch_step_f16(p, ds, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_carry(const CarryArgs& p, Act act, int ds, hipStream_t st) {
  switch (act) {
    case Act::F32: return launch_carry_f32(p, ds, st);
    case Act::BF16: return launch_carry_bf16(p, ds, st);
    case Act::F16: return launch_carry_f16(p, ds, st);
  }
  return hipErrorInvalidValue;
}
}  // namespace mscan

namespace {

thread_local std::string g_err;

int fail(int code, const char* fn, const std::string& msg) {
  g_err = std::string(fn) + ": " + msg;
  return code;
}

}  // namespace

namespace mscan {
// the layer entry points (layer_abi.hip) report through the same message
void set_last_error(const std::string& msg) { g_err = msg; }
}  // namespace mscan

namespace {

struct Plan {
  int64_t B, T, Di, Ds, R, X, nC, nG;
  int K;          // conv taps (0 for the scan entry points)
  int L;          // checkpoint interval of the caller's ckpt
  int Lb;         // interval the backward kernel walks: L, or 16 from regenerated checkpoints
  int64_t nCb;    // ceil(T / Lb)
  mscan::Act act;
  int esize;      // bytes per activation element
  int bulk_align; // alignment of activation inputs staged with 4 / 16-byte granules
  int Sf, Sb;     // segments of the forward / backward schedule
  int Fb;         // sub-segments per backward segment in the carry pass
  int64_t segf_steps;   // steps per forward segment (a multiple of 16)
  int64_t segb_tiles;   // Lb-step tiles per backward segment
  int64_t ldz = 0;      // elements between rows of z and d_z: d_inner, or the stride the layer keeps x | z in
  bool regen() const { return Lb != L; }
  int Sc() const { return Sb * Fb; }   // carry sub-segments
};

constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int kDefaultChunk = 64;   // checkpoint interval when dims.chunk is 0
constexpr int kMaxChunk = 4096;
constexpr int64_t kMaxWidth = int64_t(1) << 24;
constexpr int kMaxSegments = 4096;

// Backward segment count (see kCarryShare below): the caller's `hint`, else
// one segment when `waves` reaches kWantWaves, else the S in 1 .. about twice
// kWantWaves / waves (at least kMinSegmentTiles tiles per segment) with the
// smallest ceil(S * waves / resident) / S + kCarryShare * (S-1) / S; ties go
// to fewer segments.
void choose_segments_bwd(int hint, int64_t waves, int64_t resident, int64_t ntiles, int* S, int64_t* per);

// Backward waves that fill the GPU (1024 SIMDs): the backward's aggregate
// pass costs about a fifth of a backward and always pays for itself until
// about 8 waves per SIMD are queued.
constexpr int64_t kWantWaves = 8192;
constexpr int64_t kMinSegmentTiles = 8;
// Backward segments.  The main pass runs in rounds of `resident` waves (the
// waves per SIMD its kernel is built for, on all 1024 SIMDs), and a segment
// takes 1/S of an unsplit sweep, so S segments cost about
// ceil(S * waves / resident) / S sweeps; the carry pass adds about
// kCarryShare of a sweep times (S-1)/S.  Measured at T=8192, d_inner 5120
// (1280 waves per segment, 3072 resident): S = 3 / 4 / 5 / 7 / 12 gave
// backward 2.12 / 1.85 / 1.99 / 1.77 / 1.71 ms, the order this cost predicts.
constexpr double kCarryShare = 0.1;

void choose_segments_bwd(int hint, int64_t waves, int64_t resident, int64_t ntiles, int* S, int64_t* per) {
  int64_t s = 1;
  if (hint > 0) {
    s = hint;
  } else if (waves < kWantWaves && resident > 0) {
    int64_t hi = 2 * ((kWantWaves + waves - 1) / waves);
    const int64_t cap = ntiles / kMinSegmentTiles;
    hi = hi < cap ? hi : cap;
    hi = hi < kMaxSegments ? hi : kMaxSegments;
    double best = 0.0;
    for (int64_t c = 1; c <= (hi > 1 ? hi : 1); ++c) {
      const double rounds = static_cast<double>((c * waves + resident - 1) / resident);
      const double cost = rounds / static_cast<double>(c) + kCarryShare * static_cast<double>(c - 1) / static_cast<double>(c);
      if (c == 1 || cost < best - 1e-12) {
        best = cost;
        s = c;
      }
    }
  }
  s = s < ntiles ? s : ntiles;
  s = s < 1 ? 1 : s;
  *per = (ntiles + s - 1) / s;
  *S = static_cast<int>((ntiles + *per - 1) / *per);
}

// Sub-segments per backward segment in the carry pass.  Its grid is one
// workgroup per 32 channels of a batch row (`groups`) and sub-segment after
// the first segment; with whole segments it can leave the CUs short of
// waves (576 workgroups at batch 4, d_inner 1536, 4 segments: 0.40 ns per
// element against 0.23 with a full grid).  Halve the sub-segments until
// about 8 workgroups per CU are queued, keeping at least kCarryMinTiles
// 16-step tiles each.
constexpr int64_t kCarryWantWgs = 2048;
constexpr int64_t kCarryMinTiles = 4;

int carry_split(int64_t groups, int S, int64_t seg_steps) {
  if (S < 2) return 1;
  const int64_t tiles = seg_steps / 16;
  int64_t f = 1;
  while (groups * (S - 1) * f < kCarryWantWgs && tiles % (2 * f) == 0 && tiles / (2 * f) >= kCarryMinTiles) f *= 2;
  return static_cast<int>(f);
}

// Forward segments (one single-wave workgroup per 64 channels of a batch
// row and segment).  Each segment past the first costs an aggregate pass
// over it, so the forward splits only as far as it takes to fill the GPU in
// ONE round of resident waves: about `k` waves on each of the 1024 SIMDs,
// k being what the kernel's registers and LDS ring allow per SIMD.  More
// segments than that leave a second, mostly idle round; fewer leave SIMDs
// with fewer waves than others (measured at T=8192, d_inner 5120, 160 waves
// per segment: 12 / 19 / 25 / 32 segments gave 0.83 / 0.68 / 0.90 / 0.89 ms).
// The caller's `hint` overrides; segments are whole multiples of 16 steps
// and, when chosen here, at least kFwdMinSteps long.
constexpr int64_t kFwdMinSteps = 64;

int64_t fwd_waves_per_simd(int64_t ds, int esize) {
  const int64_t vgpr_waves = ds <= 16 ? 4 : (ds == 32 ? 3 : 2);   // the kernel's register target
  const int64_t lds = 3 * (mscan::kFwd2Tile * 2 * ds * 4 + 3 * mscan::kFwd2Tile * 64 * esize);
  const int64_t lds_waves = (mscan::kLdsBytes / lds) / 4;            // per SIMD, 4 SIMDs per CU
  const int64_t k = vgpr_waves < lds_waves ? vgpr_waves : lds_waves;
  return k < 1 ? 1 : k;
}

void choose_segments_fwd(int hint, int64_t waves, int64_t k, int64_t T, int* S, int64_t* steps) {
  const int64_t t16 = (T + 15) / 16;   // 16-step units
  int64_t s = 1;
  if (hint > 0) {
    s = hint;
  } else if (waves < k * 1024) {
    s = k * 1024 / waves;
    const int64_t cap = T / kFwdMinSteps;
    s = s < cap ? s : cap;
  }
  s = s < t16 ? s : t16;
  s = s < 1 ? 1 : s;
  *steps = (t16 + s - 1) / s * 16;
  *S = static_cast<int>((T + *steps - 1) / *steps);
}

// threads per workgroup of the backward kernel (its launch table)
int64_t bwd_threads(int64_t ds, int L) {
  return mscan::kBwdCpw * (ds / mscan::bwd_states_per_thread(static_cast<int>(ds), L));
}

int plan_dims(const mamba_dims_t* d, bool fused, const char* fn, Plan* pl) {
  if (!d) return fail(MAMBA_ERR_INVALID, fn, "dims is NULL");
  if (d->segments < 0 || d->segments > kMaxSegments)
    return fail(MAMBA_ERR_INVALID, fn, "dims.segments must be in [0, " + std::to_string(kMaxSegments) + "]");
  if (d->act < 0 || d->act > 2) return fail(MAMBA_ERR_INVALID, fn, "dims.act is not a mamba_dtype_t");
  if (d->batch < 1 || d->batch > 65535)
    return fail(d->batch < 1 ? MAMBA_ERR_INVALID : MAMBA_ERR_CAPACITY, fn, "batch must be in [1, 65535]");
  if (d->seqlen < 1) return fail(MAMBA_ERR_INVALID, fn, "seqlen must be >= 1");
  if (d->d_inner < 4 || d->d_inner % 4 != 0)
    return fail(MAMBA_ERR_INVALID, fn, "d_inner must be a positive multiple of 4");
  if (d->d_inner > kMaxWidth)   // per-tile offsets (step * d_inner) are 32-bit in the kernels
    return fail(MAMBA_ERR_CAPACITY, fn, "d_inner must be <= 2^24");
  if (d->dt_rank < 0) return fail(MAMBA_ERR_INVALID, fn, "dt_rank must be >= 0");
  if (d->dt_rank > kMaxWidth) return fail(MAMBA_ERR_CAPACITY, fn, "dt_rank must be <= 2^24");
  if (d->d_state < 1) return fail(MAMBA_ERR_INVALID, fn, "d_state must be >= 1");
  if (d->d_state != 4 && d->d_state != 8 && d->d_state != 16 && d->d_state != 32 && d->d_state != 64)
    return fail(MAMBA_ERR_UNSUPPORTED, fn, "d_state must be 4, 8, 16, 32 or 64");
  if (d->chunk < 0) return fail(MAMBA_ERR_INVALID, fn, "chunk must be >= 0");
  if (d->chunk % 16 != 0 || d->chunk > kMaxChunk)
    return fail(MAMBA_ERR_UNSUPPORTED, fn,
                "chunk must be 0 (default " + std::to_string(kDefaultChunk) + ") or a multiple of 16 up to " +
                    std::to_string(kMaxChunk));
  const int L = d->chunk ? d->chunk : kDefaultChunk;
  int K = 0;
  if (fused) {
    if (d->d_conv < 1) return fail(MAMBA_ERR_INVALID, fn, "d_conv must be >= 1");
    if (d->d_conv > 4) return fail(MAMBA_ERR_UNSUPPORTED, fn, "d_conv must be <= 4");
    K = d->d_conv;
  }
  const int64_t X = d->dt_rank + 2 * d->d_state;
  if (d->seqlen > kMaxElems / d->batch || d->batch * d->seqlen > kMaxElems / (d->d_inner > X ? d->d_inner : X))
    return fail(MAMBA_ERR_CAPACITY, fn, "B * T * max(d_inner, xdbl row) exceeds 2^46 elements");
  pl->B = d->batch;
  pl->T = d->seqlen;
  pl->Di = d->d_inner;
  pl->Ds = d->d_state;
  pl->ldz = d->d_inner;
  pl->R = d->dt_rank;
  pl->X = X;
  pl->L = L;
  pl->nC = (d->seqlen + L - 1) / L;
  // the backward kernel keeps a tile of Lb steps of state in registers; it is
  // built for 16 and, for some d_state, 32 steps.  Other intervals are walked
  // in 16-step tiles from checkpoints regenerated out of the caller's.
  pl->Lb = (L == 16 || mscan::bwd_waves_per_simd(static_cast<int>(d->d_state), L, fused) > 0) ? L : 16;
  pl->nCb = (d->seqlen + pl->Lb - 1) / pl->Lb;
  pl->nG = (d->d_inner + mscan::kBwdCpw - 1) / mscan::kBwdCpw;
  pl->K = K;
  pl->act = static_cast<mscan::Act>(d->act);
  pl->esize = d->act == MAMBA_F32 ? 4 : 2;
  pl->bulk_align = d->act == MAMBA_F32 ? 16 : 4;
  const int64_t waves_f = (d->d_inner + 63) / 64 * d->batch;   // one wave per 64 channels and segment
  const int64_t waves_b = pl->nG * d->batch * (bwd_threads(d->d_state, pl->Lb) / 64);
  choose_segments_fwd(d->segments, waves_f, fwd_waves_per_simd(d->d_state, pl->esize), d->seqlen, &pl->Sf,
                      &pl->segf_steps);
  {
    const int64_t resident =
        1024 * static_cast<int64_t>(mscan::bwd_waves_per_simd(static_cast<int>(d->d_state), pl->Lb, fused));
    choose_segments_bwd(d->segments, waves_b, resident, pl->nCb, &pl->Sb, &pl->segb_tiles);
    pl->Fb = carry_split(pl->nG * d->batch, pl->Sb, pl->segb_tiles * pl->Lb);
  }
  // a launch holds at most 2^32 - 1 threads: the forward and backward (all
  // segments in one grid), the checkpoint regeneration and the reduction
  // (one thread per d_xdbl B/C element plus one per parameter-grad slot)
  // are the largest
  const int64_t thr_f = waves_f * 64 * (pl->Sf > pl->nC ? pl->Sf : pl->nC);
  const int64_t thr_b = pl->nG * d->batch * bwd_threads(d->d_state, pl->Lb) * pl->Sb;
  const int64_t thr_r = d->batch * d->seqlen * 2 * d->d_state + d->d_inner * (d->d_state + 2 + K);
  const int64_t thr = thr_f > thr_b ? (thr_f > thr_r ? thr_f : thr_r) : (thr_b > thr_r ? thr_b : thr_r);
  if (thr > static_cast<int64_t>(UINT32_MAX))
    return fail(MAMBA_ERR_CAPACITY, fn, "a launch would need " + std::to_string(thr) +
                                            " threads (> 2^32 - 1): reduce batch * seqlen or d_inner");
  return MAMBA_OK;
}

bool misaligned(const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Checks one pointer argument; `need` false allows NULL.
int check_ptr(const char* fn, const char* name, const void* p, bool need, int align) {
  if (!p) return need ? fail(MAMBA_ERR_INVALID, fn, std::string(name) + " is NULL") : MAMBA_OK;
  if (misaligned(p, align))
    return fail(MAMBA_ERR_INVALID, fn, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return MAMBA_OK;
}

#define MSCAN_TRY(expr)               \
  do {                                \
    int rc_ = (expr);                 \
    if (rc_ != MAMBA_OK) return rc_;  \
  } while (0)

int64_t param_width(const Plan& pl) { return pl.Ds + 1; }

size_t bc_part_bytes(const Plan& pl) {
  return static_cast<size_t>(pl.nG) * pl.B * pl.T * 2 * pl.Ds * sizeof(float);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace layouts.  Forward: [bc | seg_h | seg_sd], the last two when
// segmented (nothing for the short-sequence step kernel).  Backward:
// [part_bc | part_par | seg_q | seg_sd | seg_c | bc | sub | du | part_conv],
// seg_q, seg_sd (per carry sub-segment) and seg_c (per segment) when
// segmented, bc and sub when the checkpoints are regenerated, du and
// part_conv for the fused entry.
size_t seg_state_bytes(const Plan& pl, int S) { return align256(sizeof(float) * pl.B * S * pl.Di * pl.Ds); }
size_t seg_sum_bytes(const Plan& pl, int S) { return align256(sizeof(float) * pl.B * S * pl.Di); }
size_t par_part_bytes(const Plan& pl) { return align256(sizeof(float) * pl.Sb * pl.B * pl.Di * param_width(pl)); }
// fused entry: d_u (f32) from the scan backward, and the conv adjoint's
// weight / bias partials per (batch row, conv tile)
size_t du_bytes(const Plan& pl) { return pl.K > 0 ? align256(sizeof(float) * pl.B * pl.T * pl.Di) : 0; }
size_t conv_part_bytes(const Plan& pl) {
  return pl.K > 0 ? align256(sizeof(float) * pl.B * mscan::conv_bwd_tiles(pl.T) * pl.Di * (pl.K + 1)) : 0;
}
size_t bc_f32_bytes(const Plan& pl) { return align256(sizeof(float) * pl.B * pl.T * 2 * pl.Ds); }
size_t sub_ckpt_bytes(const Plan& pl) { return align256(sizeof(float) * pl.B * ((pl.T + 15) / 16) * pl.Ds * pl.Di); }

size_t workspace_need_fwd(const Plan& pl) {
  if (pl.T <= mscan::kStepMaxT) return 0;
  return bc_f32_bytes(pl) + (pl.Sf > 1 ? seg_state_bytes(pl, pl.Sf) + seg_sum_bytes(pl, pl.Sf) : 0);
}

size_t workspace_need_bwd(const Plan& pl) {
  return align256(bc_part_bytes(pl)) + par_part_bytes(pl) +
         (pl.Sb > 1 ? seg_state_bytes(pl, pl.Sc()) + seg_sum_bytes(pl, pl.Sc()) + seg_state_bytes(pl, pl.Sb) : 0) +
         (pl.regen() ? bc_f32_bytes(pl) + sub_ckpt_bytes(pl) : 0) + du_bytes(pl) + conv_part_bytes(pl);
}

size_t workspace_need(const Plan& pl) {
  const size_t f = workspace_need_fwd(pl), b = workspace_need_bwd(pl);
  return f > b ? f : b;
}

int check_workspace(const char* fn, const void* workspace, size_t workspace_bytes, size_t need) {
  if (need == 0) return MAMBA_OK;
  MSCAN_TRY(check_ptr(fn, "workspace", workspace, true, 256));
  if (workspace_bytes < need)
    return fail(MAMBA_ERR_CAPACITY, fn,
                "workspace_bytes " + std::to_string(workspace_bytes) + " < required " + std::to_string(need));
  return MAMBA_OK;
}

// ------------------------------------------------ backward without a workspace
// Device scratch of mamba_scan_bwd_static: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.
constexpr size_t kStaticScratchBytes = size_t(MAMBA_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int static_scratch(const char* fn, void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MAMBA_ERR_HIP, fn, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MAMBA_ERR_HIP, fn, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MAMBA_OK;
}

int do_forward(const char* fn, const Plan& pl, const void* x, const float* conv_w, const float* conv_b,
               const float* conv_state0, const void* delta_raw, const float* a_log, const void* xdbl,
               const float* D, const void* z, const float* h0, void* out, void* u_out, void* y_save,
               float* h_last, float* conv_state_last, float* ckpt, void* workspace, size_t workspace_bytes,
               void* stream) {
  const int e = pl.esize, ba = pl.bulk_align;
  MSCAN_TRY(check_ptr(fn, pl.K ? "x" : "u", x, true, ba));
  MSCAN_TRY(check_ptr(fn, "delta_raw", delta_raw, true, ba));
  MSCAN_TRY(check_ptr(fn, "a_log", a_log, true, 4));
  MSCAN_TRY(check_ptr(fn, "xdbl", xdbl, true, e));
  MSCAN_TRY(check_ptr(fn, "D", D, false, 4));
  MSCAN_TRY(check_ptr(fn, "z", z, false, ba));
  MSCAN_TRY(check_ptr(fn, "h0", h0, false, 4));
  MSCAN_TRY(check_ptr(fn, "out", out, true, e));
  MSCAN_TRY(check_ptr(fn, "y_save", y_save, false, e));
  MSCAN_TRY(check_ptr(fn, "h_last", h_last, false, 4));
  MSCAN_TRY(check_ptr(fn, "ckpt", ckpt, false, 4));
  if (pl.K > 0) {
    MSCAN_TRY(check_ptr(fn, "conv_w", conv_w, true, 4));
    MSCAN_TRY(check_ptr(fn, "conv_b", conv_b, false, 4));
    MSCAN_TRY(check_ptr(fn, "conv_state0", conv_state0, false, 4));
    MSCAN_TRY(check_ptr(fn, "u_out", u_out, false, e));
    MSCAN_TRY(check_ptr(fn, "conv_state_last", conv_state_last, false, 4));
  }
  MSCAN_TRY(check_workspace(fn, workspace, workspace_bytes, workspace_need_fwd(pl)));
  mscan::FwdArgs a{};
  a.x = x;
  a.delta_raw = delta_raw;
  a.a_log = a_log;
  a.xdbl = xdbl;
  a.D = D;
  a.z = z;
  a.h0 = h0;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.conv_state0 = conv_state0;
  a.out = out;
  a.u_out = u_out;
  a.y_save = y_save;
  a.h_last = h_last;
  a.conv_state_last = conv_state_last;
  a.ckpt = ckpt;
  a.B = pl.B;
  a.T = pl.T;
  a.Di = pl.Di;
  a.R = pl.R;
  a.X = pl.X;
  a.nC = pl.nC;
  a.ldz = pl.ldz;
  a.K = pl.K;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (pl.T <= mscan::kStepMaxT) {
    // short sequences (recurrent steps): one thread per channel, no staging
    err = mscan::launch_step(a, pl.act, static_cast<int>(pl.Ds), st);
  } else {
    char* ws = static_cast<char*>(workspace);
    mscan::BcArgs c{};
    c.xdbl = xdbl;
    c.bc = reinterpret_cast<float*>(ws);
    c.rows = pl.B * pl.T;
    c.X = pl.X;
    c.R = pl.R;
    c.Ds = pl.Ds;
    err = mscan::launch_bc(c, pl.act, st);
    if (err == hipSuccess) {
      mscan::Fwd2Args f{};
      f.x = x;
      f.delta_raw = delta_raw;
      f.a_log = a_log;
      f.bc = c.bc;
      f.D = D;
      f.z = z;
      f.h0 = h0;
      f.conv_w = conv_w;
      f.conv_b = conv_b;
      f.conv_state0 = conv_state0;
      f.out = out;
      f.u_out = u_out;
      f.y_save = y_save;
      f.h_last = h_last;
      f.conv_state_last = conv_state_last;
      f.ckpt = ckpt;
      f.B = pl.B;
      f.T = pl.T;
      f.Di = pl.Di;
      f.nC = pl.nC;
      f.ldz = pl.ldz;
      f.seg_steps = pl.segf_steps;
      f.K = pl.K;
      f.L = pl.L;
      f.S = pl.Sf;
      if (pl.Sf > 1) {
        f.seg_h = reinterpret_cast<float*>(ws + bc_f32_bytes(pl));
        f.seg_sd = reinterpret_cast<float*>(ws + bc_f32_bytes(pl) + seg_state_bytes(pl, pl.Sf));
      }
      err = mscan::launch_fwd2(f, pl.act, static_cast<int>(pl.Ds), false, st);
    }
  }
  if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("forward launch: ") + hipGetErrorString(err));
  g_err.clear();
  return MAMBA_OK;
}

int do_backward(const char* fn, const Plan& pl, const void* x, const float* conv_w, const float* conv_b,
                const float* conv_state0, const void* delta_raw, const float* a_log, const void* xdbl,
                const float* D, const void* z, const void* y_saved, const float* ckpt, const void* dout,
                const void* d_u_extra, void* d_x, void* d_delta_raw, void* d_z, float* d_xdbl,
                float* d_a_log, float* d_D, float* d_conv_w, float* d_conv_b, void* workspace,
                size_t workspace_bytes, void* stream, bool use_static = false) {
  const int e = pl.esize, ba = pl.bulk_align;
  MSCAN_TRY(check_ptr(fn, pl.K ? "x" : "u", x, true, ba));
  MSCAN_TRY(check_ptr(fn, "delta_raw", delta_raw, true, ba));
  MSCAN_TRY(check_ptr(fn, "a_log", a_log, true, 4));
  MSCAN_TRY(check_ptr(fn, "xdbl", xdbl, true, e));
  MSCAN_TRY(check_ptr(fn, "D", D, false, 4));
  MSCAN_TRY(check_ptr(fn, "z", z, false, ba));
  MSCAN_TRY(check_ptr(fn, "y_saved", y_saved, z != nullptr, ba));
  MSCAN_TRY(check_ptr(fn, "ckpt", ckpt, true, 4));
  MSCAN_TRY(check_ptr(fn, "dout", dout, true, ba));
  MSCAN_TRY(check_ptr(fn, pl.K ? "d_x" : "d_u", d_x, true, e));
  MSCAN_TRY(check_ptr(fn, "d_delta_raw", d_delta_raw, true, e));
  MSCAN_TRY(check_ptr(fn, "d_z", d_z, z != nullptr, e));
  MSCAN_TRY(check_ptr(fn, "d_xdbl", d_xdbl, true, 4));
  MSCAN_TRY(check_ptr(fn, "d_a_log", d_a_log, true, 4));
  MSCAN_TRY(check_ptr(fn, "d_D", d_D, true, 4));
  if (pl.K > 0) {
    MSCAN_TRY(check_ptr(fn, "conv_w", conv_w, true, 4));
    MSCAN_TRY(check_ptr(fn, "conv_b", conv_b, false, 4));
    MSCAN_TRY(check_ptr(fn, "conv_state0", conv_state0, false, 4));
    MSCAN_TRY(check_ptr(fn, "d_u_extra", d_u_extra, false, e));
    MSCAN_TRY(check_ptr(fn, "d_conv_w", d_conv_w, true, 4));
    MSCAN_TRY(check_ptr(fn, "d_conv_b", d_conv_b, true, 4));
  }
  if (use_static) {   // after every argument check: the device is touched only for a valid call
    const size_t need = workspace_need_bwd(pl);
    if (need > kStaticScratchBytes)
      return fail(MAMBA_ERR_CAPACITY, fn,
                  "these dims need " + std::to_string(need) + " bytes of scratch, more than the " +
                      std::to_string(kStaticScratchBytes) +
                      " of the static array: call mamba_scan_bwd with a workspace");
    MSCAN_TRY(static_scratch(fn, &workspace));
    workspace_bytes = kStaticScratchBytes;
  }
  MSCAN_TRY(check_ptr(fn, "workspace", workspace, true, 256));
  MSCAN_TRY(check_workspace(fn, workspace, workspace_bytes, workspace_need_bwd(pl)));
  char* ws = static_cast<char*>(workspace);
  float* part_bc = reinterpret_cast<float*>(ws);
  float* part_par = reinterpret_cast<float*>(ws + align256(bc_part_bytes(pl)));
  char* after_par = ws + align256(bc_part_bytes(pl)) + par_part_bytes(pl);
  float* seg_q = reinterpret_cast<float*>(after_par);
  float* seg_sd = reinterpret_cast<float*>(after_par + seg_state_bytes(pl, pl.Sc()));
  float* seg_c = reinterpret_cast<float*>(after_par + seg_state_bytes(pl, pl.Sc()) + seg_sum_bytes(pl, pl.Sc()));
  char* after_seg = after_par + (pl.Sb > 1 ? seg_state_bytes(pl, pl.Sc()) + seg_sum_bytes(pl, pl.Sc()) +
                                                 seg_state_bytes(pl, pl.Sb)
                                           : 0);
  const int PW = static_cast<int>(param_width(pl));
  hipStream_t st = static_cast<hipStream_t>(stream);

  char* after_regen = after_seg + (pl.regen() ? bc_f32_bytes(pl) + sub_ckpt_bytes(pl) : 0);
  float* du_buf = reinterpret_cast<float*>(after_regen);                     // fused: d_u, f32
  float* part_conv = reinterpret_cast<float*>(after_regen + du_bytes(pl));  // fused: conv partials
  const float* ckpt_b = ckpt;   // checkpoints the backward kernel walks, every Lb steps
  if (pl.regen()) {
    // states entering every 16th step, regenerated from the caller's
    // checkpoints (every L steps) by the forward recurrence
    mscan::BcArgs c{};
    c.xdbl = xdbl;
    c.bc = reinterpret_cast<float*>(after_seg);
    c.rows = pl.B * pl.T;
    c.X = pl.X;
    c.R = pl.R;
    c.Ds = pl.Ds;
    hipError_t err = mscan::launch_bc(c, pl.act, st);
    if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("B/C copy launch: ") + hipGetErrorString(err));
    mscan::Fwd2Args f{};
    f.x = x;
    f.delta_raw = delta_raw;
    f.a_log = a_log;
    f.bc = c.bc;
    f.conv_w = conv_w;
    f.conv_b = conv_b;
    f.conv_state0 = conv_state0;
    f.ckpt = const_cast<float*>(ckpt);   // read only in this mode
    f.sub = reinterpret_cast<float*>(after_seg + bc_f32_bytes(pl));
    f.B = pl.B;
    f.T = pl.T;
    f.Di = pl.Di;
    f.nC = pl.nC;
    f.ldz = pl.ldz;
    f.seg_steps = pl.L;
    f.K = pl.K;
    f.L = pl.L;
    f.S = static_cast<int>(pl.nC);
    err = mscan::launch_fwd2(f, pl.act, static_cast<int>(pl.Ds), true, st);
    if (err != hipSuccess)
      return fail(MAMBA_ERR_HIP, fn, std::string("checkpoint regeneration launch: ") + hipGetErrorString(err));
    ckpt_b = f.sub;
  }

  if (pl.Sb > 1) {   // aggregate pass: carries the segments hand back from a zero start
    mscan::CarryArgs c{};
    c.delta_raw = delta_raw;
    c.a_log = a_log;
    c.xdbl = xdbl;
    c.z = z;
    c.dout = dout;
    c.seg_q = seg_q;
    c.seg_sd = seg_sd;
    c.B = pl.B;
    c.T = pl.T;
    c.Di = pl.Di;
    c.R = pl.R;
    c.X = pl.X;
    c.ldz = pl.ldz;
    c.seg_steps = pl.segb_tiles * pl.Lb / pl.Fb;
    c.S = pl.Sc();
    c.first = pl.Fb;
    hipError_t err = mscan::launch_carry(c, pl.act, static_cast<int>(pl.Ds), st);
    if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("carry launch: ") + hipGetErrorString(err));
    mscan::CarryFoldArgs fo{};
    fo.a_log = a_log;
    fo.seg_q = seg_q;
    fo.seg_sd = seg_sd;
    fo.seg_c = seg_c;
    fo.B = pl.B;
    fo.Di = pl.Di;
    fo.Ds = pl.Ds;
    fo.S = pl.Sb;
    fo.F = pl.Fb;
    err = mscan::launch_carry_fold(fo, st);
    if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("carry fold launch: ") + hipGetErrorString(err));
  }

  mscan::BwdArgs a{};
  a.x = x;
  a.delta_raw = delta_raw;
  a.a_log = a_log;
  a.xdbl = xdbl;
  a.D = D;
  a.z = z;
  a.y_saved = y_saved;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.conv_state0 = conv_state0;
  a.ckpt = ckpt_b;
  a.dout = dout;
  a.d_x = d_x;
  a.du_out = du_buf;
  a.d_delta_raw = d_delta_raw;
  a.d_z = d_z;
  a.part_bc = part_bc;
  a.part_par = part_par;
  a.B = pl.B;
  a.T = pl.T;
  a.Di = pl.Di;
  a.R = pl.R;
  a.X = pl.X;
  a.nC = pl.nCb;
  a.ldz = pl.ldz;
  a.K = pl.K;
  a.L = pl.Lb;
  a.PW = PW;
  a.S = pl.Sb;
  a.seg_tiles = pl.segb_tiles;
  if (pl.Sb > 1) a.seg_c = seg_c;
  hipError_t err = mscan::launch_bwd(a, pl.act, static_cast<int>(pl.Ds), pl.Lb, st);
  if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("backward launch: ") + hipGetErrorString(err));
  if (pl.K > 0) {   // the conv + SiLU adjoint over the d_u just written
    mscan::ConvBwdArgs cv{};
    cv.x = x;
    cv.conv_w = conv_w;
    cv.conv_b = conv_b;
    cv.conv_state0 = conv_state0;
    cv.du = du_buf;
    cv.d_u_extra = d_u_extra;
    cv.d_x = d_x;
    cv.part = part_conv;
    cv.B = pl.B;
    cv.T = pl.T;
    cv.Di = pl.Di;
    cv.K = pl.K;
    err = mscan::launch_conv_bwd(cv, pl.act, st);
    if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("conv backward launch: ") + hipGetErrorString(err));
  }

  mscan::ReduceArgs r{};
  r.part_bc = part_bc;
  r.part_par = part_par;
  r.d_xdbl = d_xdbl;
  r.d_a_log = d_a_log;
  r.d_D = d_D;
  r.d_conv_w = d_conv_w;
  r.d_conv_b = d_conv_b;
  r.B = pl.B;
  r.T = pl.T;
  r.Di = pl.Di;
  r.Ds = pl.Ds;
  r.R = pl.R;
  r.X = pl.X;
  r.nG = pl.nG;
  r.par_rows = static_cast<int64_t>(pl.Sb) * pl.B;
  r.part_conv = part_conv;
  r.conv_rows = pl.B * mscan::conv_bwd_tiles(pl.T);
  r.K = pl.K;
  r.PW = PW;
  err = mscan::launch_reduce(r, st);
  if (err != hipSuccess) return fail(MAMBA_ERR_HIP, fn, std::string("reduce launch: ") + hipGetErrorString(err));
  g_err.clear();
  return MAMBA_OK;
}

}  // namespace

extern "C" {

int mamba_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

const char* mamba_last_error(void) { return g_err.c_str(); }

int mamba_ckpt_bytes(const mamba_dims_t* dims, size_t* bytes) {
  const char* fn = "mamba_ckpt_bytes";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  if (!bytes) return fail(MAMBA_ERR_INVALID, fn, "bytes is NULL");
  *bytes = static_cast<size_t>(pl.B) * pl.nC * pl.Ds * pl.Di * sizeof(float);
  g_err.clear();
  return MAMBA_OK;
}

int mamba_workspace_bytes(const mamba_dims_t* dims, size_t* bytes) {
  const char* fn = "mamba_workspace_bytes";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  if (!bytes) return fail(MAMBA_ERR_INVALID, fn, "bytes is NULL");
  size_t need = workspace_need(pl);
  if (dims->d_conv > 0) {   // the fused entry points plan with the conv taps
    Plan pf;
    MSCAN_TRY(plan_dims(dims, true, fn, &pf));
    const size_t nf = workspace_need(pf);
    need = nf > need ? nf : need;
  }
  *bytes = need;
  g_err.clear();
  return MAMBA_OK;
}

int mamba_scan_fwd(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                   const void* xdbl, const float* D, const void* z, const float* h0, void* out,
                   void* y_save, float* h_last, float* ckpt, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const char* fn = "mamba_scan_fwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  return do_forward(fn, pl, u, nullptr, nullptr, nullptr, delta_raw, a_log, xdbl, D, z, h0, out, nullptr,
                    y_save, h_last, nullptr, ckpt, workspace, workspace_bytes, stream);
}

int mamba_scan_bwd(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                   const void* xdbl, const float* D, const void* z, const void* y_saved, const float* ckpt,
                   const void* dout, void* d_u, void* d_delta_raw, void* d_z, float* d_xdbl, float* d_a_log,
                   float* d_D, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mamba_scan_bwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  return do_backward(fn, pl, u, nullptr, nullptr, nullptr, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout,
                     nullptr, d_u, d_delta_raw, d_z, d_xdbl, d_a_log, d_D, nullptr, nullptr, workspace,
                     workspace_bytes, stream);
}

int mamba_scan_bwd_static(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                          const void* xdbl, const float* D, const void* z, const void* y_saved, const float* ckpt,
                          const void* dout, void* d_u, void* d_delta_raw, void* d_z, float* d_xdbl,
                          float* d_a_log, float* d_D, void* stream) {
  const char* fn = "mamba_scan_bwd_static";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  // every scratch byte the kernels read is written earlier in the same call
  // (per-group partials, per-segment pairs), so nothing needs clearing
  return do_backward(fn, pl, u, nullptr, nullptr, nullptr, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout,
                     nullptr, d_u, d_delta_raw, d_z, d_xdbl, d_a_log, d_D, nullptr, nullptr, nullptr, 0, stream,
                     true);
}

int mamba_conv_scan_gate_fwd(const mamba_dims_t* dims, const void* x, const float* conv_w, const float* conv_b,
                             const float* conv_state0, const void* delta_raw, const float* a_log,
                             const void* xdbl, const float* D, const void* z, const float* h0, void* out,
                             void* u_out, void* y_save, float* h_last, float* conv_state_last, float* ckpt,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mamba_conv_scan_gate_fwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, true, fn, &pl));
  return do_forward(fn, pl, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D, z, h0, out, u_out,
                    y_save, h_last, conv_state_last, ckpt, workspace, workspace_bytes, stream);
}

int mamba_conv_scan_gate_bwd(const mamba_dims_t* dims, const void* x, const float* conv_w, const float* conv_b,
                             const float* conv_state0, const void* delta_raw, const float* a_log,
                             const void* xdbl, const float* D, const void* z, const void* y_saved,
                             const float* ckpt, const void* dout, const void* d_u_extra, void* d_x,
                             void* d_delta_raw, void* d_z, float* d_xdbl, float* d_a_log, float* d_D,
                             float* d_conv_w, float* d_conv_b, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const char* fn = "mamba_conv_scan_gate_bwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, true, fn, &pl));
  return do_backward(fn, pl, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout,
                     d_u_extra, d_x, d_delta_raw, d_z, d_xdbl, d_a_log, d_D, d_conv_w, d_conv_b, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

namespace mscan {

// mamba_scan_fwd / mamba_scan_bwd with the rows of z (and d_z) ldz elements
// apart, for the layer, which keeps x | z and d_x | d_z interleaved.
int scan_fwd_ldz(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                 const void* xdbl, const float* D, const void* z, int64_t ldz, const float* h0, void* out,
                 void* y_save, float* h_last, float* ckpt, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mamba_scan_fwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  if (ldz < pl.Di || ldz % 4 != 0) return fail(MAMBA_ERR_INVALID, fn, "z rows: stride below d_inner or not a multiple of 4");
  pl.ldz = ldz;
  return do_forward(fn, pl, u, nullptr, nullptr, nullptr, delta_raw, a_log, xdbl, D, z, h0, out, nullptr,
                    y_save, h_last, nullptr, ckpt, workspace, workspace_bytes, stream);
}

int scan_bwd_ldz(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                 const void* xdbl, const float* D, const void* z, int64_t ldz, const void* y_saved,
                 const float* ckpt, const void* dout, void* d_u, void* d_delta_raw, void* d_z, float* d_xdbl,
                 float* d_a_log, float* d_D, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mamba_scan_bwd";
  Plan pl;
  MSCAN_TRY(plan_dims(dims, false, fn, &pl));
  if (ldz < pl.Di || ldz % 4 != 0) return fail(MAMBA_ERR_INVALID, fn, "z rows: stride below d_inner or not a multiple of 4");
  pl.ldz = ldz;
  return do_backward(fn, pl, u, nullptr, nullptr, nullptr, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout,
                     nullptr, d_u, d_delta_raw, d_z, d_xdbl, d_a_log, d_D, nullptr, nullptr, workspace,
                     workspace_bytes, stream);
}

}  // namespace mscan
