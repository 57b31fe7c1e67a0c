// Entry points of the scan for the whole-layer code in this library: the
// calls of include/mamba_scan.h (mamba_scan_fwd, mamba_scan_bwd) with the
// rows of z and d_z `ldz` elements apart (ldz >= d_inner, a multiple of 4),
// so that the layer can keep its in_proj output x | z, and the gradient
// d_x | d_z, interleaved in rows of 2 d_inner: one product each way instead
// of two.  Arguments, errors and every other layout are those of the public
// calls.
#pragma once
#include <cstddef>
#include <cstdint>

#include "mamba_scan.h"

namespace mscan {

int scan_fwd_ldz(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                 const void* xdbl, const float* D, const void* z, int64_t ldz, const float* h0, void* out,
                 void* y_save, float* h_last, float* ckpt, void* workspace, size_t workspace_bytes, void* stream);

int scan_bwd_ldz(const mamba_dims_t* dims, const void* u, const void* delta_raw, const float* a_log,
                 const void* xdbl, const float* D, const void* z, int64_t ldz, const void* y_saved,
                 const float* ckpt, const void* dout, void* d_u, void* d_delta_raw, void* d_z, float* d_xdbl,
                 float* d_a_log, float* d_D, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace mscan
