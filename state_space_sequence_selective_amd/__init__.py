"""MI355X (gfx950) selective-scan layer core for Mamba-1 training.

The compute lives in libmamba_scan.so (HIP kernels behind the C ABI in
include/mamba_scan.h).  This package is its thin binding: ``_lib`` marshals
torch device tensors into the C entry points and ``layer`` keeps the
buffers of one layer so a forward/backward pair can be issued repeatedly.
"""
from ._lib import (EXPORTED, LIB_PATH, MAMBA_BF16, MAMBA_F16, MAMBA_F32, Dims, MambaScanError, abi_version,
                   ckpt_bytes, ckpt_shape, conv_scan_gate_bwd, conv_scan_gate_fwd, last_error, load, scan_bwd,
                   scan_fwd, workspace_bytes)
from .layer import LayerCore

__all__ = ["Dims", "MambaScanError", "LayerCore", "abi_version", "last_error", "ckpt_bytes", "ckpt_shape",
           "workspace_bytes", "scan_fwd", "scan_bwd", "conv_scan_gate_fwd", "conv_scan_gate_bwd", "load",
           "LIB_PATH", "EXPORTED", "MAMBA_F32", "MAMBA_BF16", "MAMBA_F16"]
