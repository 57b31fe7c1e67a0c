"""MI355X (gfx950) selective-scan layer core for Mamba-1 training.

The compute lives in libmamba_scan.so (HIP kernels behind the C ABI in
include/mamba_scan.h, and a whole Mamba-1 layer around it in
include/mamba_layer.h).  This package is its thin binding: ``_lib`` marshals
torch device tensors into the C entry points; ``layer`` (the scan core) and
``mamba_layer`` (the whole layer) keep the buffers of one layer so a
forward/backward pair can be issued repeatedly; ``mamba3`` does the same for
the Mamba-3 SISO core (include/mamba3.h).
"""
from ._lib import (EXPORTED, LAYER_PARAMS, LAYER_TYPED, LIB_PATH, MAMBA_BF16, MAMBA_F16, MAMBA_F32, Dims,
                   LayerDims, M3Dims, MambaScanError, abi_version, ckpt_bytes, ckpt_shape, conv_scan_gate_bwd,
                   conv_scan_gate_fwd, last_error, layer_bwd, layer_fwd, layer_param_shapes, layer_saved_bytes,
                   layer_workspace_bytes, load, m3_bwd, m3_fwd, m3_states_bytes, m3_workspace_bytes, scan_bwd,
                   scan_bwd_static, scan_fwd, workspace_bytes)
from .layer import LayerCore
from .mamba_layer import MambaLayer
from .mamba3 import Mamba3Core

__all__ = ["Dims", "MambaScanError", "LayerCore", "abi_version", "last_error", "ckpt_bytes", "ckpt_shape",
           "workspace_bytes", "scan_fwd", "scan_bwd", "scan_bwd_static", "conv_scan_gate_fwd", "conv_scan_gate_bwd", "load",
           "LIB_PATH", "EXPORTED", "MAMBA_F32", "MAMBA_BF16", "MAMBA_F16", "LayerDims", "MambaLayer",
           "LAYER_PARAMS", "LAYER_TYPED", "layer_param_shapes", "layer_saved_bytes", "layer_workspace_bytes",
           "layer_fwd", "layer_bwd", "M3Dims", "m3_states_bytes", "m3_workspace_bytes", "m3_fwd", "m3_bwd",
           "Mamba3Core"]
