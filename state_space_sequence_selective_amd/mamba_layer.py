"""One whole Mamba-1 layer (RMSNorm, projections, conv, scan core,
residual) around the C entry points of include/mamba_layer.h.

``MambaLayer`` owns the layer's saved activations, workspace and f32
gradient buffers, allocated once, so that ``forward`` and ``backward``
issue only launches.  The weights are the caller's tensors: the typed
projection weights in the activation dtype, the rest f32.
"""
from __future__ import annotations

import torch

from . import _lib


class MambaLayer:
    def __init__(self, dims: _lib.LayerDims, weights: dict, device="cuda"):
        self.dims = d = dims
        self.weights = weights
        c = d.core
        kw = dict(device=device)
        rs = (c.batch, c.seqlen, d.d_model)
        self.resid_out = torch.empty(rs, dtype=torch.float32, **kw)
        self.d_resid_in = torch.empty(rs, dtype=torch.float32, **kw)
        self.saved = torch.empty(_lib.layer_saved_bytes(d), dtype=torch.uint8, **kw)
        self.workspace = torch.empty(_lib.layer_workspace_bytes(d), dtype=torch.uint8, **kw)
        # the gradients share one arena (views on 256-byte boundaries), so
        # clearing them once per step is a single fill
        shapes = _lib.layer_param_shapes(d)
        sizes = {n: -(-torch.Size(s).numel() // 64) * 64 for n, s in shapes.items()}
        self._grad_arena = torch.zeros(sum(sizes.values()), dtype=torch.float32, **kw)
        self.grads, off = {}, 0
        for n, s in shapes.items():
            self.grads[n] = self._grad_arena[off:off + torch.Size(s).numel()].view(s)
            off += sizes[n]

    def zero_grads(self):
        """Weight gradients accumulate; clear them once per step."""
        self._grad_arena.zero_()

    def forward(self, resid_in, stream=None):
        _lib.layer_fwd(self.dims, self.weights, resid_in, resid_out=self.resid_out, saved=self.saved,
                       workspace=self.workspace, stream=stream)
        return self.resid_out

    def backward(self, resid_in, d_resid_out, stream=None):
        _lib.layer_bwd(self.dims, self.weights, resid_in, self.saved, d_resid_out, d_resid_in=self.d_resid_in,
                       grads=self.grads, workspace=self.workspace, stream=stream)
        return self.d_resid_in
