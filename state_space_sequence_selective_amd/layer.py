"""One layer's device buffers around the C entry points.

``LayerCore`` owns the saved activations (y, checkpoints), the outputs and
the workspace of one layer, allocated once, so that ``forward`` and
``backward`` issue only kernel launches (no allocation on the hot path).
"""
from __future__ import annotations

import torch

from . import _lib


class LayerCore:
    def __init__(self, dims: _lib.Dims, device="cuda", gate=True, keep_u=False):
        self.dims = d = dims
        self.fused = d.d_conv > 0
        self.gate = gate
        at, f = d.act_dtype, torch.float32
        act = (d.batch, d.seqlen, d.d_inner)
        kw = dict(device=device)
        self.out = torch.empty(act, dtype=at, **kw)
        self.y = torch.empty(act, dtype=at, **kw) if gate else None
        self.u_out = torch.empty(act, dtype=at, **kw) if (self.fused and keep_u) else None
        self.h_last = torch.empty((d.batch, d.d_inner, d.d_state), dtype=f, **kw)
        self.ckpt = torch.empty(_lib.ckpt_shape(d), dtype=f, **kw)
        self.conv_state_last = torch.empty((d.batch, d.d_inner, d.d_conv), dtype=f, **kw) if self.fused else None
        self.d_x = torch.empty(act, dtype=at, **kw)
        self.d_delta_raw = torch.empty(act, dtype=at, **kw)
        self.d_z = torch.empty(act, dtype=at, **kw) if gate else None
        # the accumulated gradients share one arena (256-byte aligned views), so
        # clearing them once per step is a single fill
        shapes = [("d_xdbl", (d.batch, d.seqlen, d.xdbl_dim)), ("d_a_log", (d.d_inner, d.d_state)),
                  ("d_D", (d.d_inner,))]
        if self.fused:
            shapes += [("d_conv_w", (d.d_inner, d.d_conv)), ("d_conv_b", (d.d_inner,))]
        sizes = [-(-torch.Size(s).numel() // 64) * 64 for _, s in shapes]   # floats, rounded up to 256 bytes
        self._grad_arena = torch.zeros(sum(sizes), dtype=f, **kw)
        off = 0
        for (name, shape), n in zip(shapes, sizes):
            setattr(self, name, self._grad_arena[off:off + torch.Size(shape).numel()].view(shape))
            off += n
        if not self.fused:
            self.d_conv_w = self.d_conv_b = None
        self.workspace = torch.empty(_lib.workspace_bytes(d), dtype=torch.uint8, **kw)

    def zero_grads(self):
        """Parameter grads and d_xdbl accumulate; clear them once per step."""
        self._grad_arena.zero_()

    def forward(self, inp: dict, stream=None):
        d = self.dims
        z = inp.get("z") if self.gate else None
        if self.fused:
            _lib.conv_scan_gate_fwd(d, inp["x"], inp["conv_w"], inp.get("conv_b"), inp.get("conv_state0"),
                                    inp["delta_raw"], inp["a_log"], inp["xdbl"], inp.get("D"), z, inp.get("h0"),
                                    out=self.out, u_out=self.u_out, y_save=self.y, h_last=self.h_last,
                                    conv_state_last=self.conv_state_last, ckpt=self.ckpt,
                                    workspace=self.workspace, stream=stream)
        else:
            _lib.scan_fwd(d, inp["x"], inp["delta_raw"], inp["a_log"], inp["xdbl"], inp.get("D"), z,
                          inp.get("h0"), out=self.out, y_save=self.y, h_last=self.h_last, ckpt=self.ckpt,
                          workspace=self.workspace, stream=stream)
        return self.out

    def backward(self, inp: dict, dout, stream=None):
        d = self.dims
        z = inp.get("z") if self.gate else None
        if self.fused:
            _lib.conv_scan_gate_bwd(d, inp["x"], inp["conv_w"], inp.get("conv_b"), inp.get("conv_state0"),
                                    inp["delta_raw"], inp["a_log"], inp["xdbl"], inp.get("D"), z, self.y,
                                    self.ckpt, dout, inp.get("d_u_extra"), d_x=self.d_x,
                                    d_delta_raw=self.d_delta_raw, d_z=self.d_z, d_xdbl=self.d_xdbl,
                                    d_a_log=self.d_a_log, d_D=self.d_D, d_conv_w=self.d_conv_w,
                                    d_conv_b=self.d_conv_b, workspace=self.workspace, stream=stream)
        else:
            _lib.scan_bwd(d, inp["x"], inp["delta_raw"], inp["a_log"], inp["xdbl"], inp.get("D"), z, self.y,
                          self.ckpt, dout, d_u=self.d_x, d_delta_raw=self.d_delta_raw, d_z=self.d_z,
                          d_xdbl=self.d_xdbl, d_a_log=self.d_a_log, d_D=self.d_D, workspace=self.workspace,
                          stream=stream)
