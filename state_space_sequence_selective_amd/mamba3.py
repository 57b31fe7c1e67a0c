"""One Mamba-3 SISO core's device buffers around the C entry points of
include/mamba3.h.

``Mamba3Core`` owns the output, the chunk states the backward reads, every
gradient and the workspace, allocated once, so that ``forward`` and
``backward`` issue only kernel launches.
"""
from __future__ import annotations

import torch

from . import _lib

GRADS = ("x", "b_in", "c_in", "dd_dt_raw", "dd_a_raw", "trap_raw", "angles_raw", "b_bias", "c_bias", "dt_bias", "D")
PARAMS = ("b_bias", "c_bias", "dt_bias", "D")   # their gradients accumulate


class Mamba3Core:
    def __init__(self, dims: _lib.M3Dims, device="cuda"):
        self.dims = d = dims
        s, at, f = d.shapes(), d.act_dtype, torch.float32
        kw = dict(device=device)
        self.y = torch.empty(s["x"], dtype=at, **kw)
        self.states = torch.empty(s["states"], dtype=f, **kw)
        shp = dict(x=(s["x"], at), b_in=(s["bc"], at), c_in=(s["bc"], at), dd_dt_raw=(s["bth"], f),
                   dd_a_raw=(s["bth"], f), trap_raw=(s["bth"], f), angles_raw=(s["ang"], f), b_bias=(s["hn"], f),
                   c_bias=(s["hn"], f), dt_bias=(s["h"], f), D=(s["h"], f))
        self.grads = {k: torch.empty(shp[k][0], dtype=shp[k][1], **kw) for k in GRADS if k not in PARAMS}
        # the accumulating parameter gradients are views of one f32 block (each
        # at a 256-byte boundary), so clearing them is one fill
        sizes = [int(torch.Size(shp[k][0]).numel()) for k in PARAMS]
        padded = [(n + 63) // 64 * 64 for n in sizes]
        self._param_grads = torch.empty(sum(padded), dtype=f, **kw)
        off = 0
        for k, n, pn in zip(PARAMS, sizes, padded):
            self.grads[k] = self._param_grads[off:off + n].view(shp[k][0])
            off += pn
        self.workspace = torch.empty(_lib.m3_workspace_bytes(d), dtype=torch.uint8, **kw)

    def zero_grads(self):
        """The parameter gradients accumulate; clear them once per step."""
        self._param_grads.zero_()

    def _inputs(self, inp):
        return (inp["x"], inp["b_in"], inp["c_in"], inp["dd_dt_raw"], inp["dd_a_raw"], inp["trap_raw"],
                inp.get("angles_raw"), inp["b_bias"], inp["c_bias"], inp["dt_bias"], inp.get("D"))

    def forward(self, inp: dict, stream=None):
        _lib.m3_fwd(self.dims, *self._inputs(inp), y=self.y, states=self.states, workspace=self.workspace,
                    stream=stream)
        return self.y

    def backward(self, inp: dict, dy, stream=None):
        g = self.grads
        _lib.m3_bwd(self.dims, *self._inputs(inp), self.states, dy, d_x=g["x"], d_b_in=g["b_in"], d_c_in=g["c_in"],
                    d_dd_dt_raw=g["dd_dt_raw"], d_dd_a_raw=g["dd_a_raw"], d_trap_raw=g["trap_raw"],
                    d_angles_raw=g["angles_raw"] if self.dims.n_angles else None, d_b_bias=g["b_bias"],
                    d_c_bias=g["c_bias"], d_dt_bias=g["dt_bias"], d_D=g["D"] if inp.get("D") is not None else None,
                    workspace=self.workspace, stream=stream)
        return g
