"""ctypes binding of libmamba_scan.so (include/mamba_scan.h, include/mamba_layer.h,
include/mamba3.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
size, their device pointers are handed to the C entry points, and a non-zero
status becomes MambaScanError.  There is no fallback: without the built HIP
library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmamba_scan.so")

MAMBA_F32, MAMBA_BF16, MAMBA_F16 = 0, 1, 2
STATUS = {0: "MAMBA_OK", 1: "MAMBA_ERR_INVALID", 2: "MAMBA_ERR_UNSUPPORTED",
          3: "MAMBA_ERR_CAPACITY", 4: "MAMBA_ERR_HIP"}
ACT_CODES = {"f32": MAMBA_F32, "bf16": MAMBA_BF16, "f16": MAMBA_F16}
TORCH_DTYPES = {MAMBA_F32: torch.float32, MAMBA_BF16: torch.bfloat16, MAMBA_F16: torch.float16}

EXPORTED = ("mamba_abi_version", "mamba_last_error", "mamba_ckpt_bytes", "mamba_workspace_bytes",
            "mamba_scan_fwd", "mamba_scan_bwd", "mamba_scan_bwd_static", "mamba_conv_scan_gate_fwd",
            "mamba_conv_scan_gate_bwd",
            "mamba_layer_saved_bytes", "mamba_layer_workspace_bytes", "mamba_layer_fwd", "mamba_layer_bwd",
            "mamba3_states_bytes", "mamba3_workspace_bytes", "mamba3_siso_fwd", "mamba3_siso_bwd")

# weights of one layer (mamba_layer_weights_t / mamba_layer_grads_t field order)
LAYER_PARAMS = ("norm_w", "w_in", "conv_w", "conv_b", "w_x", "w_dt", "b_dt", "a_log", "D", "w_out")
# those held in the activation dtype (the others, and every gradient, are f32)
LAYER_TYPED = ("w_in", "w_x", "w_dt", "w_out")


class MambaScanError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, message))
        self.status = status


class Dims(ctypes.Structure):
    """mamba_dims_t."""
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("dt_rank", ctypes.c_int64), ("d_conv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("act", ctypes.c_int32), ("segments", ctypes.c_int32)]

    @classmethod
    def make(cls, batch, seqlen, d_inner, d_state, dt_rank=0, d_conv=0, chunk=0, act="bf16", segments=0):
        code = ACT_CODES[act] if isinstance(act, str) else int(act)
        return cls(batch, seqlen, d_inner, d_state, dt_rank, d_conv, chunk, code, segments)

    @property
    def L(self) -> int:
        """Checkpoint interval: dims.chunk, or the library's default of 64."""
        return self.chunk if self.chunk else 64

    @property
    def xdbl_dim(self) -> int:
        return self.dt_rank + 2 * self.d_state

    @property
    def act_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.act]

    def __repr__(self):
        return "Dims(%s)" % ", ".join("%s=%d" % (f, getattr(self, f)) for f, _ in self._fields_)


_lib = None


def load():
    """Load the built library; raises if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmamba_scan.so is not built (expected at %s); run __graft_entry__.build() "
                          "or state_space_sequence_selective_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, D = ctypes.c_void_p, ctypes.POINTER(Dims)
    lib.mamba_abi_version.restype = ctypes.c_int
    lib.mamba_abi_version.argtypes = []
    lib.mamba_last_error.restype = ctypes.c_char_p
    lib.mamba_last_error.argtypes = []
    for name in ("mamba_ckpt_bytes", "mamba_workspace_bytes"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.mamba_scan_fwd.restype = ctypes.c_int
    lib.mamba_scan_fwd.argtypes = [D] + [P] * 12 + [ctypes.c_size_t, P]
    lib.mamba_scan_bwd.restype = ctypes.c_int
    lib.mamba_scan_bwd.argtypes = [D] + [P] * 16 + [ctypes.c_size_t, P]
    lib.mamba_scan_bwd_static.restype = ctypes.c_int
    lib.mamba_scan_bwd_static.argtypes = [D] + [P] * 16
    lib.mamba_conv_scan_gate_fwd.restype = ctypes.c_int
    lib.mamba_conv_scan_gate_fwd.argtypes = [D] + [P] * 17 + [ctypes.c_size_t, P]
    lib.mamba_conv_scan_gate_bwd.restype = ctypes.c_int
    lib.mamba_conv_scan_gate_bwd.argtypes = [D] + [P] * 22 + [ctypes.c_size_t, P]
    LD = ctypes.POINTER(LayerDims)
    for name in ("mamba_layer_saved_bytes", "mamba_layer_workspace_bytes"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [LD, ctypes.POINTER(ctypes.c_size_t)]
    lib.mamba_layer_fwd.restype = ctypes.c_int
    lib.mamba_layer_fwd.argtypes = [LD, ctypes.POINTER(LayerWeights), P, P, P, ctypes.c_size_t, P,
                                    ctypes.c_size_t, P]
    lib.mamba_layer_bwd.restype = ctypes.c_int
    lib.mamba_layer_bwd.argtypes = [LD, ctypes.POINTER(LayerWeights), P, P, ctypes.c_size_t, P, P,
                                    ctypes.POINTER(LayerGrads), P, ctypes.c_size_t, P]
    M3 = ctypes.POINTER(M3Dims)
    for name in ("mamba3_states_bytes", "mamba3_workspace_bytes"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [M3, ctypes.POINTER(ctypes.c_size_t)]
    lib.mamba3_siso_fwd.restype = ctypes.c_int
    lib.mamba3_siso_fwd.argtypes = [M3] + [P] * 14 + [ctypes.c_size_t, P]
    lib.mamba3_siso_bwd.restype = ctypes.c_int
    lib.mamba3_siso_bwd.argtypes = [M3] + [P] * 25 + [ctypes.c_size_t, P]
    _lib = lib
    return lib


def last_error() -> str:
    return load().mamba_last_error().decode()


def abi_version() -> int:
    return load().mamba_abi_version()


def _check(status: int):
    if status != 0:
        raise MambaScanError(status, last_error())


def ckpt_bytes(dims: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba_ckpt_bytes(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def workspace_bytes(dims: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba_workspace_bytes(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def ckpt_shape(dims: Dims):
    return (dims.batch, -(-dims.seqlen // dims.L), dims.d_state, dims.d_inner)


# ---------------------------------------------------------------- marshalling


def _ptr(t, name, dtype, shape, required=False):
    """Device address of ``t`` after checking it (None passes as NULL unless required).

    The common case is one conjunction of cheap attribute tests; the specific
    error is worked out only when it fails (a recurrent step calls this for
    every tensor on every call)."""
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return None
    if isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.shape == shape and t.is_contiguous():
        return t.data_ptr()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    raise ValueError("%s must be contiguous" % name)


def _workspace(workspace):
    if workspace is None:
        return None, 0
    n = workspace.numel()
    return _ptr(workspace, "workspace", torch.uint8, (n,), True), n


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


_SHAPES = {}


def _shapes(d: Dims):
    """Expected tensor shapes for ``d`` (cached per distinct dims)."""
    key = bytes(d)
    s = _SHAPES.get(key)
    if s is None:
        act = (d.batch, d.seqlen, d.d_inner)
        s = dict(act=act, xdbl=(d.batch, d.seqlen, d.xdbl_dim), a_log=(d.d_inner, d.d_state),
                 vec=(d.d_inner,), state=(d.batch, d.d_inner, d.d_state), ckpt=ckpt_shape(d),
                 conv_w=(d.d_inner, d.d_conv), conv_state=(d.batch, d.d_inner, d.d_conv))
        if len(_SHAPES) > 256:
            _SHAPES.clear()
        _SHAPES[key] = s
    return s


def scan_fwd(d: Dims, u, delta_raw, a_log, xdbl, D=None, z=None, h0=None, *, out, y_save=None,
             h_last=None, ckpt=None, workspace=None, stream=None):
    s, at, f = _shapes(d), d.act_dtype, torch.float32
    args = [ctypes.byref(d), _ptr(u, "u", at, s["act"], True), _ptr(delta_raw, "delta_raw", at, s["act"], True),
            _ptr(a_log, "a_log", f, s["a_log"], True), _ptr(xdbl, "xdbl", at, s["xdbl"], True),
            _ptr(D, "D", f, s["vec"]), _ptr(z, "z", at, s["act"]), _ptr(h0, "h0", f, s["state"]),
            _ptr(out, "out", at, s["act"], True), _ptr(y_save, "y_save", at, s["act"]),
            _ptr(h_last, "h_last", f, s["state"]), _ptr(ckpt, "ckpt", f, s["ckpt"]), *_workspace(workspace),
            _stream(stream)]
    _check(load().mamba_scan_fwd(*args))


def scan_bwd(d: Dims, u, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout, *, d_u, d_delta_raw, d_z,
             d_xdbl, d_a_log, d_D, workspace, stream=None):
    s, at, f = _shapes(d), d.act_dtype, torch.float32
    ws, wsn = _workspace(workspace)
    args = [ctypes.byref(d), _ptr(u, "u", at, s["act"], True), _ptr(delta_raw, "delta_raw", at, s["act"], True),
            _ptr(a_log, "a_log", f, s["a_log"], True), _ptr(xdbl, "xdbl", at, s["xdbl"], True),
            _ptr(D, "D", f, s["vec"]), _ptr(z, "z", at, s["act"]), _ptr(y_saved, "y_saved", at, s["act"]),
            _ptr(ckpt, "ckpt", f, s["ckpt"], True), _ptr(dout, "dout", at, s["act"], True),
            _ptr(d_u, "d_u", at, s["act"], True), _ptr(d_delta_raw, "d_delta_raw", at, s["act"], True),
            _ptr(d_z, "d_z", at, s["act"]), _ptr(d_xdbl, "d_xdbl", f, s["xdbl"], True),
            _ptr(d_a_log, "d_a_log", f, s["a_log"], True), _ptr(d_D, "d_D", f, s["vec"], True),
            ws, wsn, _stream(stream)]
    _check(load().mamba_scan_bwd(*args))


def scan_bwd_static(d: Dims, u, delta_raw, a_log, xdbl, D, z, y_saved, ckpt, dout, *, d_u, d_delta_raw, d_z,
                    d_xdbl, d_a_log, d_D, stream=None):
    """mamba_scan_bwd_static: scan_bwd with the library's static device
    scratch instead of a workspace (nothing is allocated)."""
    s, at, f = _shapes(d), d.act_dtype, torch.float32
    args = [ctypes.byref(d), _ptr(u, "u", at, s["act"], True), _ptr(delta_raw, "delta_raw", at, s["act"], True),
            _ptr(a_log, "a_log", f, s["a_log"], True), _ptr(xdbl, "xdbl", at, s["xdbl"], True),
            _ptr(D, "D", f, s["vec"]), _ptr(z, "z", at, s["act"]), _ptr(y_saved, "y_saved", at, s["act"]),
            _ptr(ckpt, "ckpt", f, s["ckpt"], True), _ptr(dout, "dout", at, s["act"], True),
            _ptr(d_u, "d_u", at, s["act"], True), _ptr(d_delta_raw, "d_delta_raw", at, s["act"], True),
            _ptr(d_z, "d_z", at, s["act"]), _ptr(d_xdbl, "d_xdbl", f, s["xdbl"], True),
            _ptr(d_a_log, "d_a_log", f, s["a_log"], True), _ptr(d_D, "d_D", f, s["vec"], True),
            _stream(stream)]
    _check(load().mamba_scan_bwd_static(*args))


def conv_scan_gate_fwd(d: Dims, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D=None, z=None,
                       h0=None, *, out, u_out=None, y_save=None, h_last=None, conv_state_last=None, ckpt=None,
                       workspace=None, stream=None):
    s, at, f = _shapes(d), d.act_dtype, torch.float32
    args = [ctypes.byref(d), _ptr(x, "x", at, s["act"], True), _ptr(conv_w, "conv_w", f, s["conv_w"], True),
            _ptr(conv_b, "conv_b", f, s["vec"]), _ptr(conv_state0, "conv_state0", f, s["conv_state"]),
            _ptr(delta_raw, "delta_raw", at, s["act"], True), _ptr(a_log, "a_log", f, s["a_log"], True),
            _ptr(xdbl, "xdbl", at, s["xdbl"], True), _ptr(D, "D", f, s["vec"]), _ptr(z, "z", at, s["act"]),
            _ptr(h0, "h0", f, s["state"]), _ptr(out, "out", at, s["act"], True),
            _ptr(u_out, "u_out", at, s["act"]), _ptr(y_save, "y_save", at, s["act"]),
            _ptr(h_last, "h_last", f, s["state"]), _ptr(conv_state_last, "conv_state_last", f, s["conv_state"]),
            _ptr(ckpt, "ckpt", f, s["ckpt"]), *_workspace(workspace), _stream(stream)]
    _check(load().mamba_conv_scan_gate_fwd(*args))


def conv_scan_gate_bwd(d: Dims, x, conv_w, conv_b, conv_state0, delta_raw, a_log, xdbl, D, z, y_saved, ckpt,
                       dout, d_u_extra=None, *, d_x, d_delta_raw, d_z, d_xdbl, d_a_log, d_D, d_conv_w, d_conv_b,
                       workspace, stream=None):
    s, at, f = _shapes(d), d.act_dtype, torch.float32
    ws, wsn = _workspace(workspace)
    args = [ctypes.byref(d), _ptr(x, "x", at, s["act"], True), _ptr(conv_w, "conv_w", f, s["conv_w"], True),
            _ptr(conv_b, "conv_b", f, s["vec"]), _ptr(conv_state0, "conv_state0", f, s["conv_state"]),
            _ptr(delta_raw, "delta_raw", at, s["act"], True), _ptr(a_log, "a_log", f, s["a_log"], True),
            _ptr(xdbl, "xdbl", at, s["xdbl"], True), _ptr(D, "D", f, s["vec"]), _ptr(z, "z", at, s["act"]),
            _ptr(y_saved, "y_saved", at, s["act"]), _ptr(ckpt, "ckpt", f, s["ckpt"], True),
            _ptr(dout, "dout", at, s["act"], True), _ptr(d_u_extra, "d_u_extra", at, s["act"]),
            _ptr(d_x, "d_x", at, s["act"], True), _ptr(d_delta_raw, "d_delta_raw", at, s["act"], True),
            _ptr(d_z, "d_z", at, s["act"]), _ptr(d_xdbl, "d_xdbl", f, s["xdbl"], True),
            _ptr(d_a_log, "d_a_log", f, s["a_log"], True), _ptr(d_D, "d_D", f, s["vec"], True),
            _ptr(d_conv_w, "d_conv_w", f, s["conv_w"], True), _ptr(d_conv_b, "d_conv_b", f, s["vec"], True),
            ws, wsn, _stream(stream)]
    _check(load().mamba_conv_scan_gate_bwd(*args))


# ------------------------------------------------------------- whole layer


class LayerDims(ctypes.Structure):
    """mamba_layer_dims_t."""
    _fields_ = [("core", Dims), ("d_model", ctypes.c_int64)]

    @classmethod
    def make(cls, batch, seqlen, d_model, d_inner, d_state, dt_rank, d_conv, chunk=0, act="bf16", segments=0):
        return cls(Dims.make(batch, seqlen, d_inner, d_state, dt_rank, d_conv, chunk, act, segments), d_model)


class LayerWeights(ctypes.Structure):
    """mamba_layer_weights_t (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_PARAMS]


class LayerGrads(ctypes.Structure):
    """mamba_layer_grads_t (device pointers, f32, accumulated)."""
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_PARAMS]


def layer_param_shapes(ld: LayerDims) -> dict:
    c = ld.core
    Di, Ds, R, K, dm = c.d_inner, c.d_state, c.dt_rank, c.d_conv, ld.d_model
    return dict(norm_w=(dm,), w_in=(2 * Di, dm), conv_w=(Di, K), conv_b=(Di,), w_x=(R + 2 * Ds, Di),
                w_dt=(Di, R), b_dt=(Di,), a_log=(Di, Ds), D=(Di,), w_out=(dm, Di))


def layer_saved_bytes(ld: LayerDims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba_layer_saved_bytes(ctypes.byref(ld), ctypes.byref(out)))
    return out.value


def layer_workspace_bytes(ld: LayerDims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba_layer_workspace_bytes(ctypes.byref(ld), ctypes.byref(out)))
    return out.value


def _layer_struct(cls, ld, tensors: dict, grads: bool):
    shapes = layer_param_shapes(ld)
    at = ld.core.act_dtype
    vals = []
    for n in LAYER_PARAMS:
        dt = at if (n in LAYER_TYPED and not grads) else torch.float32
        vals.append(_ptr(tensors.get(n), ("grads." if grads else "w.") + n, dt, shapes[n], True))
    return cls(*vals)


def _buffer(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    return _ptr(t, name, torch.uint8, (t.numel(),), True), t.numel()


def layer_fwd(ld: LayerDims, weights: dict, resid_in, *, resid_out, saved, workspace, stream=None):
    c = ld.core
    rs = (c.batch, c.seqlen, ld.d_model)
    w = _layer_struct(LayerWeights, ld, weights, False)
    sp, sn = _buffer(saved, "saved")
    wp, wn = _buffer(workspace, "workspace")
    _check(load().mamba_layer_fwd(ctypes.byref(ld), ctypes.byref(w), _ptr(resid_in, "resid_in", torch.float32, rs, True),
                                  _ptr(resid_out, "resid_out", torch.float32, rs, True), sp, sn, wp, wn,
                                  _stream(stream)))


def layer_bwd(ld: LayerDims, weights: dict, resid_in, saved, d_resid_out, *, d_resid_in, grads: dict, workspace,
              stream=None):
    c = ld.core
    rs = (c.batch, c.seqlen, ld.d_model)
    w = _layer_struct(LayerWeights, ld, weights, False)
    g = _layer_struct(LayerGrads, ld, grads, True)
    sp, sn = _buffer(saved, "saved")
    wp, wn = _buffer(workspace, "workspace")
    _check(load().mamba_layer_bwd(ctypes.byref(ld), ctypes.byref(w), _ptr(resid_in, "resid_in", torch.float32, rs, True),
                                  sp, sn, _ptr(d_resid_out, "d_resid_out", torch.float32, rs, True),
                                  _ptr(d_resid_in, "d_resid_in", torch.float32, rs, True), ctypes.byref(g), wp, wn,
                                  _stream(stream)))


# ------------------------------------------------------ Mamba-3 SISO core


class M3Dims(ctypes.Structure):
    """mamba3_dims_t."""
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("d_state", ctypes.c_int64), ("groups", ctypes.c_int64),
                ("n_angles", ctypes.c_int64), ("chunk", ctypes.c_int32), ("act", ctypes.c_int32),
                ("a_floor", ctypes.c_float)]

    @classmethod
    def make(cls, batch, seqlen, heads, headdim, d_state, groups, n_angles, act="bf16", a_floor=1e-4, chunk=0):
        code = ACT_CODES[act] if isinstance(act, str) else int(act)
        return cls(batch, seqlen, heads, headdim, d_state, groups, n_angles, chunk, code, a_floor)

    @property
    def act_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.act]

    @property
    def n_chunks(self) -> int:
        return -(-self.seqlen // 64)

    def shapes(self) -> dict:
        B, T, H, P, N, G, A = (self.batch, self.seqlen, self.heads, self.headdim, self.d_state, self.groups,
                               self.n_angles)
        return dict(x=(B, T, H * P), bc=(B, T, G, N), bth=(B, T, H), ang=(B, T, A), hn=(H, N), h=(H,),
                    states=(B, H, self.n_chunks, P, N))


def m3_states_bytes(d: M3Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba3_states_bytes(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def m3_workspace_bytes(d: M3Dims) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mamba3_workspace_bytes(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def _m3_inputs(d: M3Dims, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D):
    s, at, f = d.shapes(), d.act_dtype, torch.float32
    return [_ptr(x, "x", at, s["x"], True), _ptr(b_in, "b_in", at, s["bc"], True),
            _ptr(c_in, "c_in", at, s["bc"], True), _ptr(dd_dt_raw, "dd_dt_raw", f, s["bth"], True),
            _ptr(dd_a_raw, "dd_a_raw", f, s["bth"], True), _ptr(trap_raw, "trap_raw", f, s["bth"], True),
            _ptr(angles_raw, "angles_raw", f, s["ang"], d.n_angles > 0), _ptr(b_bias, "b_bias", f, s["hn"], True),
            _ptr(c_bias, "c_bias", f, s["hn"], True), _ptr(dt_bias, "dt_bias", f, s["h"], True),
            _ptr(D, "D", f, s["h"])]


def m3_fwd(d: M3Dims, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D=None, *,
           y, states, workspace, stream=None):
    s = d.shapes()
    args = [ctypes.byref(d)] + _m3_inputs(d, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias,
                                          c_bias, dt_bias, D)
    args += [_ptr(y, "y", d.act_dtype, s["x"], True), _ptr(states, "states", torch.float32, s["states"], True),
             *_workspace(workspace), _stream(stream)]
    _check(load().mamba3_siso_fwd(*args))


def m3_bwd(d: M3Dims, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D, states,
           dy, *, d_x, d_b_in, d_c_in, d_dd_dt_raw, d_dd_a_raw, d_trap_raw, d_angles_raw, d_b_bias, d_c_bias,
           d_dt_bias, d_D, workspace, stream=None):
    s, at, f = d.shapes(), d.act_dtype, torch.float32
    args = [ctypes.byref(d)] + _m3_inputs(d, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias,
                                          c_bias, dt_bias, D)
    args += [_ptr(states, "states", f, s["states"], True), _ptr(dy, "dy", at, s["x"], True),
             _ptr(d_x, "d_x", at, s["x"], True), _ptr(d_b_in, "d_b_in", at, s["bc"], True),
             _ptr(d_c_in, "d_c_in", at, s["bc"], True), _ptr(d_dd_dt_raw, "d_dd_dt_raw", f, s["bth"], True),
             _ptr(d_dd_a_raw, "d_dd_a_raw", f, s["bth"], True), _ptr(d_trap_raw, "d_trap_raw", f, s["bth"], True),
             _ptr(d_angles_raw, "d_angles_raw", f, s["ang"], d.n_angles > 0),
             _ptr(d_b_bias, "d_b_bias", f, s["hn"], True), _ptr(d_c_bias, "d_c_bias", f, s["hn"], True),
             _ptr(d_dt_bias, "d_dt_bias", f, s["h"], True), _ptr(d_D, "d_D", f, s["h"], D is not None),
             *_workspace(workspace), _stream(stream)]
    _check(load().mamba3_siso_bwd(*args))
