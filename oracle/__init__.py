"""Plain CPU oracle for the Mamba-1 selective-scan layer core.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product (the HIP
library and its binding) never imports this package, and this package
imports nothing from the product.

The arithmetic lives in ``mamba_oracle.c`` (double precision, sequential in
time, one channel at a time); this module only marshals numpy arrays into
it.  Channels are independent in every output except d_xdbl (a sum over
channels), so contiguous channel ranges are spread over threads (ctypes
releases the GIL); each range sums its d_xdbl into a private buffer and the
buffers are added afterwards in range order.

``precision="f32"`` runs the same C source built with float in place of
double.  That build only times the oracle on the host (the benchmark's CPU
baseline); parity is always checked against the double build.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_LIB_PATHS = {"f64": os.path.join(_HERE, "libmamba_oracle.so"),
              "f32": os.path.join(_HERE, "libmamba_oracle_f32.so")}
_LIB_PATH = _LIB_PATHS["f64"]
_DTYPES = {"f64": np.float64, "f32": np.float32}
_libs = {}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc: ``oracle/libmamba_oracle.so`` (double,
    the reference) and ``oracle/libmamba_oracle_f32.so`` (float, timing only)."""
    for prec, path in _LIB_PATHS.items():
        if force or not os.path.exists(path):
            tmp = path + ".tmp%d" % os.getpid()
            flags = ["-DORA_REAL=float"] if prec == "f32" else []
            subprocess.check_call(
                ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra"] + flags +
                ["-o", tmp, _SRC, "-lm"])
            os.replace(tmp, path)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("dt_rank", ctypes.c_int64), ("d_conv", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]


def _load(precision="f64"):
    lib = _libs.get(precision)
    if lib is None:
        path = _LIB_PATHS[precision]
        if not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int64
        lib.ora_forward.argtypes = [ctypes.POINTER(_Dims), I, I, I, I] + [P] * 16
        lib.ora_forward.restype = ctypes.c_int
        lib.ora_backward.argtypes = [ctypes.POINTER(_Dims), I, I, I, I] + [P] * 21
        lib.ora_backward.restype = ctypes.c_int
        _libs[precision] = lib
    return lib


def _cast(a, precision):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=_DTYPES[precision]))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(B, T, Di, Ds, R, K, L):
    return _Dims(B, T, Di, Ds, R, K, L)


def _shape_info(x, xdbl, a_log, conv_w, chunk):
    B, T, Di = x.shape
    Ds = a_log.shape[1]
    X = xdbl.shape[2]
    R = X - 2 * Ds
    K = 0 if conv_w is None else conv_w.shape[1]
    L = int(chunk) if chunk else 64
    return B, T, Di, Ds, R, K, L


def _channel_ranges(Di, threads):
    """Contiguous channel ranges, one per thread (at most one per channel)."""
    threads = max(1, min(int(threads), Di))
    bounds = np.linspace(0, Di, threads + 1).astype(int)
    return [(int(bounds[j]), int(bounds[j + 1])) for j in range(threads) if bounds[j] < bounds[j + 1]]


def default_threads():
    """Host threads to use: OMP_NUM_THREADS when set (a shared machine's share
    of cores), else the cores this process may run on, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def forward(x, delta_raw, a_log, xdbl, D=None, z=None, h0=None, conv_w=None, conv_b=None,
            conv_state0=None, chunk=64, threads=None, precision="f64"):
    """Forward pass.  ``x`` is u when ``conv_w`` is None, the conv input otherwise.

    Returns a dict with out, y (pre-gate), u (conv+SiLU output, = x without
    conv), h_last [B,Di,Ds], ckpt [B,nC,Ds,Di] and conv_state_last [B,Di,K]
    (only with conv).
    """
    lib = _load(precision)
    c = lambda a: _cast(a, precision)  # noqa: E731
    x, delta_raw, a_log, xdbl = c(x), c(delta_raw), c(a_log), c(xdbl)
    D, z, h0 = c(D), c(z), c(h0)
    conv_w, conv_b, conv_state0 = c(conv_w), c(conv_b), c(conv_state0)
    B, T, Di, Ds, R, K, L = _shape_info(x, xdbl, a_log, conv_w, chunk)
    nC = -(-T // L)
    dims = _dims(B, T, Di, Ds, R, K, L)
    ft = _DTYPES[precision]
    out = np.empty((B, T, Di), ft)
    y = np.empty((B, T, Di), ft)
    u = np.empty((B, T, Di), ft)
    h_last = np.empty((B, Di, Ds), ft)
    ckpt = np.empty((B, nC, Ds, Di), ft)
    csl = np.empty((B, Di, K), ft) if K > 0 else None

    def run(rng):
        rc = lib.ora_forward(ctypes.byref(dims), 0, B, rng[0], rng[1], _ptr(x), _ptr(conv_w), _ptr(conv_b),
                             _ptr(conv_state0), _ptr(delta_raw), _ptr(a_log), _ptr(xdbl), _ptr(D),
                             _ptr(z), _ptr(h0), _ptr(out), _ptr(y), _ptr(u), _ptr(h_last),
                             _ptr(csl), _ptr(ckpt))
        if rc != 0:
            raise RuntimeError("ora_forward failed with code %d" % rc)

    ranges = _channel_ranges(Di, threads or default_threads())
    with ThreadPoolExecutor(len(ranges)) as ex:
        list(ex.map(run, ranges))
    res = dict(out=out, y=y, u=u, h_last=h_last, ckpt=ckpt)
    if K > 0:
        res["conv_state_last"] = csl
    return res


def backward(x, delta_raw, a_log, xdbl, dout, D=None, z=None, h0=None, conv_w=None, conv_b=None,
             conv_state0=None, d_u_extra=None, threads=None, precision="f64"):
    """Backward pass of ``forward`` for the loss sum(dout*out) + sum(d_u_extra*u).

    Returns a dict with d_x (d_u without conv), d_delta_raw, d_delta,
    d_z (gate only), d_xdbl (B/C columns; dt columns are zero), d_a_log,
    d_D and, with conv, d_conv_w and d_conv_b.  Nothing is accumulated.
    """
    lib = _load(precision)
    c = lambda a: _cast(a, precision)  # noqa: E731
    x, delta_raw, a_log, xdbl, dout = c(x), c(delta_raw), c(a_log), c(xdbl), c(dout)
    D, z, h0 = c(D), c(z), c(h0)
    conv_w, conv_b, conv_state0, d_u_extra = c(conv_w), c(conv_b), c(conv_state0), c(d_u_extra)
    B, T, Di, Ds, R, K, L = _shape_info(x, xdbl, a_log, conv_w, 64)
    dims = _dims(B, T, Di, Ds, R, K, L)
    ft = _DTYPES[precision]
    d_x = np.empty((B, T, Di), ft)
    d_delta_raw = np.empty((B, T, Di), ft)
    d_delta = np.empty((B, T, Di), ft)
    d_z = np.empty((B, T, Di), ft) if z is not None else None
    d_a_log = np.empty((Di, Ds), ft)
    d_D = np.empty(Di, ft)
    d_conv_w = np.empty((Di, K), ft) if K > 0 else None
    d_conv_b = np.empty(Di, ft) if K > 0 else None
    ranges = _channel_ranges(Di, threads or default_threads())
    # each channel range sums its channels' d_B / d_C into a private buffer
    parts = [np.zeros((B, T, xdbl.shape[2]), ft) for _ in ranges]

    def run(j):
        rng = ranges[j]
        rc = lib.ora_backward(ctypes.byref(dims), 0, B, rng[0], rng[1], _ptr(x), _ptr(conv_w), _ptr(conv_b),
                              _ptr(conv_state0), _ptr(delta_raw), _ptr(a_log), _ptr(xdbl), _ptr(D),
                              _ptr(z), _ptr(h0), _ptr(dout), _ptr(d_u_extra), _ptr(d_x),
                              _ptr(d_delta_raw), _ptr(d_delta), _ptr(d_z), _ptr(parts[j]),
                              _ptr(d_a_log), _ptr(d_D), _ptr(d_conv_w), _ptr(d_conv_b))
        if rc != 0:
            raise RuntimeError("ora_backward failed with code %d" % rc)

    with ThreadPoolExecutor(len(ranges)) as ex:
        list(ex.map(run, range(len(ranges))))
    d_xdbl = parts[0]
    for p in parts[1:]:          # fixed order: channel ranges ascending
        d_xdbl += p
    res = dict(d_x=d_x, d_delta_raw=d_delta_raw, d_delta=d_delta, d_xdbl=d_xdbl, d_a_log=d_a_log, d_D=d_D)
    if d_z is not None:
        res["d_z"] = d_z
    if K > 0:
        res["d_conv_w"] = d_conv_w
        res["d_conv_b"] = d_conv_b
    return res
