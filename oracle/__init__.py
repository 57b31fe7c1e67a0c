"""Plain CPU oracle for the Mamba-1 selective-scan layer core.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product (the HIP
library and its binding) never imports this package, and this package
imports nothing from the product.

The arithmetic lives in ``mamba_oracle.c`` (double precision, sequential in
time, one channel at a time); this module only marshals numpy arrays into
it.  Batch rows are independent in every output except the parameter
gradients, so rows are spread over threads (ctypes releases the GIL) and the
per-row parameter gradients are summed afterwards in row order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmamba_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/libmamba_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("dt_rank", ctypes.c_int64), ("d_conv", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.ora_forward.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.c_int64] + [P] * 16
        lib.ora_forward.restype = ctypes.c_int
        lib.ora_backward.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.c_int64] + [P] * 21
        lib.ora_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


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


def _row_groups(B, threads):
    threads = max(1, min(int(threads), B))
    bounds = np.linspace(0, B, threads + 1).astype(int)
    return [(int(bounds[j]), int(bounds[j + 1])) for j in range(threads) if bounds[j] < bounds[j + 1]]


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def forward(x, delta_raw, a_log, xdbl, D=None, z=None, h0=None, conv_w=None, conv_b=None,
            conv_state0=None, chunk=64, threads=None):
    """Forward pass.  ``x`` is u when ``conv_w`` is None, the conv input otherwise.

    Returns a dict with out, y (pre-gate), u (conv+SiLU output, = x without
    conv), h_last [B,Di,Ds], ckpt [B,nC,Ds,Di] and conv_state_last [B,Di,K]
    (only with conv).
    """
    lib = _load()
    x, delta_raw, a_log, xdbl = _f64(x), _f64(delta_raw), _f64(a_log), _f64(xdbl)
    D, z, h0 = _f64(D), _f64(z), _f64(h0)
    conv_w, conv_b, conv_state0 = _f64(conv_w), _f64(conv_b), _f64(conv_state0)
    B, T, Di, Ds, R, K, L = _shape_info(x, xdbl, a_log, conv_w, chunk)
    nC = -(-T // L)
    dims = _dims(B, T, Di, Ds, R, K, L)
    out = np.empty((B, T, Di))
    y = np.empty((B, T, Di))
    u = np.empty((B, T, Di))
    h_last = np.empty((B, Di, Ds))
    ckpt = np.empty((B, nC, Ds, Di))
    csl = np.empty((B, Di, K)) if K > 0 else None

    def run(rng):
        rc = lib.ora_forward(ctypes.byref(dims), rng[0], rng[1], _ptr(x), _ptr(conv_w), _ptr(conv_b),
                             _ptr(conv_state0), _ptr(delta_raw), _ptr(a_log), _ptr(xdbl), _ptr(D),
                             _ptr(z), _ptr(h0), _ptr(out), _ptr(y), _ptr(u), _ptr(h_last),
                             _ptr(csl), _ptr(ckpt))
        if rc != 0:
            raise RuntimeError("ora_forward failed with code %d" % rc)

    groups = _row_groups(B, threads or default_threads())
    with ThreadPoolExecutor(len(groups)) as ex:
        list(ex.map(run, groups))
    res = dict(out=out, y=y, u=u, h_last=h_last, ckpt=ckpt)
    if K > 0:
        res["conv_state_last"] = csl
    return res


def backward(x, delta_raw, a_log, xdbl, dout, D=None, z=None, h0=None, conv_w=None, conv_b=None,
             conv_state0=None, d_u_extra=None, threads=None):
    """Backward pass of ``forward`` for the loss sum(dout*out) + sum(d_u_extra*u).

    Returns a dict with d_x (d_u without conv), d_delta_raw, d_delta,
    d_z (gate only), d_xdbl (B/C columns; dt columns are zero), d_a_log,
    d_D and, with conv, d_conv_w and d_conv_b.  Nothing is accumulated.
    """
    lib = _load()
    x, delta_raw, a_log, xdbl, dout = _f64(x), _f64(delta_raw), _f64(a_log), _f64(xdbl), _f64(dout)
    D, z, h0 = _f64(D), _f64(z), _f64(h0)
    conv_w, conv_b, conv_state0, d_u_extra = _f64(conv_w), _f64(conv_b), _f64(conv_state0), _f64(d_u_extra)
    B, T, Di, Ds, R, K, L = _shape_info(x, xdbl, a_log, conv_w, 64)
    dims = _dims(B, T, Di, Ds, R, K, L)
    d_x = np.empty((B, T, Di))
    d_delta_raw = np.empty((B, T, Di))
    d_delta = np.empty((B, T, Di))
    d_z = np.empty((B, T, Di)) if z is not None else None
    d_xdbl = np.zeros((B, T, xdbl.shape[2]))
    groups = _row_groups(B, threads or default_threads())
    parts = []
    for _ in groups:
        p = dict(d_a_log=np.empty((Di, Ds)), d_D=np.empty(Di))
        if K > 0:
            p["d_conv_w"] = np.empty((Di, K))
            p["d_conv_b"] = np.empty(Di)
        parts.append(p)

    def run(j):
        rng, p = groups[j], parts[j]
        rc = lib.ora_backward(ctypes.byref(dims), rng[0], rng[1], _ptr(x), _ptr(conv_w), _ptr(conv_b),
                              _ptr(conv_state0), _ptr(delta_raw), _ptr(a_log), _ptr(xdbl), _ptr(D),
                              _ptr(z), _ptr(h0), _ptr(dout), _ptr(d_u_extra), _ptr(d_x),
                              _ptr(d_delta_raw), _ptr(d_delta), _ptr(d_z), _ptr(d_xdbl),
                              _ptr(p["d_a_log"]), _ptr(p["d_D"]), _ptr(p.get("d_conv_w")),
                              _ptr(p.get("d_conv_b")))
        if rc != 0:
            raise RuntimeError("ora_backward failed with code %d" % rc)

    with ThreadPoolExecutor(len(groups)) as ex:
        list(ex.map(run, range(len(groups))))
    res = dict(d_x=d_x, d_delta_raw=d_delta_raw, d_delta=d_delta, d_xdbl=d_xdbl)
    if d_z is not None:
        res["d_z"] = d_z
    for key in parts[0]:
        acc = np.zeros_like(parts[0][key])
        for p in parts:          # fixed order: row groups ascending
            acc += p[key]
        res[key] = acc
    return res
