"""Plain CPU oracle for one whole Mamba-1 layer around the selective-scan core.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite and
the benchmark's CPU-baseline leg are its only callers, and it imports
nothing from the product.

The steps follow the per-layer forward of the mamba-rs 0.3.1
``src/mamba_ssm/gpu/forward_mixed.rs`` page (the list of steps F1..F6 and
the launches behind them):
  F1  RMSNorm of the f32 residual stream (eps 1e-5), typed output
  F2  in_proj, one GEMM [B*T, d_model] -> [B*T, 2*d_inner]; the first
      d_inner columns are the x branch, the rest the gate input z
  F4a causal depthwise conv1d + SiLU of the x branch -> u
  F4b x_proj GEMM u -> xdbl = [dt | B | C]
  F4c dt_proj GEMM of the dt columns, plus its bias -> delta_raw
  F4d/e the selective-scan core (softplus, recurrence, C.h + D*u, gate),
      i.e. ``oracle.forward`` / ``oracle.backward``
  F5  out_proj GEMM [B*T, d_inner] -> [B*T, d_model]
  F6  residual add in f32
Readings where the page names a step but not its formula: RMSNorm is
x * w / sqrt(mean(x^2) + eps); the split puts x before z; the conv is the
same causal cross-correlation the core oracle reads (tap K-1 on x_t).

Everything is float64.  ``act`` ("bf16" / "f16" / None) rounds, to nearest
even, exactly the tensors the GPU layer stores in the activation dtype
(listed in ``ROUNDED_FWD`` / ``ROUNDED_BWD``); with None nothing is rounded,
which is what the finite-difference pins use.  The gate's adjoint reads y
as the forward stored it (the forward_mixed page keeps y among the typed
saved activations), so with ``act`` set d_z uses the rounded y.  The matrix products are
numpy's (a library primitive as one step).
"""
from __future__ import annotations

import numpy as np

from . import backward as core_backward
from . import forward as core_forward

NORM_EPS = 1e-5

# tensors held in the activation dtype between steps (forward, then backward)
ROUNDED_FWD = ("xn", "x", "z", "u", "xdbl", "delta_raw", "gated", "y")
ROUNDED_BWD = ("dy_act", "d_gated", "d_u_core", "d_delta_raw", "d_z", "d_xdbl_act", "d_x")


def round_bf16(a):
    """Round float64 values to bfloat16 (nearest even) and back, via float32."""
    f = np.asarray(a, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return (bits.astype(np.uint32)).view(np.float32).astype(np.float64)


def round_act(a, act):
    if act is None:
        return np.asarray(a, dtype=np.float64)
    if act == "bf16":
        return round_bf16(a)
    if act == "f16":
        return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)
    if act == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(act)


def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def rmsnorm(x, w, eps=NORM_EPS):
    """y = x * w / sqrt(mean(x^2) + eps) over the last axis; also returns 1/rms."""
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * rstd * w, rstd


def rmsnorm_backward(dy, x, w, rstd):
    """Adjoint of ``rmsnorm``: (d_x, d_w) for the loss sum(dy * y)."""
    g = dy * w
    dx = rstd * g - x * rstd ** 3 * np.mean(g * x, axis=-1, keepdims=True)
    dw = np.sum(dy * x * rstd, axis=tuple(range(dy.ndim - 1)))
    return dx, dw


def conv_silu(x, conv_w, conv_b):
    """u = silu(p), p_t = b + sum_k w[:, k] x_{t-K+1+k}, zero history. x: [B, T, Di]."""
    B, T, Di = x.shape
    K = conv_w.shape[1]
    p = np.zeros_like(x) + (0.0 if conv_b is None else conv_b)
    for k in range(K):
        shift = K - 1 - k                      # tap k reads x_{t - shift}
        p[:, shift:, :] += conv_w[:, k] * x[:, :T - shift, :]
    return p * sigmoid(p), p


def conv_silu_backward(du, x, conv_w, p):
    """Adjoint of ``conv_silu``: (d_x, d_conv_w, d_conv_b)."""
    B, T, Di = x.shape
    K = conv_w.shape[1]
    s = sigmoid(p)
    dp = du * s * (1.0 + p * (1.0 - s))
    dx = np.zeros_like(x)
    dw = np.zeros_like(conv_w)
    for k in range(K):
        shift = K - 1 - k
        dx[:, :T - shift, :] += conv_w[:, k] * dp[:, shift:, :]
        dw[:, k] = np.sum(dp[:, shift:, :] * x[:, :T - shift, :], axis=(0, 1))
    return dx, dw, np.sum(dp, axis=(0, 1))


def gate_backward(dout, y, z):
    """d_z of out = y * silu(z): dout * y * silu'(z), silu'(z) = s (1 + z (1 - s))."""
    s = sigmoid(z)
    return dout * y * s * (1.0 + z * (1.0 - s))


def layer_forward(resid, p, act=None, chunk=16):
    """One layer.  ``resid``: [B, T, d_model]; ``p``: dict of weights
    (norm_w [dm], w_in [2Di, dm], conv_w [Di, K], conv_b [Di], w_x [R+2Ds, Di],
    w_dt [Di, R], b_dt [Di], a_log [Di, Ds], D [Di], w_out [dm, Di]).
    Returns the new residual and the saved intermediates."""
    r = lambda a: round_act(a, act)
    Di = p["w_in"].shape[0] // 2
    Ds = p["a_log"].shape[1]
    R = p["w_dt"].shape[1]
    xn_f, rstd = rmsnorm(resid, p["norm_w"])
    xn = r(xn_f)
    xz = xn @ p["w_in"].T
    x, z = r(xz[..., :Di]), r(xz[..., Di:])
    u_f, pre = conv_silu(x, p["conv_w"], p["conv_b"])
    u = r(u_f)
    xdbl = r(u @ p["w_x"].T)
    delta_raw = r(xdbl[..., :R] @ p["w_dt"].T + p["b_dt"])
    core = core_forward(u, delta_raw, p["a_log"], xdbl, D=p["D"], z=z, chunk=chunk)
    gated = r(core["out"])
    out = resid + gated @ p["w_out"].T
    saved = dict(xn=xn, rstd=rstd, x=x, z=z, pre=pre, u=u, xdbl=xdbl, delta_raw=delta_raw, gated=gated,
                 y=r(core["y"]), Ds=Ds, R=R)
    return out, saved


def layer_backward(resid, p, saved, d_out, act=None):
    """Adjoint of ``layer_forward`` for the loss sum(d_out * out).  Returns
    d_resid and a dict of parameter gradients (nothing accumulated)."""
    r = lambda a: round_act(a, act)
    s = saved
    Di = p["w_in"].shape[0] // 2
    R = s["R"]
    g = {}
    dy = r(d_out)                                          # out_proj operands are typed
    g["w_out"] = np.einsum("btm,bti->mi", dy, s["gated"])
    d_gated = r(dy @ p["w_out"])
    cb = core_backward(s["u"], s["delta_raw"], p["a_log"], s["xdbl"], d_gated, D=p["D"], z=s["z"])
    d_u_core, d_delta_raw = r(cb["d_x"]), r(cb["d_delta_raw"])
    d_z = r(gate_backward(d_gated, s["y"], s["z"]))
    g["a_log"], g["D"] = cb["d_a_log"], cb["d_D"]
    d_xdbl = cb["d_xdbl"].copy()                           # B/C columns; dt columns next
    d_xdbl[..., :R] = d_delta_raw @ p["w_dt"]
    g["w_dt"] = np.einsum("bti,btr->ir", d_delta_raw, s["xdbl"][..., :R])
    g["b_dt"] = np.sum(d_delta_raw, axis=(0, 1))
    d_xdbl_act = r(d_xdbl)
    g["w_x"] = np.einsum("btc,bti->ci", d_xdbl_act, s["u"])
    d_u = d_u_core + d_xdbl_act @ p["w_x"]
    d_x, g["conv_w"], g["conv_b"] = conv_silu_backward(d_u, s["x"], p["conv_w"], s["pre"])
    d_x = r(d_x)
    g["w_in"] = np.concatenate([np.einsum("bti,btm->im", d_x, s["xn"]),
                                np.einsum("bti,btm->im", d_z, s["xn"])], axis=0)
    d_xn = d_x @ p["w_in"][:Di] + d_z @ p["w_in"][Di:]
    d_norm_in, g["norm_w"] = rmsnorm_backward(d_xn, resid, p["norm_w"], s["rstd"])
    return d_out + d_norm_in, g
