"""Plain CPU oracle for the Mamba-3 SISO selective state-space core.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite,
the package smoke check and the benchmark's CPU-baseline leg are its only
callers, and it imports nothing from the product.

What it computes.  The mamba-rs 0.4.0 ``src/mamba3_siso/gpu/backward_mixed.rs``
page ("Mamba-3 backward page") shows the per-layer backward of a Mamba-3
SISO layer as launches with their arguments, but neither the forward nor
any kernel body.  This module is the plain definition that those launches
are the chunked adjoint of, in the readings below (each one is what the
names and arguments on that page support; the page states none of them):

  per batch row b and head h (V = x split into heads of ``headdim``; the
  head uses B/C group h // (heads / groups), contiguous heads per group):
    dt_t    = softplus(dd_dt_raw_t + dt_bias_h)          ("dd_dt_raw", "dt_bias")
    A_t     = -max(softplus(dd_a_raw_t), a_floor)        ("dd_a_raw", "a_floor", "a_val")
    lam_t   = sigmoid(trap_raw_t)                        ("trap", "d_trap_raw")
    theta_t = sum_{s<=t} dt_s * angles_raw_s             ("angle_cumsum", "angles_raw";
                                                           one angle per pair, shared by heads)
    K_t     = rot(theta_t)(B_t + b_bias_h),  Q_t = rot(theta_t)(C_t + c_bias_h)
              (rot turns state pairs (a, a + n_angles), a < n_angles, by
              theta_t[a]; later state dims are not turned)   ("K_raw = b_biased",
              "Q_rot", "d_b_pre_rope", "bc_bias_add_bwd")
    alpha_t = exp(dt_t A_t)
    S_t     = alpha_t S_{t-1} + (1 - lam_t) dt_t alpha_t V_{t-1} K_{t-1}^T
              + lam_t dt_t V_t K_t^T                      (exponential-trapezoidal
              update: "trap", "gamma", "scale", "k_scaled"; S_{-1} = 0 and
              V_{-1} K_{-1} = 0)
    y_t     = S_t Q_t + D_h V_t                           ("d_param", "dD_partials")

with S_t a [headdim, d_state] matrix.  Everything is float64 and sequential
in time: every S_t is formed, nothing is chunked.  ``backward`` is the
exact reverse-time adjoint of ``forward``, step by step, followed by the
chain rule through the rotation, the angle sum, softplus, sigmoid, the
clamp, the bias and the group broadcast.  Gradients are returned for every
input; where the clamp of A is active (softplus(dd_a_raw) <= a_floor) the
gradient of dd_a_raw is 0.
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _rotate(v, theta, na):
    """Turn pairs (a, a + na) of the last axis of v by theta[..., a]."""
    if na == 0:
        return v.copy()
    c, s = np.cos(theta), np.sin(theta)
    out = v.copy()
    x1, x2 = v[..., :na], v[..., na:2 * na]
    out[..., :na] = x1 * c - x2 * s
    out[..., na:2 * na] = x1 * s + x2 * c
    return out


def _rotate_back(g, theta, na):
    """Transpose of _rotate: gradient with respect to the unturned vector."""
    if na == 0:
        return g.copy()
    c, s = np.cos(theta), np.sin(theta)
    out = g.copy()
    g1, g2 = g[..., :na], g[..., na:2 * na]
    out[..., :na] = g1 * c + g2 * s
    out[..., na:2 * na] = -g1 * s + g2 * c
    return out


def _prepare(x, b_in, c_in, dd_dt, dd_a, trap, angles, b_bias, c_bias, dt_bias, a_floor, heads, headdim):
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, b_in, c_in, dd_dt, dd_a, trap, angles = map(f, (x, b_in, c_in, dd_dt, dd_a, trap, angles))
    b_bias, c_bias, dt_bias = map(f, (b_bias, c_bias, dt_bias))
    B, T, _ = x.shape
    ng, N = b_in.shape[2], b_in.shape[3]
    na = angles.shape[2]
    assert heads % ng == 0 and 2 * na <= N
    grp = np.arange(heads) // (heads // ng)
    V = x.reshape(B, T, heads, headdim)
    Kb = b_in[:, :, grp, :] + b_bias[None, None]
    Qb = c_in[:, :, grp, :] + c_bias[None, None]
    dt = softplus(dd_dt + dt_bias[None, None])
    sa = softplus(dd_a)
    A = -np.maximum(sa, a_floor)
    lam = sigmoid(trap)
    theta = np.cumsum(dt[..., None] * angles[:, :, None, :], axis=1)   # [B, T, heads, na]
    K = _rotate(Kb, theta, na)
    Q = _rotate(Qb, theta, na)
    alpha = np.exp(dt * A)
    return dict(B=B, T=T, H=heads, P=headdim, N=N, ng=ng, na=na, grp=grp, V=V, Kb=Kb, Qb=Qb, dt=dt, sa=sa,
                A=A, lam=lam, theta=theta, K=K, Q=Q, alpha=alpha, dd_dt=dd_dt, dd_a=dd_a, angles=angles,
                dt_bias=dt_bias, a_floor=a_floor)


def forward(x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D, a_floor,
            heads, headdim, keep_states=False):
    """y [B, T, heads * headdim] (and, with keep_states, every S_t as
    [B, T, heads, headdim, d_state]).

    x [B, T, heads * headdim]; b_in, c_in [B, T, groups, d_state];
    dd_dt_raw, dd_a_raw, trap_raw [B, T, heads]; angles_raw [B, T, n_angles];
    b_bias, c_bias [heads, d_state]; dt_bias, D [heads]; a_floor a float."""
    p = _prepare(x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, a_floor,
                 heads, headdim)
    B, T, H, P, N = p["B"], p["T"], p["H"], p["P"], p["N"]
    V, K, Q, dt, lam, alpha = p["V"], p["K"], p["Q"], p["dt"], p["lam"], p["alpha"]
    Dh = np.asarray(D, dtype=np.float64)
    S = np.zeros((B, H, P, N))
    y = np.empty((B, T, H, P))
    states = np.empty((B, T, H, P, N)) if keep_states else None
    for t in range(T):
        S = alpha[:, t, :, None, None] * S
        S += (lam[:, t] * dt[:, t])[:, :, None, None] * V[:, t, :, :, None] * K[:, t, :, None, :]
        if t > 0:
            beta = (1.0 - lam[:, t]) * dt[:, t] * alpha[:, t]
            S += beta[:, :, None, None] * V[:, t - 1, :, :, None] * K[:, t - 1, :, None, :]
        y[:, t] = np.einsum("bhpn,bhn->bhp", S, Q[:, t]) + Dh[None, :, None] * V[:, t]
        if keep_states:
            states[:, t] = S
    y = y.reshape(B, T, H * P)
    return (y, states) if keep_states else y


def backward(dy, x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D, a_floor,
             heads, headdim):
    """Gradients of sum(dy * y) with respect to every input, as a dict:
    x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias,
    dt_bias, D (shapes as the inputs)."""
    p = _prepare(x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, a_floor,
                 heads, headdim)
    B, T, H, P, N, na = p["B"], p["T"], p["H"], p["P"], p["N"], p["na"]
    V, K, Q, dt, A, lam, alpha = p["V"], p["K"], p["Q"], p["dt"], p["A"], p["lam"], p["alpha"]
    Dh = np.asarray(D, dtype=np.float64)
    _, states = forward(x, b_in, c_in, dd_dt_raw, dd_a_raw, trap_raw, angles_raw, b_bias, c_bias, dt_bias, D,
                        a_floor, heads, headdim, keep_states=True)
    dY = np.asarray(dy, dtype=np.float64).reshape(B, T, H, P)

    dV = np.zeros_like(V)
    dK = np.zeros_like(K)
    dQ = np.zeros_like(Q)
    d_alpha = np.zeros_like(dt)
    d_beta = np.zeros_like(dt)
    d_gamma = np.zeros_like(dt)
    dD = np.zeros(H)
    dS = np.zeros((B, H, P, N))
    for t in range(T - 1, -1, -1):
        # y_t = S_t Q_t + D V_t
        dS += dY[:, t, :, :, None] * Q[:, t, :, None, :]
        dQ[:, t] += np.einsum("bhpn,bhp->bhn", states[:, t], dY[:, t])
        dV[:, t] += Dh[None, :, None] * dY[:, t]
        dD += np.einsum("bhp,bhp->h", dY[:, t], V[:, t])
        # S_t = alpha_t S_{t-1} + beta_t V_{t-1} K_{t-1}^T + gamma_t V_t K_t^T
        S_prev = states[:, t - 1] if t > 0 else np.zeros((B, H, P, N))
        d_alpha[:, t] = np.einsum("bhpn,bhpn->bh", dS, S_prev)
        gam = lam[:, t] * dt[:, t]
        d_gamma[:, t] = np.einsum("bhpn,bhp,bhn->bh", dS, V[:, t], K[:, t])
        dV[:, t] += gam[:, :, None] * np.einsum("bhpn,bhn->bhp", dS, K[:, t])
        dK[:, t] += gam[:, :, None] * np.einsum("bhpn,bhp->bhn", dS, V[:, t])
        if t > 0:
            beta = (1.0 - lam[:, t]) * dt[:, t] * alpha[:, t]
            d_beta[:, t] = np.einsum("bhpn,bhp,bhn->bh", dS, V[:, t - 1], K[:, t - 1])
            dV[:, t - 1] += beta[:, :, None] * np.einsum("bhpn,bhn->bhp", dS, K[:, t - 1])
            dK[:, t - 1] += beta[:, :, None] * np.einsum("bhpn,bhp->bhn", dS, V[:, t - 1])
        dS = alpha[:, t, :, None, None] * dS

    # per-step scalars: alpha = exp(dt A), beta = (1 - lam) dt alpha, gamma = lam dt
    d_alpha_tot = d_alpha + d_beta * (1.0 - lam) * dt
    d_dt = d_alpha_tot * alpha * A + d_beta * (1.0 - lam) * alpha + d_gamma * lam
    d_A = d_alpha_tot * alpha * dt
    d_lam = -d_beta * dt * alpha + d_gamma * dt

    # rotation: K = rot(theta) Kb, Q = rot(theta) Qb; d rot/d theta turns each
    # pair by a right angle: d(x1', x2')/d theta = (-x2', x1')
    d_theta = np.zeros_like(p["theta"])
    if na:
        for Mr, dM in ((K, dK), (Q, dQ)):
            d_theta += -dM[..., :na] * Mr[..., na:2 * na] + dM[..., na:2 * na] * Mr[..., :na]
    dKb = _rotate_back(dK, p["theta"], na)
    dQb = _rotate_back(dQ, p["theta"], na)
    # theta_t = sum_{s<=t} dt_s angles_s: reverse cumulative sum
    g = np.flip(np.cumsum(np.flip(d_theta, axis=1), axis=1), axis=1)       # [B, T, H, na]
    d_angles = np.einsum("bthA,bth->btA", g, dt)
    d_dt += np.einsum("bthA,btA->bth", g, p["angles"])

    # scalar chains
    d_dd_dt = d_dt * sigmoid(p["dd_dt"] + p["dt_bias"][None, None])
    d_dt_bias = d_dd_dt.sum(axis=(0, 1))
    active = p["sa"] > p["a_floor"]
    d_dd_a = np.where(active, -d_A * sigmoid(p["dd_a"]), 0.0)
    d_trap = d_lam * lam * (1.0 - lam)

    # bias and group broadcast
    grp, ng = p["grp"], p["ng"]
    d_b_in = np.zeros((B, T, ng, N))
    d_c_in = np.zeros((B, T, ng, N))
    for h in range(H):
        d_b_in[:, :, grp[h]] += dKb[:, :, h]
        d_c_in[:, :, grp[h]] += dQb[:, :, h]
    return {"x": dV.reshape(B, T, H * P), "b_in": d_b_in, "c_in": d_c_in, "dd_dt_raw": d_dd_dt,
            "dd_a_raw": d_dd_a, "trap_raw": d_trap, "angles_raw": d_angles, "b_bias": dKb.sum(axis=(0, 1)),
            "c_bias": dQb.sum(axis=(0, 1)), "dt_bias": d_dt_bias, "D": dD}
