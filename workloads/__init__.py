"""Seeded synthetic inputs for the selective-scan layer core.

This module only draws random numbers and rounds them to the activation
dtype; it holds none of the method's arithmetic.  Both the oracle-side tests
and the GPU side consume the arrays it returns, so the two always see the
same (already rounded) values.

Workloads follow the shapes and value distributions of the five
configurations the layer core is measured on (see ``CONFIGS``).  Draw order
per layer: x (or u), delta_raw, B, C, z, dout, then the conv weights, then the
dt columns of xdbl, all from ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

ACT_DTYPES = ("f32", "bf16", "f16")


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    dt_rank: int
    d_conv: int          # 0: no convolution (scan-only entry points)
    act: str             # activation dtype: "f32" | "bf16" | "f16"
    gate: bool           # z gate present
    chunk: int = 0       # checkpoint interval; 0 = library default
    layers: int = 1
    delta_mean: float = -4.0   # delta_raw ~ N(delta_mean, 1)
    conv_std: float = 0.5      # conv weights and bias ~ N(0, conv_std^2)

    @property
    def xdbl_dim(self) -> int:
        return self.dt_rank + 2 * self.d_state

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    # single layer, f32 throughout, no conv and no gate
    "tiny_f32": Workload("tiny_f32", 1, 64, 16, 4, 0, 0, "f32", False, delta_mean=0.0),
    # conv1d(4) + SiLU + scan + gate, bf16 activations (d_model 128 -> d_inner 256)
    "fused_small_bf16": Workload("fused_small_bf16", 8, 128, 256, 16, 8, 4, "bf16", True),
    # scan + gate at a ~130M-model layer shape, bf16
    "scan_130m_bf16": Workload("scan_130m_bf16", 4, 2048, 1536, 16, 0, 0, "bf16", True),
    # long-sequence scan + gate at a ~2.8B-model layer shape, bf16
    "scan_2p8b_t8192_bf16": Workload("scan_2p8b_t8192_bf16", 2, 8192, 5120, 16, 0, 0, "bf16", True),
    # 24 stacked fused layers (d_model 1024 -> d_inner 2048), f16
    "fused_24l_f16": Workload("fused_24l_f16", 8, 4096, 2048, 16, 64, 4, "f16", True, layers=24),
}


def round_to(act: str, a) -> np.ndarray:
    """Round to the activation dtype (round-to-nearest-even); returns float32."""
    a = np.asarray(a, dtype=np.float32)
    if act == "f32":
        return np.ascontiguousarray(a)
    if act == "f16":
        return a.astype(np.float16).astype(np.float32)
    if act == "bf16":
        bits = np.ascontiguousarray(a).view(np.uint32).astype(np.uint64)
        bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
        return bits.astype(np.uint32).view(np.float32)
    raise ValueError("unknown activation dtype %r" % act)


def s4d_real_a_log(d_inner: int, d_state: int) -> np.ndarray:
    """a_log[i, n] = log(n + 1), i.e. A = -(n + 1) (S4D-real initialisation)."""
    return np.ascontiguousarray(
        np.broadcast_to(np.log(np.arange(1, d_state + 1, dtype=np.float64)), (d_inner, d_state))
    ).astype(np.float32)


def make_inputs(w: Workload, seed: int = 0, h0: bool = False, conv_state0: bool = False,
                d_u_extra: bool = False) -> dict:
    """Draw one layer's inputs.  Activations come back as float32 arrays whose
    values are exactly representable in ``w.act``; parameters are float32.

    Keys: x (u for scan-only workloads), delta_raw, xdbl, z (gate only), dout,
    a_log, D, and with conv: conv_w, conv_b.  Optional: h0, conv_state0,
    d_u_extra (independent extra draws after everything else).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Di, Ds, R = w.batch, w.seqlen, w.d_inner, w.d_state, w.dt_rank
    shape = (B, T, Di)

    def normal(size, mean=0.0, std=1.0):
        a = rng.standard_normal(size, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        if mean != 0.0:
            a += np.float32(mean)
        return a

    out = {}
    out["x"] = round_to(w.act, normal(shape))
    out["delta_raw"] = round_to(w.act, normal(shape, mean=w.delta_mean))
    Bm = normal((B, T, Ds))
    Cm = normal((B, T, Ds))
    out["z"] = round_to(w.act, normal(shape)) if w.gate else None
    out["dout"] = round_to(w.act, normal(shape))
    if w.d_conv > 0:
        out["conv_w"] = normal((Di, w.d_conv), std=w.conv_std)
        out["conv_b"] = normal((Di,), std=w.conv_std)
    xdbl = np.empty((B, T, R + 2 * Ds), dtype=np.float32)
    xdbl[..., R:R + Ds] = Bm
    xdbl[..., R + Ds:] = Cm
    if R > 0:
        xdbl[..., :R] = normal((B, T, R))   # dt columns: never read by the core
    out["xdbl"] = round_to(w.act, xdbl)
    out["a_log"] = s4d_real_a_log(Di, Ds)
    out["D"] = np.ones(Di, dtype=np.float32)
    if h0:
        out["h0"] = normal((B, Di, Ds), std=0.5)
    if conv_state0 and w.d_conv > 0:
        out["conv_state0"] = round_to(w.act, normal((B, Di, w.d_conv)))
    if d_u_extra:
        out["d_u_extra"] = round_to(w.act, normal(shape, std=0.5))
    return out


# ------------------------------------------------------------- whole layer


@dataclass(frozen=True)
class LayerWorkload:
    """One Mamba-1 layer: residual width d_model around the core's sizes."""
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    d_state: int
    dt_rank: int
    d_conv: int
    act: str

    def with_(self, **kw) -> "LayerWorkload":
        return replace(self, **kw)


LAYER_CONFIGS = {
    # small layer the oracle finishes in seconds (several tiles, ragged tail)
    "layer_small_bf16": LayerWorkload("layer_small_bf16", 2, 150, 96, 192, 16, 6, 4, "bf16"),
    # the 130M model's layer shape (d_model 768, d_inner 1536, dt_rank 48), B=4, T=2048
    "layer_130m_bf16": LayerWorkload("layer_130m_bf16", 4, 2048, 768, 1536, 16, 48, 4, "bf16"),
    # the 2.8B model's layer widths (d_model 2560, d_inner 5120, dt_rank 160), B=2, T=2048
    "layer_2p8b_t2048_bf16": LayerWorkload("layer_2p8b_t2048_bf16", 2, 2048, 2560, 5120, 16, 160, 4, "bf16"),
}


def make_layer_inputs(w: LayerWorkload, seed: int = 0) -> dict:
    """Draw a layer's weights, input residual and output-residual gradient.

    Readings (the pages give shapes, not initialisations): residual and its
    gradient N(0, 1); norm weight 1 + N(0, 0.1^2); projections N(0, 1/fan_in);
    conv weight and bias N(0, 0.5^2); dt bias the inverse softplus of
    dt = exp(U(log 1e-3, log 1e-1)); a_log S4D-real; D = 1.  The projection
    weights come back rounded to the activation dtype (the compute copies
    a layer multiplies with), everything else float32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, dm, Di, Ds, R, K = w.batch, w.seqlen, w.d_model, w.d_inner, w.d_state, w.dt_rank, w.d_conv
    X = R + 2 * Ds

    def normal(size, std=1.0):
        a = rng.standard_normal(size, dtype=np.float32)
        return a * np.float32(std) if std != 1.0 else a

    out = {}
    out["resid"] = normal((B, T, dm))
    out["norm_w"] = 1.0 + normal((dm,), 0.1)
    out["w_in"] = round_to(w.act, normal((2 * Di, dm), dm ** -0.5))
    out["conv_w"] = normal((Di, K), 0.5)
    out["conv_b"] = normal((Di,), 0.5)
    out["w_x"] = round_to(w.act, normal((X, Di), Di ** -0.5))
    out["w_dt"] = round_to(w.act, normal((Di, R), R ** -0.5))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), Di))
    out["b_dt"] = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    out["a_log"] = s4d_real_a_log(Di, Ds)
    out["D"] = np.ones(Di, dtype=np.float32)
    out["w_out"] = round_to(w.act, normal((dm, Di), Di ** -0.5))
    out["d_resid_out"] = normal((B, T, dm))
    return out


# ------------------------------------------------- Mamba-3 SISO state-space core


@dataclass(frozen=True)
class M3Workload:
    """One Mamba-3 SISO layer core: x split into `heads` heads of `headdim`
    channels, B/C in `groups` groups of `d_state`, `n_angles` rotation
    angles per step."""
    name: str
    batch: int
    seqlen: int
    heads: int
    headdim: int
    d_state: int
    groups: int
    n_angles: int
    act: str
    a_floor: float = 1e-4

    @property
    def d_inner(self) -> int:
        return self.heads * self.headdim

    def with_(self, **kw) -> "M3Workload":
        return replace(self, **kw)


M3_CONFIGS = {
    # small: three 64-step chunks and a ragged tail, two B/C groups
    "m3_small_bf16": M3Workload("m3_small_bf16", 2, 200, 4, 64, 64, 2, 16, "bf16"),
    # d_model 768 -> d_inner 1536 = 24 heads of 64, d_state 128, half of the
    # state dims turned (32 angles), B=4, T=2048
    "m3_siso_bf16": M3Workload("m3_siso_bf16", 4, 2048, 24, 64, 128, 1, 32, "bf16"),
}


def make_m3_inputs(w: M3Workload, seed: int = 0) -> dict:
    """Draw one Mamba-3 SISO core's inputs and its output gradient.

    Readings (the pages give names and shapes only): x, the normalised B and
    C, trap_raw, dd_a_raw and dy N(0, 1); dd_dt_raw N(0, 0.5^2) around a dt
    bias that is the inverse softplus of dt = exp(U(log 1e-3, log 1e-1)) per
    head; angles_raw N(0, 1); B and C biases N(0, 0.1^2); D = 1.  The
    activations (x, B, C, dy) come back rounded to the activation dtype,
    everything else float32.

    Keys: x [B,T,heads*headdim], b_in / c_in [B,T,groups,d_state],
    dd_dt_raw / dd_a_raw / trap_raw [B,T,heads], angles_raw [B,T,n_angles],
    b_bias / c_bias [heads,d_state], dt_bias / D [heads], dy.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, P, N, G, NA = w.batch, w.seqlen, w.heads, w.headdim, w.d_state, w.groups, w.n_angles

    def normal(size, std=1.0):
        a = rng.standard_normal(size, dtype=np.float32)
        return a * np.float32(std) if std != 1.0 else a

    out = {}
    out["x"] = round_to(w.act, normal((B, T, H * P)))
    out["b_in"] = round_to(w.act, normal((B, T, G, N)))
    out["c_in"] = round_to(w.act, normal((B, T, G, N)))
    out["dd_dt_raw"] = normal((B, T, H), 0.5)
    out["dd_a_raw"] = normal((B, T, H))
    out["trap_raw"] = normal((B, T, H))
    out["angles_raw"] = normal((B, T, NA))
    out["b_bias"] = normal((H, N), 0.1)
    out["c_bias"] = normal((H, N), 0.1)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H))
    out["dt_bias"] = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    out["D"] = np.ones(H, dtype=np.float32)
    out["dy"] = round_to(w.act, normal((B, T, H * P)))
    return out
