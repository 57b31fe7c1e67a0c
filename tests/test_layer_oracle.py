"""Pins of the whole-layer oracle (oracle/layer.py) against facts other than
itself: finite differences of the unrounded layer, the core oracle's own
conv path, closed forms of RMSNorm, an exact identity, and the rounding
helper against hand-worked ties and torch's conversion."""
import numpy as np
import pytest

import oracle
from oracle import layer as L


def _params(rng, dm=5, Di=6, Ds=4, R=2, K=3):
    X = R + 2 * Ds
    return dict(norm_w=1.0 + 0.3 * rng.standard_normal(dm),
                w_in=0.4 * rng.standard_normal((2 * Di, dm)),
                conv_w=0.5 * rng.standard_normal((Di, K)),
                conv_b=0.3 * rng.standard_normal(Di),
                w_x=0.4 * rng.standard_normal((X, Di)),
                w_dt=0.5 * rng.standard_normal((Di, R)),
                b_dt=-1.0 + 0.3 * rng.standard_normal(Di),
                a_log=np.log(np.tile(np.arange(1, Ds + 1, dtype=np.float64), (Di, 1))) + 0.1 * rng.standard_normal((Di, Ds)),
                D=1.0 + 0.2 * rng.standard_normal(Di),
                w_out=0.4 * rng.standard_normal((dm, Di)))


def _loss(resid, p, G):
    out, _ = L.layer_forward(resid, p)
    return float(np.sum(out * G))


def test_layer_gradients_match_finite_differences():
    """Every parameter gradient and the input gradient of the unrounded layer
    against central differences of the forward (loss sum(G * out))."""
    rng = np.random.default_rng(11)
    B, T, dm = 2, 7, 5
    p = _params(rng, dm=dm)
    resid = rng.standard_normal((B, T, dm))
    G = rng.standard_normal((B, T, dm))
    out, saved = L.layer_forward(resid, p)
    d_resid, g = L.layer_backward(resid, p, saved, G)
    eps = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + eps
        lp = _loss(resid, p, G)
        arr[idx] = old - eps
        lm = _loss(resid, p, G)
        arr[idx] = old
        return (lp - lm) / (2 * eps)

    checks = [(name, p[name], g[name]) for name in p] + [("resid", resid, d_resid)]
    for name, arr, ana in checks:
        assert ana.shape == arr.shape, name
        idxs = list(np.ndindex(arr.shape))
        if len(idxs) > 24:
            idxs = [idxs[j] for j in rng.choice(len(idxs), 24, replace=False)]
        num = np.array([fd(arr, ix) for ix in idxs])
        an = np.array([ana[ix] for ix in idxs])
        np.testing.assert_allclose(an, num, rtol=1e-5, atol=1e-7, err_msg=name)


def test_gate_backward_matches_the_core_oracle():
    """The layer's d_z formula (used so that it can read the stored, rounded
    y) equals the core oracle's d_z when nothing is rounded."""
    rng = np.random.default_rng(9)
    B, T, Di, Ds = 2, 11, 6, 4
    u, dr, z, dout = (rng.standard_normal((B, T, Di)) for _ in range(4))
    dr -= 3.0
    xdbl = rng.standard_normal((B, T, 2 * Ds))
    a_log = np.log(np.tile(np.arange(1.0, Ds + 1), (Di, 1)))
    f = oracle.forward(u, dr, a_log, xdbl, D=np.ones(Di), z=z, chunk=16)
    g = oracle.backward(u, dr, a_log, xdbl, dout, D=np.ones(Di), z=z)
    np.testing.assert_allclose(L.gate_backward(dout, f["y"], z), g["d_z"], rtol=1e-12, atol=1e-14)


def test_conv_matches_the_core_oracle_conv_path():
    """The layer's conv + SiLU (numpy, tap by tap) equals the u the core
    oracle's fused path computes (C, step by step) from the same input."""
    rng = np.random.default_rng(3)
    B, T, Di, Ds, K = 2, 9, 6, 4, 4
    x = rng.standard_normal((B, T, Di))
    w = 0.5 * rng.standard_normal((Di, K))
    b = 0.3 * rng.standard_normal(Di)
    u, _ = L.conv_silu(x, w, b)
    f = oracle.forward(x, rng.standard_normal((B, T, Di)), np.zeros((Di, Ds)), rng.standard_normal((B, T, 2 * Ds)),
                       conv_w=w, conv_b=b, chunk=16)
    np.testing.assert_allclose(u, f["u"], rtol=1e-13, atol=1e-13)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 4, 8))
    ones = np.ones(8)
    y, rstd = L.rmsnorm(x, ones)
    m = np.mean(x * x, axis=-1)
    # with unit weights the output's mean square is m / (m + eps)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), m / (m + L.NORM_EPS), rtol=1e-12)
    np.testing.assert_allclose(rstd[..., 0], 1.0 / np.sqrt(m + L.NORM_EPS), rtol=1e-12)
    # without eps the output does not depend on the input's scale
    y1, _ = L.rmsnorm(x, ones, eps=0.0)
    y2, _ = L.rmsnorm(7.5 * x, ones, eps=0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-12)
    # a constant row c gives w * sign(c) up to eps
    y3, _ = L.rmsnorm(np.full((1, 8), -3.0), np.arange(1.0, 9.0), eps=0.0)
    np.testing.assert_allclose(y3[0], -np.arange(1.0, 9.0), rtol=1e-12)


@pytest.mark.parametrize("act", [None, "bf16"])
def test_zero_out_proj_leaves_the_residual(act):
    rng = np.random.default_rng(5)
    p = _params(rng)
    p["w_out"] = np.zeros_like(p["w_out"])
    resid = rng.standard_normal((2, 6, 5))
    G = rng.standard_normal((2, 6, 5))
    out, saved = L.layer_forward(resid, p, act=act)
    assert np.array_equal(out, resid)
    d_resid, g = L.layer_backward(resid, p, saved, G, act=act)
    assert np.array_equal(d_resid, G)
    for name in ("w_in", "w_x", "w_dt", "b_dt", "conv_w", "conv_b", "norm_w", "a_log", "D"):
        assert not np.any(g[name]), name


def test_round_bf16_ties_and_torch():
    # spacing at 1 is 2^-7: 1 + 2^-8 is a tie (to the even 1.0); 1 + 3*2^-8
    # ties between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -20])
    np.testing.assert_array_equal(L.round_bf16(vals), [1.0, 1.0 + 2.0 ** -6, -1.0, 1.0 + 2.0 ** -7])
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(6).standard_normal(10000) * 10.0 ** np.random.default_rng(7).uniform(-6, 6, 10000)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(L.round_bf16(x.astype(np.float32)), ref)
    np.testing.assert_array_equal(L.round_act(L.round_act(x, "bf16"), "bf16"), L.round_act(x, "bf16"))


def test_rounded_layer_stores_representable_values():
    rng = np.random.default_rng(8)
    p = _params(rng)
    resid = rng.standard_normal((2, 6, 5))
    _, saved = L.layer_forward(resid, p, act="bf16")
    for name in L.ROUNDED_FWD:
        if name in saved:
            v = saved[name]
            assert np.array_equal(L.round_act(v, "bf16"), v), name
