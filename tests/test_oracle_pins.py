"""Pins for the CPU oracle: every check here compares the oracle with something
other than itself (closed forms, hand-worked fixtures, an independent
materialised-matrix form, a scipy filter, finite differences of its own
forward, and exact identities).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _xdbl(Bm, Cm, R=0, rng=None):
    b, t, ds = Bm.shape
    x = np.zeros((b, t, R + 2 * ds))
    if R:
        x[..., :R] = rng.standard_normal((b, t, R)) if rng is not None else 7.0
    x[..., R:R + ds] = Bm
    x[..., R + ds:] = Cm
    return x


def _inv_softplus(d):
    """delta_raw that gives softplus(delta_raw) = d exactly (up to rounding)."""
    return np.log(np.expm1(d))


# ---------------------------------------------------------------------------
# hand-worked fixtures


def test_worked_example_fixture(oracle_lib):
    g = _load("worked_example_T2.json")
    inp, exp = g["inputs"], g["expected"]
    u = np.array(inp["u"]).reshape(1, 2, 1)
    draw = np.array(inp["delta_raw"]).reshape(1, 2, 1)
    a_log = np.array(inp["a_log"]).reshape(1, 1)
    xdbl = _xdbl(np.array(inp["B"]).reshape(1, 2, 1), np.array(inp["C"]).reshape(1, 2, 1))
    D = np.array(inp["D"])
    dout = np.array(inp["dout"]).reshape(1, 2, 1)
    f = oracle_lib.forward(u, draw, a_log, xdbl, D=D, chunk=1)
    b = oracle_lib.backward(u, draw, a_log, xdbl, dout, D=D)
    tol = dict(rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(f["y"].ravel(), exp["y"], **tol)
    np.testing.assert_allclose(f["out"].ravel(), exp["y"], **tol)
    np.testing.assert_allclose(f["h_last"].ravel(), exp["h_last"], **tol)
    np.testing.assert_allclose(b["d_x"].ravel(), exp["d_u"], **tol)
    np.testing.assert_allclose(b["d_delta"].ravel(), exp["d_delta"], **tol)
    np.testing.assert_allclose(b["d_delta_raw"].ravel(), exp["d_delta_raw"], **tol)
    np.testing.assert_allclose(b["d_xdbl"][0, :, 0], exp["d_B"], **tol)
    np.testing.assert_allclose(b["d_xdbl"][0, :, 1], exp["d_C"], **tol)
    np.testing.assert_allclose(b["d_a_log"].ravel(), exp["d_a_log"], **tol)
    np.testing.assert_allclose(b["d_D"].ravel(), exp["d_D"], **tol)


def test_conv_fixture(oracle_lib):
    g = _load("conv_example_K2.json")
    inp, exp = g["inputs"], g["expected"]
    x = np.array(inp["x"]).reshape(1, 2, 1)
    w = np.array(inp["conv_w"]).reshape(1, 2)
    cb = np.array(inp["conv_b"])
    cs0 = np.array(inp["conv_state0"]).reshape(1, 1, 2)
    # Ds = 1 scan with delta = 0 so that out = D * u exposes u directly
    draw = np.full((1, 2, 1), -1000.0)
    xdbl = _xdbl(np.zeros((1, 2, 1)), np.zeros((1, 2, 1)))
    f = oracle_lib.forward(x, draw, np.zeros((1, 1)), xdbl, D=np.ones(1), conv_w=w, conv_b=cb,
                           conv_state0=cs0)
    np.testing.assert_allclose(f["u"].ravel(), exp["u"], rtol=1e-14)
    np.testing.assert_allclose(f["out"].ravel(), exp["u"], rtol=1e-14)
    np.testing.assert_allclose(f["conv_state_last"].ravel(), exp["conv_state_last"], rtol=0)


# ---------------------------------------------------------------------------
# P-1: constant delta, B and u give a geometric series


def test_geometric_closed_form(oracle_lib):
    rng = np.random.default_rng(1)
    Bt, T, Di, Ds = 2, 40, 3, 5
    delta = 0.37
    u_c = rng.standard_normal((Bt, 1, Di))
    B_c = rng.standard_normal((Bt, 1, Ds))
    u = np.broadcast_to(u_c, (Bt, T, Di)).copy()
    Bm = np.broadcast_to(B_c, (Bt, T, Ds)).copy()
    Cm = rng.standard_normal((Bt, T, Ds))
    a_log = rng.uniform(-1.0, 1.0, (Di, Ds))
    h0 = rng.standard_normal((Bt, Di, Ds))
    draw = np.full((Bt, T, Di), _inv_softplus(delta))
    f = oracle_lib.forward(u, draw, a_log, _xdbl(Bm, Cm), h0=h0, chunk=1)
    A = -np.exp(a_log)                                        # [Di, Ds]
    a = np.exp(delta * A)[None]                               # [1, Di, Ds]
    bb = delta * u_c[:, 0, :, None] * B_c[:, 0, None, :]      # [Bt, Di, Ds]
    for t in range(T):
        k = t + 1
        h_t = a ** k * h0 + bb * (1 - a ** k) / (1 - a)       # h after k steps
        if t + 1 < T:
            np.testing.assert_allclose(f["ckpt"][:, t + 1].transpose(0, 2, 1), h_t, rtol=1e-12, atol=1e-13)
        y_t = np.einsum("bn,bin->bi", Cm[:, t], h_t)
        np.testing.assert_allclose(f["y"][:, t], y_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f["h_last"], h_t, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f["ckpt"][:, 0].transpose(0, 2, 1), h0, rtol=0, atol=0)


# ---------------------------------------------------------------------------
# P-2: delta = 0 leaves the state unchanged


def test_delta_zero_keeps_state(oracle_lib):
    rng = np.random.default_rng(2)
    Bt, T, Di, Ds = 2, 17, 4, 3
    u = rng.standard_normal((Bt, T, Di))
    Bm, Cm = rng.standard_normal((Bt, T, Ds)), rng.standard_normal((Bt, T, Ds))
    h0 = rng.standard_normal((Bt, Di, Ds))
    D = rng.standard_normal(Di)
    draw = np.full((Bt, T, Di), -1000.0)    # softplus(-1000) is exactly 0 in double
    a_log = rng.standard_normal((Di, Ds))
    f = oracle_lib.forward(u, draw, a_log, _xdbl(Bm, Cm), D=D, h0=h0, chunk=1)
    for t in range(1, T):
        np.testing.assert_array_equal(f["ckpt"][:, t].transpose(0, 2, 1), h0)
    np.testing.assert_array_equal(f["h_last"], h0)
    y_exp = np.einsum("btn,bin->bti", Cm, h0) + D * u
    np.testing.assert_allclose(f["y"], y_exp, rtol=1e-14, atol=1e-14)
    dout = rng.standard_normal((Bt, T, Di))
    g = oracle_lib.backward(u, draw, a_log, _xdbl(Bm, Cm), dout, D=D, h0=h0)
    np.testing.assert_array_equal(g["d_delta_raw"], 0.0)
    np.testing.assert_allclose(g["d_x"], D * dout, rtol=1e-14)           # no path through the state
    np.testing.assert_allclose(g["d_xdbl"][..., Ds:], np.einsum("bti,bin->btn", dout, h0), rtol=1e-13)
    np.testing.assert_array_equal(g["d_xdbl"][..., :Ds], 0.0)
    np.testing.assert_array_equal(g["d_a_log"], 0.0)


# ---------------------------------------------------------------------------
# P-3: A so negative that exp(delta A) underflows to 0: a memoryless map


def test_memoryless_limit(oracle_lib):
    rng = np.random.default_rng(3)
    Bt, T, Di, Ds = 1, 12, 3, 4
    u = rng.standard_normal((Bt, T, Di))
    draw = rng.uniform(0.0, 2.0, (Bt, T, Di))     # delta in [0.69, 2.13]
    Bm, Cm = rng.standard_normal((Bt, T, Ds)), rng.standard_normal((Bt, T, Ds))
    a_log = np.full((Di, Ds), math.log(1e4))     # A = -1e4: exp(-6.9e3) == 0.0
    D = np.full(Di, 0.5)
    f = oracle_lib.forward(u, draw, a_log, _xdbl(Bm, Cm), D=D)
    delta = np.log1p(np.exp(draw))
    y_exp = delta * u * np.einsum("btn,btn->bt", Bm, Cm)[..., None] + D * u
    np.testing.assert_allclose(f["y"], y_exp, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# P-4: independent materialised-matrix form on tiny T


def _materialised(u, delta, a_log, Bm, Cm, D, h0):
    """y_t = sum_{k<=t} sum_n C_t B_k delta_k exp(A sum_{j=k+1..t} delta_j) u_k
             + sum_n C_t exp(A sum_{j<=t} delta_j) h0 + D u_t"""
    Bt, T, Di = u.shape
    A = -np.exp(a_log)
    y = np.zeros((Bt, T, Di))
    S = np.cumsum(delta, axis=1)                   # S_t = sum_{j<=t} delta_j
    for b in range(Bt):
        for t in range(T):
            for k in range(t + 1):
                decay = np.exp(A * (S[b, t] - S[b, k])[:, None])           # [Di, Ds]
                y[b, t] += (decay * Bm[b, k][None] * Cm[b, t][None]).sum(1) * delta[b, k] * u[b, k]
            y[b, t] += (np.exp(A * S[b, t][:, None]) * h0[b] * Cm[b, t][None]).sum(1)
            y[b, t] += D * u[b, t]
    return y


@pytest.mark.parametrize("seed", [4, 5])
def test_materialised_matrix_form(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    Bt, T, Di, Ds, R = 2, 19, 3, 4, 2
    u = rng.standard_normal((Bt, T, Di))
    draw = rng.standard_normal((Bt, T, Di))
    Bm, Cm = rng.standard_normal((Bt, T, Ds)), rng.standard_normal((Bt, T, Ds))
    a_log = rng.uniform(-1.5, 1.0, (Di, Ds))
    D = rng.standard_normal(Di)
    h0 = rng.standard_normal((Bt, Di, Ds))
    z = rng.standard_normal((Bt, T, Di))
    f = oracle_lib.forward(u, draw, a_log, _xdbl(Bm, Cm, R, rng), D=D, h0=h0, z=z)
    delta = np.log1p(np.exp(draw))
    y = _materialised(u, delta, a_log, Bm, Cm, D, h0)
    np.testing.assert_allclose(f["y"], y, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f["out"], y * z / (1 + np.exp(-z)), rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# P-5: library special cases (first-order IIR filter; numpy convolution)


def test_single_state_is_iir_filter(oracle_lib):
    rng = np.random.default_rng(6)
    T, Di = 200, 3
    delta = 0.05
    u = rng.standard_normal((1, T, Di))
    Bc, Cc = 1.3, -0.7
    a_log = np.array([[0.2], [-0.4], [0.9]])
    Bm = np.full((1, T, 1), Bc)
    Cm = np.full((1, T, 1), Cc)
    f = oracle_lib.forward(u, np.full((1, T, Di), _inv_softplus(delta)), a_log, _xdbl(Bm, Cm))
    for i in range(Di):
        a = math.exp(-delta * math.exp(a_log[i, 0]))
        h = scipy.signal.lfilter([delta * Bc], [1.0, -a], u[0, :, i])
        np.testing.assert_allclose(f["y"][0, :, i], Cc * h, rtol=1e-11, atol=1e-12)


def test_conv_matches_numpy_convolve(oracle_lib):
    rng = np.random.default_rng(7)
    T, Di, K = 30, 3, 4
    x = rng.standard_normal((1, T, Di))
    w = rng.standard_normal((Di, K))
    cb = rng.standard_normal(Di)
    cs0 = rng.standard_normal((1, Di, K))
    draw = np.full((1, T, Di), -1000.0)       # delta = 0: out = D * u = u
    xdbl = _xdbl(np.zeros((1, T, 1)), np.zeros((1, T, 1)))
    f = oracle_lib.forward(x, draw, np.zeros((Di, 1)), xdbl, D=np.ones(Di), conv_w=w, conv_b=cb,
                           conv_state0=cs0)
    for i in range(Di):
        padded = np.concatenate([cs0[0, i, 1:], x[0, :, i]])     # the last K-1 state entries
        p = np.convolve(padded, w[i, ::-1], mode="valid") + cb[i]
        np.testing.assert_allclose(f["u"][0, :, i], p / (1 + np.exp(-p)), rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(f["conv_state_last"][0, i], x[0, T - K:, i])


# ---------------------------------------------------------------------------
# P-6: central finite differences of the oracle's own forward, every input


def _fd_case(rng, fused):
    Bt, T, Di, Ds, R, K = 2, 9, 3, 3, 2, 3
    c = dict(
        x=rng.standard_normal((Bt, T, Di)),
        delta_raw=rng.standard_normal((Bt, T, Di)) - 0.5,
        a_log=rng.uniform(-1.0, 0.7, (Di, Ds)),
        xdbl=_xdbl(rng.standard_normal((Bt, T, Ds)), rng.standard_normal((Bt, T, Ds)), R, rng),
        D=rng.standard_normal(Di),
        z=rng.standard_normal((Bt, T, Di)),
        h0=rng.standard_normal((Bt, Di, Ds)),
    )
    if fused:
        c.update(conv_w=rng.standard_normal((Di, K)) * 0.5, conv_b=rng.standard_normal(Di) * 0.5,
                 conv_state0=rng.standard_normal((Bt, Di, K)))
    return c


@pytest.mark.parametrize("fused", [False, True])
def test_finite_differences_every_input(oracle_lib, fused):
    rng = np.random.default_rng(8 + fused)
    c = _fd_case(rng, fused)
    Bt, T, Di = c["x"].shape
    dout = rng.standard_normal((Bt, T, Di))
    d_u_extra = rng.standard_normal((Bt, T, Di)) if fused else None

    def loss(cc):
        f = oracle_lib.forward(**cc)
        val = np.sum(dout * f["out"])
        if d_u_extra is not None:
            val += np.sum(d_u_extra * f["u"])
        return val

    g = oracle_lib.backward(dout=dout, d_u_extra=d_u_extra, **c)
    wanted = {"x": "d_x", "delta_raw": "d_delta_raw", "z": "d_z", "a_log": "d_a_log", "D": "d_D",
              "xdbl": "d_xdbl"}
    if fused:
        wanted.update(conv_w="d_conv_w", conv_b="d_conv_b")
    R = c["xdbl"].shape[2] - 2 * c["a_log"].shape[1]
    for name, gname in wanted.items():
        base = c[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            if name == "xdbl" and idx[-1] < R:
                continue       # dt columns are not read by the core
            eps = 1e-6 * max(1.0, abs(base[idx]))
            cp, cm = dict(c), dict(c)
            cp[name], cm[name] = base.copy(), base.copy()
            cp[name][idx] += eps
            cm[name][idx] -= eps
            num[idx] = (loss(cp) - loss(cm)) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        err = np.abs(g[gname] - num).max() / scale
        assert err < 1e-6, (name, err)
    # the dt columns of d_xdbl are never written
    np.testing.assert_array_equal(g["d_xdbl"][..., :R], 0.0)


# ---------------------------------------------------------------------------
# P-7 adjoint identity, P-8 parameter grads, P-10 linearity/permutation


def test_adjoint_identity(oracle_lib):
    rng = np.random.default_rng(10)
    Bt, T, Di, Ds = 2, 33, 5, 4
    u = rng.standard_normal((Bt, T, Di))
    draw = rng.standard_normal((Bt, T, Di))
    a_log = rng.standard_normal((Di, Ds)) * 0.5
    xdbl = _xdbl(rng.standard_normal((Bt, T, Ds)), rng.standard_normal((Bt, T, Ds)))
    D = rng.standard_normal(Di)
    dy = rng.standard_normal((Bt, T, Di))
    y = oracle_lib.forward(u, draw, a_log, xdbl, D=D)["out"]        # linear in u (h0 = 0, no gate)
    du = oracle_lib.backward(u, draw, a_log, xdbl, dy, D=D)["d_x"]
    lhs, rhs = np.sum(dy * y), np.sum(du * u)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_param_grads_closed_forms(oracle_lib):
    rng = np.random.default_rng(11)
    c = _fd_case(rng, fused=True)
    Bt, T, Di = c["x"].shape
    dout = rng.standard_normal((Bt, T, Di))
    f = oracle_lib.forward(**c)
    g = oracle_lib.backward(dout=dout, **c)
    z = c["z"]
    silu = z / (1 + np.exp(-z))
    dy = dout * silu
    np.testing.assert_allclose(g["d_D"], np.sum(dy * f["u"], axis=(0, 1)), rtol=1e-12)
    # d_z: out = y silu(z); silu'(z) = silu(z) + sigmoid(z)(1 - silu(z))
    sig = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(g["d_z"], dout * f["y"] * (silu + sig * (1 - silu)), rtol=1e-12, atol=1e-14)
    # d_a_log = A * d_A, with d_A from the same loss differentiated w.r.t. A by FD
    A = -np.exp(c["a_log"])
    i, n = 1, 2
    eps = 1e-6
    def loss_A(Aval):
        cc = dict(c)
        al = c["a_log"].copy()
        al[i, n] = np.log(-Aval)
        cc["a_log"] = al
        return np.sum(dout * oracle_lib.forward(**cc)["out"])
    dA = (loss_A(A[i, n] + eps) - loss_A(A[i, n] - eps)) / (2 * eps)
    assert abs(g["d_a_log"][i, n] - A[i, n] * dA) <= 1e-6 * max(1.0, abs(A[i, n] * dA))


def test_backward_linear_in_dout_and_channel_permutation(oracle_lib):
    rng = np.random.default_rng(12)
    c = _fd_case(rng, fused=True)
    Bt, T, Di = c["x"].shape
    d1, d2 = rng.standard_normal((Bt, T, Di)), rng.standard_normal((Bt, T, Di))
    g1 = oracle_lib.backward(dout=d1, **c)
    g2 = oracle_lib.backward(dout=d2, **c)
    g12 = oracle_lib.backward(dout=2.0 * d1 - 3.0 * d2, **c)
    for k in g1:
        np.testing.assert_allclose(g12[k], 2.0 * g1[k] - 3.0 * g2[k], rtol=1e-10, atol=1e-10)
    perm = rng.permutation(Di)
    cp = dict(c)
    for k in ("x", "delta_raw", "z"):
        cp[k] = c[k][..., perm]
    cp["a_log"], cp["D"] = c["a_log"][perm], c["D"][perm]
    cp["conv_w"], cp["conv_b"] = c["conv_w"][perm], c["conv_b"][perm]
    cp["h0"], cp["conv_state0"] = c["h0"][:, perm], c["conv_state0"][:, perm]
    fp = oracle_lib.forward(**cp)
    f = oracle_lib.forward(**c)
    np.testing.assert_allclose(fp["out"], f["out"][..., perm], rtol=1e-13, atol=1e-14)
    gp = oracle_lib.backward(dout=d1[..., perm], **cp)
    np.testing.assert_allclose(gp["d_x"], g1["d_x"][..., perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gp["d_xdbl"], g1["d_xdbl"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gp["d_a_log"], g1["d_a_log"][perm], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P-9: truncated-BPTT split: fwd(0..T) == fwd(0..T1) then fwd(T1..T)


@pytest.mark.parametrize("T1", [1, 2, 7])
def test_state_carry_split(oracle_lib, T1):
    rng = np.random.default_rng(13)
    c = _fd_case(rng, fused=True)
    full = oracle_lib.forward(**c)
    a = dict(c)
    for k in ("x", "delta_raw", "z"):
        a[k] = c[k][:, :T1]
    a["xdbl"] = c["xdbl"][:, :T1]
    fa = oracle_lib.forward(**a)
    b = dict(c)
    for k in ("x", "delta_raw", "z"):
        b[k] = c[k][:, T1:]
    b["xdbl"] = c["xdbl"][:, T1:]
    b["h0"], b["conv_state0"] = fa["h_last"], fa["conv_state_last"]
    fb = oracle_lib.forward(**b)
    np.testing.assert_allclose(np.concatenate([fa["out"], fb["out"]], axis=1), full["out"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fb["h_last"], full["h_last"], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(fb["conv_state_last"], full["conv_state_last"])


def test_checkpoints_are_sampled_states(oracle_lib):
    """ckpt at interval L equals every L-th entry of the interval-1 history."""
    rng = np.random.default_rng(14)
    c = _fd_case(rng, fused=False)
    T = c["x"].shape[1]
    h1 = oracle_lib.forward(chunk=1, **c)["ckpt"]
    for L in (2, 4, 5, 9, 64):
        hl = oracle_lib.forward(chunk=L, **c)["ckpt"]
        assert hl.shape[1] == -(-T // L)
        np.testing.assert_array_equal(hl, h1[:, ::L])


def test_workload_generator_is_seeded_and_rounded():
    w = workloads.CONFIGS["fused_small_bf16"].with_(batch=2, seqlen=8, d_inner=16)
    a = workloads.make_inputs(w, seed=3)
    b = workloads.make_inputs(w, seed=3)
    for k in a:
        if a[k] is not None:
            np.testing.assert_array_equal(a[k], b[k])
    bits = a["x"].view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)            # bf16-representable
    np.testing.assert_array_equal(workloads.round_to("f16", a["x"]), a["x"].astype(np.float16).astype(np.float32))
    np.testing.assert_allclose(a["a_log"][0], np.log(np.arange(1, 17)), rtol=1e-7)


@pytest.mark.parametrize("threads", [1, 3, 7])
def test_channel_ranges_do_not_change_results(oracle_lib, threads):
    """Channels are independent except in d_xdbl (a sum over channels): any
    split of the channels over threads gives the same forward bits and the
    same backward bits, and d_xdbl up to the order of its channel sum."""
    w = workloads.Workload("split_ch", 2, 37, 13, 4, 3, 3, "f32", True)
    inp = workloads.make_inputs(w, 21, h0=True, conv_state0=True, d_u_extra=True)
    kw = dict(x=inp["x"], delta_raw=inp["delta_raw"], a_log=inp["a_log"], xdbl=inp["xdbl"], D=inp["D"],
              z=inp["z"], h0=inp["h0"], conv_w=inp["conv_w"], conv_b=inp["conv_b"],
              conv_state0=inp["conv_state0"])
    f1 = oracle_lib.forward(chunk=16, threads=1, **kw)
    fn = oracle_lib.forward(chunk=16, threads=threads, **kw)
    for k in f1:
        assert np.array_equal(f1[k], fn[k]), k
    g1 = oracle_lib.backward(dout=inp["dout"], d_u_extra=inp["d_u_extra"], threads=1, **kw)
    gn = oracle_lib.backward(dout=inp["dout"], d_u_extra=inp["d_u_extra"], threads=threads, **kw)
    for k in g1:
        if k == "d_xdbl":
            np.testing.assert_allclose(gn[k], g1[k], rtol=1e-13, atol=1e-13)
            assert np.all(gn[k][..., :w.dt_rank] == 0.0)
        else:
            assert np.array_equal(g1[k], gn[k]), k


def test_single_precision_build_tracks_double(oracle_lib):
    """The float build (host timing only) computes the same definition: its
    results stay within single-precision rounding of the double build."""
    w = workloads.Workload("f32_build", 2, 50, 24, 8, 2, 4, "f32", True)
    inp = workloads.make_inputs(w, 4)
    kw = dict(x=inp["x"], delta_raw=inp["delta_raw"], a_log=inp["a_log"], xdbl=inp["xdbl"], D=inp["D"],
              z=inp["z"], conv_w=inp["conv_w"], conv_b=inp["conv_b"])
    f64 = oracle_lib.forward(chunk=16, **kw)
    f32 = oracle_lib.forward(chunk=16, precision="f32", **kw)
    g64 = oracle_lib.backward(dout=inp["dout"], **kw)
    g32 = oracle_lib.backward(dout=inp["dout"], precision="f32", **kw)
    assert f32["out"].dtype == np.float32 and g32["d_x"].dtype == np.float32
    for a, b in [(f32[k], f64[k]) for k in f64] + [(g32[k], g64[k]) for k in g64]:
        scale = max(1.0, np.abs(b).max())
        assert np.abs(a.astype(np.float64) - b).max() / scale < 1e-4
