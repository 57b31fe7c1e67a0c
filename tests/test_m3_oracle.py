"""Pins of the Mamba-3 SISO core oracle (oracle/mamba3.py) to things other
than itself: an O(T^2) closed form written from the update rule, a library
IIR filter for the one-state case, finite differences for every gradient,
and invariants of the rotation, the decay clamp and the head groups.

The definition the oracle follows is a set of readings of the mamba-rs 0.4.0
``src/mamba3_siso/gpu/backward_mixed.rs`` page (listed in the oracle's
docstring); these tests pin the oracle to those readings, not the readings
to the page, which does not state them.
"""
import numpy as np
import pytest
import scipy.signal

from oracle import mamba3 as m3

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def draw(B=1, T=6, H=2, P=2, N=4, G=1, NA=2, seed=0, scale_dt=1.0):
    r = np.random.default_rng(seed)
    return dict(x=r.normal(size=(B, T, H * P)), b_in=r.normal(size=(B, T, G, N)), c_in=r.normal(size=(B, T, G, N)),
                dd_dt_raw=r.normal(size=(B, T, H)) * scale_dt, dd_a_raw=r.normal(size=(B, T, H)),
                trap_raw=r.normal(size=(B, T, H)), angles_raw=r.normal(size=(B, T, NA)),
                b_bias=r.normal(size=(H, N)) * 0.3, c_bias=r.normal(size=(H, N)) * 0.3,
                dt_bias=r.normal(size=H) * 0.3, D=r.normal(size=H), a_floor=0.3, heads=H, headdim=P)


def fwd(inp):
    return m3.forward(**inp)


def closed_form(inp):
    """y_t = sum_{s<=t} w(t, s) (Q_t . K_s) V_s + D V_t with
    w(t, t) = lam_t dt_t and, for s < t,
    w(t, s) = (lam_s dt_s + (1 - lam_{s+1}) dt_{s+1}) prod_{r=s+1..t} exp(dt_r A_r):
    the input of step s enters with weight lam_s dt_s at step s and with
    (1 - lam_{s+1}) dt_{s+1} alpha_{s+1} at step s+1, then decays.  Q and K
    are turned by explicit 2x2 rotation matrices."""
    x, H, P = inp["x"], inp["heads"], inp["headdim"]
    B, T, _ = x.shape
    G, N = inp["b_in"].shape[2:]
    NA = inp["angles_raw"].shape[2]
    sp = lambda v: np.log1p(np.exp(v))
    y = np.zeros((B, T, H, P))
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            dt = sp(inp["dd_dt_raw"][b, :, h] + inp["dt_bias"][h])
            A = -np.maximum(sp(inp["dd_a_raw"][b, :, h]), inp["a_floor"])
            lam = 1.0 / (1.0 + np.exp(-inp["trap_raw"][b, :, h]))
            la = dt * A                                   # log alpha
            theta = np.cumsum(dt[:, None] * inp["angles_raw"][b], axis=0)

            def turn(v, t):
                R = np.eye(N)
                for a in range(NA):
                    c, s = np.cos(theta[t, a]), np.sin(theta[t, a])
                    R[a, a], R[a, a + NA], R[a + NA, a], R[a + NA, a + NA] = c, -s, s, c
                return R @ v

            K = [turn(inp["b_in"][b, t, g] + inp["b_bias"][h], t) for t in range(T)]
            Q = [turn(inp["c_in"][b, t, g] + inp["c_bias"][h], t) for t in range(T)]
            V = inp["x"][b, :, h * P:(h + 1) * P]
            for t in range(T):
                acc = inp["D"][h] * V[t]
                for s in range(t + 1):
                    if s == t:
                        w = lam[t] * dt[t]
                    else:
                        w = (lam[s] * dt[s] + (1 - lam[s + 1]) * dt[s + 1]) * np.exp(la[s + 1:t + 1].sum())
                    acc = acc + w * (Q[t] @ K[s]) * V[s]
                y[b, t, h] = acc
    return y.reshape(B, T, H * P)


@pytest.mark.parametrize("NA,G,H", [(2, 1, 2), (1, 1, 2), (0, 2, 2), (3, 2, 4)])
def test_closed_form(NA, G, H):
    inp = draw(B=2, T=9, H=H, G=G, N=6, NA=NA, P=3, seed=NA + 10 * G)
    np.testing.assert_allclose(fwd(inp), closed_form(inp), rtol=1e-11, atol=1e-11)


def test_one_state_is_a_two_tap_iir_filter():
    """d_state 1 and constant dt, A, lam, B, C: the trapezoidal update is the
    IIR filter with numerator [lam dt, (1 - lam) dt alpha] and denominator
    [1, -alpha], scaled by B C, plus D x (scipy.signal.lfilter)."""
    T = 40
    r = np.random.default_rng(3)
    x = r.normal(size=(1, T, 1))
    c = dict(dd_dt_raw=0.4, dd_a_raw=-0.2, trap_raw=0.7, dt_bias=-0.1)
    inp = dict(x=x, b_in=np.full((1, T, 1, 1), 0.8), c_in=np.full((1, T, 1, 1), -1.3),
               dd_dt_raw=np.full((1, T, 1), c["dd_dt_raw"]), dd_a_raw=np.full((1, T, 1), c["dd_a_raw"]),
               trap_raw=np.full((1, T, 1), c["trap_raw"]), angles_raw=np.zeros((1, T, 0)),
               b_bias=np.zeros((1, 1)), c_bias=np.zeros((1, 1)), dt_bias=np.array([c["dt_bias"]]),
               D=np.array([0.6]), a_floor=1e-4, heads=1, headdim=1)
    dt = np.log1p(np.exp(c["dd_dt_raw"] + c["dt_bias"]))
    A = -max(np.log1p(np.exp(c["dd_a_raw"])), 1e-4)
    lam = 1 / (1 + np.exp(-c["trap_raw"]))
    al = np.exp(dt * A)
    ref = scipy.signal.lfilter([lam * dt, (1 - lam) * dt * al], [1.0, -al], x[0, :, 0]) * 0.8 * -1.3 + 0.6 * x[0, :, 0]
    np.testing.assert_allclose(fwd(inp)[0, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_common_angle_offset_leaves_output_unchanged():
    """Q_t and K_s are turned by theta_t and theta_s, so only differences of
    angles reach y: an angle added at step 0 (which shifts every theta_t of a
    head by the same amount) changes nothing, one added at a later step does."""
    inp = draw(B=1, T=8, H=2, N=6, NA=3, P=2, seed=5)
    y0 = fwd(inp)
    a = dict(inp)
    a["angles_raw"] = inp["angles_raw"].copy()
    a["angles_raw"][:, 0] += 1.7
    np.testing.assert_allclose(fwd(a), y0, rtol=1e-11, atol=1e-11)
    a["angles_raw"][:, 4] += 1.7
    assert np.abs(fwd(a) - y0).max() > 1e-3


def test_decay_clamp_memoryless():
    """a_floor = 1e7 makes every A_t = -1e7, so alpha_t = 0: the state keeps
    only the current step, y_t = lam_t dt_t (Qb_t . Kb_t) V_t + D V_t, with no
    rotation left (both vectors turn by theta_t)."""
    inp = draw(B=1, T=7, H=2, N=6, NA=3, P=3, seed=7)
    inp["a_floor"] = 1e7
    y = fwd(inp).reshape(1, 7, 2, 3)
    sp = lambda v: np.log1p(np.exp(v))
    for h in range(2):
        dt = sp(inp["dd_dt_raw"][0, :, h] + inp["dt_bias"][h])
        lam = 1 / (1 + np.exp(-inp["trap_raw"][0, :, h]))
        kb = inp["b_in"][0, :, 0] + inp["b_bias"][h]
        qb = inp["c_in"][0, :, 0] + inp["c_bias"][h]
        V = inp["x"][0, :, h * 3:(h + 1) * 3]
        ref = (lam * dt * (qb * kb).sum(-1))[:, None] * V + inp["D"][h] * V
        np.testing.assert_allclose(y[0, :, h], ref, rtol=1e-12, atol=1e-12)


def test_heads_of_a_group_share_b_and_c():
    """Four heads in two groups equal four one-head runs on their group's B/C."""
    inp = draw(B=2, T=6, H=4, G=2, N=4, NA=2, P=2, seed=9)
    y = fwd(inp).reshape(2, 6, 4, 2)
    for h in range(4):
        g = h // 2
        one = dict(inp, x=inp["x"][:, :, 2 * h:2 * h + 2], b_in=inp["b_in"][:, :, g:g + 1],
                   c_in=inp["c_in"][:, :, g:g + 1], dd_dt_raw=inp["dd_dt_raw"][:, :, h:h + 1],
                   dd_a_raw=inp["dd_a_raw"][:, :, h:h + 1], trap_raw=inp["trap_raw"][:, :, h:h + 1],
                   b_bias=inp["b_bias"][h:h + 1], c_bias=inp["c_bias"][h:h + 1], dt_bias=inp["dt_bias"][h:h + 1],
                   D=inp["D"][h:h + 1], heads=1)
        np.testing.assert_allclose(fwd(one).reshape(2, 6, 2), y[:, :, h], rtol=1e-12, atol=1e-12)


def test_adjoint_identity_in_x():
    """With everything but x fixed, y is linear in x, so <dy, y(x)> = <d_x, x>."""
    inp = draw(B=2, T=7, H=2, N=4, NA=2, P=3, seed=11)
    dy = np.random.default_rng(12).normal(size=inp["x"].shape)
    g = m3.backward(dy, **inp)
    assert abs((dy * fwd(inp)).sum() - (g["x"] * inp["x"]).sum()) < 1e-10 * (1 + abs((dy * fwd(inp)).sum()))


NAMES = ["x", "b_in", "c_in", "dd_dt_raw", "dd_a_raw", "trap_raw", "angles_raw", "b_bias", "c_bias", "dt_bias", "D"]


@pytest.mark.parametrize("NA,G,H", [(2, 1, 2), (1, 2, 2), (0, 1, 1)])
def test_finite_differences_every_input(NA, G, H):
    """Central differences of sum(dy * y) for every element of every input,
    against the oracle's adjoint.  a_floor 0.3 clamps some steps (their
    dd_a_raw gradient is 0); no drawn value sits within the step of the kink."""
    inp = draw(B=1, T=6, H=H, G=G, N=4, NA=NA, P=2, seed=20 + NA)
    dy = np.random.default_rng(21).normal(size=inp["x"].shape)
    g = m3.backward(dy, **inp)
    sp = np.log1p(np.exp(inp["dd_a_raw"]))
    assert np.all(np.abs(sp - inp["a_floor"]) > 1e-4)
    assert np.any(sp < inp["a_floor"]) and np.any(sp > inp["a_floor"])
    for name in NAMES:
        base = np.asarray(inp[name], dtype=np.float64)
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            vals = []
            for sgn in (1, -1):
                pert = base.copy()
                pert[idx] += sgn * eps
                vals.append((dy * fwd(dict(inp, **{name: pert}))).sum())
            num[idx] = (vals[0] - vals[1]) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=2e-6, atol=2e-7, err_msg=name)
