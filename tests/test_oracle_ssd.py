"""Pins of the SSD oracle against facts outside it (CPU only).

Each test pins the oracle to something that is not the oracle: the dual
(quadratic) form derived independently in tests/dual_form.py, central finite
differences of the oracle's own forward, closed forms (A -> 0, T = 1), a
hand-worked example (tests/golden/hand_worked_t2.json), skip paths, group
replication and linearity.  A dropped term, a wrong sign or index or a
transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import dual_form
from ssd_inputs import CONFIGS, P1TEST, make_inputs, make_p1test_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, b=2, T=9, H=4, G=2, P=3, N=5, h0=True, a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, G, N))
    C = rng.standard_normal((b, T, G, N))
    dt = np.logaddexp(0, rng.standard_normal((b, T, H)) - 1.0)
    A_log = rng.uniform(0, np.log(4.0), size=H) + np.log(a_scale)
    D = rng.standard_normal(H)
    hz = rng.standard_normal((b, H, P, N)) if h0 else None
    dy = rng.standard_normal((b, T, H, P))
    return dict(x=x, dt=dt, A_log=A_log, B=B, C=C, D=D, h0=hz, dy=dy)


def fwd(p, **kw):
    return oracle.ssd_fwd(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["h0"], **kw)


def bwd(p, **kw):
    return oracle.ssd_bwd(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["dy"], p["h0"], **kw)


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("seed,h0", [(1, True), (2, False)])
def test_forward_matches_dual_form(seed, h0):
    p = rand_problem(seed, h0=h0)
    y_dual = dual_form.forward(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["h0"])
    assert rel(fwd(p)["y"], y_dual) < 1e-13


def test_chunk_states_and_final_match_unrolled_states():
    p = rand_problem(3, T=12)
    out = fwd(p, chunk=4)
    hs = dual_form.states(p["x"], p["dt"], p["A_log"], p["B"], p["h0"])
    cs = out["chunk_states"]
    assert cs.shape == (2, 3, 4, 3, 5)
    assert np.array_equal(cs[:, 0], p["h0"])  # the state entering chunk 0 is h0
    for c in (1, 2):
        assert rel(cs[:, c], hs[:, 4 * c - 1]) < 1e-13
    assert rel(out["final"], hs[:, -1]) < 1e-13


def test_a_to_zero_closed_form():
    # A_log = -60: exp(dt*A) == 1 in f64, so h_t is a plain cumulative sum and
    # y_t = sum_{s<=t} dt_s (B_s . C_t) x_s + C_t . h0 + D x_t.
    p = rand_problem(4)
    p["A_log"] = np.full(4, -60.0)
    b, T, H, P = p["x"].shape
    G = p["B"].shape[2]
    hpg = H // G
    y = np.zeros_like(p["x"])
    for h in range(H):
        g = h // hpg
        st = p["h0"][:, h].copy()
        for t in range(T):
            st = st + p["dt"][:, t, h, None, None] * p["x"][:, t, h, :, None] * p["B"][:, t, g, None, :]
            y[:, t, h] = np.einsum("bpn,bn->bp", st, p["C"][:, t, g]) + p["D"][h] * p["x"][:, t, h]
    # same sum written as cumsum over time
    drive = p["dt"][..., None, None] * p["x"][..., None] * np.repeat(p["B"], hpg, axis=2)[:, :, :, None, :]
    st2 = np.cumsum(drive, axis=1) + p["h0"][:, None]
    y2 = np.einsum("bthpn,bthn->bthp", st2, np.repeat(p["C"], hpg, axis=2)) + p["D"][None, None, :, None] * p["x"]
    assert rel(y, y2) < 1e-13
    assert rel(fwd(p)["y"], y2) < 1e-13
    g = bwd(p)
    assert np.max(np.abs(g["dA_log"])) < 1e-20
    # dh0 = sum_t dy_t (outer) C_t when there is no decay
    dh0 = np.einsum("bthp,bthn->bhpn", p["dy"], np.repeat(p["C"], hpg, axis=2))
    assert rel(g["dh0"], dh0) < 1e-13


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_t2.json")) as f:
        gold = json.load(f)
    i = gold["inputs"]
    x = np.array(i["x"]).reshape(1, 2, 1, 1)
    dt = np.array(i["dt"]).reshape(1, 2, 1)
    B = np.array(i["B"]).reshape(1, 2, 1, 1)
    C = np.array(i["C"]).reshape(1, 2, 1, 1)
    h0 = np.array(i["h0"]).reshape(1, 1, 1, 1)
    dy = np.array(i["dy"]).reshape(1, 2, 1, 1)
    A_log, D = np.array(i["A_log"]), np.array(i["D"])
    f = oracle.ssd_fwd(x, dt, A_log, B, C, D, h0)
    g = oracle.ssd_bwd(x, dt, A_log, B, C, D, dy, h0)
    e = gold["expected"]
    np.testing.assert_allclose(f["y"].ravel(), e["y"], rtol=1e-14)
    np.testing.assert_allclose(f["final"].ravel(), e["final"], rtol=1e-14)
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "dh0"):
        np.testing.assert_allclose(g[k].ravel(), e[k], rtol=1e-13, atol=1e-14, err_msg=k)


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("seed,h0", [(5, True), (6, False)])
def test_backward_matches_dual_form(seed, h0):
    p = rand_problem(seed, h0=h0)
    g = bwd(p)
    ref = dual_form.backward(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["dy"], p["h0"])
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "dh0"):
        assert rel(g[k], ref[k]) < 1e-12, k


def _loss(p):
    return float(np.sum(fwd(p)["y"] * p["dy"]))


def _fd_check(p, g, names, eps=1e-6, sample=None, seed=0):
    rng = np.random.default_rng(seed)
    gmap = {"x": "dx", "dt": "ddt", "A_log": "dA_log", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
    worst = 0.0
    for name in names:
        arr = p[name]
        flat_idx = np.arange(arr.size)
        if sample is not None and arr.size > sample:
            flat_idx = rng.choice(arr.size, size=sample, replace=False)
        an = g[gmap[name]].ravel()
        scale = max(1.0, np.max(np.abs(an)))
        for k in flat_idx:
            q = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in p.items()}
            q[name].ravel()[k] += eps
            lp = _loss(q)
            q[name].ravel()[k] -= 2 * eps
            lm = _loss(q)
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - an[k]) / scale
            worst = max(worst, err)
            assert err < 2e-7, (name, int(k), fd, an[k])
    return worst


def test_finite_differences_every_gradient():
    p = rand_problem(7, b=2, T=7, H=4, G=2, P=2, N=3)
    _fd_check(p, bwd(p), ["x", "dt", "A_log", "B", "C", "D", "h0"])


def test_finite_differences_p1_test_shape_sampled():
    d = make_p1test_inputs()
    p = dict(x=d["x"].values.astype(np.float64), dt=d["dt"].values.astype(np.float64),
             A_log=d["A_log"].astype(np.float64), B=d["B"].values.astype(np.float64),
             C=d["C"].values.astype(np.float64), D=d["D"].astype(np.float64),
             h0=d["h0"].astype(np.float64), dy=d["dy"].values.astype(np.float64))
    _fd_check(p, bwd(p), ["x", "dt", "A_log", "B", "C", "D", "h0"], sample=24)


def _loss_with_final(p):
    f = fwd(p)
    return float(np.sum(f["y"] * p["dy"]) + np.sum(f["final"] * p["dfinal"]))


def test_finite_differences_with_final_state_gradient():
    # L = sum(dy y) + <dfinal, final>: every gradient against central
    # differences of the oracle's forward
    p = rand_problem(11, b=2, T=6, H=4, G=2, P=2, N=3)
    p["dfinal"] = np.random.default_rng(12).standard_normal((2, 4, 2, 3))
    g = oracle.ssd_bwd(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["dy"], p["h0"], dfinal=p["dfinal"])
    gmap = {"x": "dx", "dt": "ddt", "A_log": "dA_log", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
    eps = 1e-6
    for name, gk in gmap.items():
        an = g[gk].ravel()
        scale = max(1.0, np.max(np.abs(an)))
        for k in range(p[name].size):
            q = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in p.items()}
            q[name].ravel()[k] += eps
            lp = _loss_with_final(q)
            q[name].ravel()[k] -= 2 * eps
            lm = _loss_with_final(q)
            assert abs((lp - lm) / (2 * eps) - an[k]) / scale < 2e-7, (name, k)


def test_final_state_gradient_only_closed_form():
    # With dy = 0 the loss is <dfinal, final>, and unrolling the recurrence
    # final = prod_t exp(dt_t A) h0 + sum_t exp(A sum_{s>t} dt_s) dt_t x_t (outer) B_t
    # gives the gradients in closed form.
    p = rand_problem(13, b=2, T=5, H=2, G=1, P=3, N=2)
    p["dy"] = np.zeros_like(p["dy"])
    dfin = np.random.default_rng(14).standard_normal((2, 2, 3, 2))
    g = oracle.ssd_bwd(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["dy"], p["h0"], dfinal=dfin)
    A = -np.exp(p["A_log"])
    b, T, H, P = p["x"].shape
    for bi in range(b):
        for h in range(H):
            dts = p["dt"][bi, :, h]
            np.testing.assert_allclose(g["dh0"][bi, h], np.exp(A[h] * dts.sum()) * dfin[bi, h], rtol=1e-13)
            for t in range(T):
                w = np.exp(A[h] * dts[t + 1:].sum()) * dts[t]
                np.testing.assert_allclose(g["dx"][bi, t, h], w * dfin[bi, h] @ p["B"][bi, t, 0],
                                           rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(g["dC"], 0.0)
    np.testing.assert_array_equal(g["dD"], 0.0)


def test_single_step_closed_form():
    p = rand_problem(8, b=1, T=1, H=2, G=1, P=3, N=4)
    x, dt, B, C, h0, dy = p["x"][0, 0], p["dt"][0, 0], p["B"][0, 0, 0], p["C"][0, 0, 0], p["h0"][0], p["dy"][0, 0]
    A = -np.exp(p["A_log"])
    e = np.exp(dt * A)
    f = fwd(p)
    g = bwd(p)
    for h in range(2):
        hst = e[h] * h0[h] + dt[h] * np.outer(x[h], B)
        np.testing.assert_allclose(f["y"][0, 0, h], hst @ C + p["D"][h] * x[h], rtol=1e-13)
        np.testing.assert_allclose(g["dx"][0, 0, h], p["D"][h] * dy[h] + dt[h] * (B @ C) * dy[h], rtol=1e-13)
        np.testing.assert_allclose(g["ddt"][0, 0, h], (B @ C) * (dy[h] @ x[h]) + A[h] * e[h] * (dy[h] @ h0[h] @ C),
                                   rtol=1e-12)
        np.testing.assert_allclose(g["dA_log"][h], A[h] * dt[h] * e[h] * (dy[h] @ h0[h] @ C), rtol=1e-12)
        np.testing.assert_allclose(g["dh0"][0, h], e[h] * np.outer(dy[h], C), rtol=1e-13)
        np.testing.assert_allclose(g["dD"][h], dy[h] @ x[h], rtol=1e-13)
    dB = sum(dt[h] * (dy[h] @ x[h]) * C for h in range(2))
    dC = sum(dy[h] @ (e[h] * h0[h] + dt[h] * np.outer(x[h], B)) for h in range(2))
    np.testing.assert_allclose(g["dB"][0, 0, 0], dB, rtol=1e-12)
    np.testing.assert_allclose(g["dC"][0, 0, 0], dC, rtol=1e-12)


def test_skip_path_c_zero():
    p = rand_problem(9)
    p["C"] = np.zeros_like(p["C"])
    f, g = fwd(p), bwd(p)
    np.testing.assert_allclose(f["y"], p["D"][None, None, :, None] * p["x"], rtol=1e-15)
    np.testing.assert_allclose(g["dx"], p["D"][None, None, :, None] * p["dy"], rtol=1e-15)
    for k in ("dB", "ddt", "dA_log", "dh0"):
        assert np.max(np.abs(g[k])) == 0.0, k
    np.testing.assert_allclose(g["dD"], np.einsum("bthp,bthp->h", p["dy"], p["x"]), rtol=1e-13)
    hs = dual_form.states(p["x"], p["dt"], p["A_log"], p["B"], p["h0"])
    hpg = 2
    dC = np.einsum("bthp,bthpn->btn", p["dy"][:, :, :hpg], hs[:, :, :hpg])
    assert rel(g["dC"][:, :, 0], dC) < 1e-13


def test_skip_path_b_zero_no_initial_state():
    p = rand_problem(10, h0=False)
    p["B"] = np.zeros_like(p["B"])
    f, g = fwd(p), bwd(p)
    np.testing.assert_allclose(f["y"], p["D"][None, None, :, None] * p["x"], rtol=1e-15)
    assert np.max(np.abs(g["dC"])) == 0.0
    assert np.max(np.abs(g["dA_log"])) == 0.0


def test_group_replication():
    # G groups give the same y as B/C replicated to one group per head, and dB
    # of the grouped problem is the head-sum of the replicated dB.
    p = rand_problem(11, H=4, G=2)
    q = dict(p)
    q["B"] = np.repeat(p["B"], 2, axis=2)
    q["C"] = np.repeat(p["C"], 2, axis=2)
    assert rel(fwd(p)["y"], fwd(q)["y"]) < 1e-14
    gp, gq = bwd(p), bwd(q)
    b, T = p["x"].shape[:2]
    assert rel(gp["dB"], gq["dB"].reshape(b, T, 2, 2, -1).sum(3)) < 1e-13
    assert rel(gp["dC"], gq["dC"].reshape(b, T, 2, 2, -1).sum(3)) < 1e-13
    for k in ("dx", "ddt", "dA_log", "dD", "dh0"):
        assert rel(gp[k], gq[k]) < 1e-13, k


def test_linearity():
    p1, p2 = rand_problem(12, h0=False), rand_problem(13, h0=False)
    q = dict(p1)
    q["x"] = p1["x"] + 2.0 * p2["x"]
    p2x = dict(p1)
    p2x["x"] = p2["x"]
    assert rel(fwd(q)["y"], fwd(p1)["y"] + 2.0 * fwd(p2x)["y"]) < 1e-13
    # every gradient is linear in dy
    r = dict(p1)
    r["dy"] = p1["dy"] - 3.0 * p2["dy"]
    r2 = dict(p1)
    r2["dy"] = p2["dy"]
    g, g1, g2 = bwd(r), bwd(p1), bwd(r2)
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "dh0"):
        assert rel(g[k], g1[k] - 3.0 * g2[k]) < 1e-12, k


def test_thread_count_does_not_change_results():
    p = rand_problem(14, b=3, T=70, H=4, G=2, P=4, N=6)
    g1, g8 = bwd(p, nthreads=1), bwd(p, nthreads=8)
    for k in g1:
        assert np.array_equal(g1[k], g8[k]), k
    f1, f8 = fwd(p, nthreads=1, chunk=10), fwd(p, nthreads=8, chunk=10)
    for k in f1:
        assert np.array_equal(f1[k], f8[k]), k


def test_long_time_checkpoint_segments():
    # T spans several internal checkpoint segments plus a ragged tail.
    p = rand_problem(15, b=1, T=150, H=2, G=1, P=2, N=3, a_scale=0.05)
    ref = dual_form.backward(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["dy"], p["h0"])
    g = bwd(p)
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "dh0"):
        assert rel(g[k], ref[k]) < 1e-11, k


def test_generated_inputs_follow_the_recipe():
    cfg = CONFIGS["tiny"]
    d = make_inputs(cfg)
    assert d["x"].shape == (1, 64, 2, 8) and d["B"].shape == (1, 64, 1, 4)
    assert np.all(d["dt"].values > 0)
    A = -np.exp(d["A_log"])
    assert np.all(A <= -1.0) and np.all(A >= -16.0)
    assert d["h0"] is None
    d2 = make_inputs(cfg)
    assert np.array_equal(d["x"].values, d2["x"].values)
    assert P1TEST.nheads == 4 and make_p1test_inputs()["x"].values[0, 0, 0, 0] == np.float32(-0.5)
