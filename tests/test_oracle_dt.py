"""Pins of the oracle's dt activation (dt = softplus(dt_raw + dt_bias) and its
gradient; the burn_dragon_kernel src/sequence/mamba2/backward.rs page, the dt_pre and
grad_dt_pre / grad_dt_bias lines of tensorized_mamba2_backward_impl) against
closed forms of softplus and against central differences of the whole chain
dt_raw, dt_bias -> dt -> SSD forward -> L = sum(dy * y)."""
import math

import numpy as np

import oracle


def test_softplus_closed_forms():
    bias = np.zeros(3)
    v = np.array([[0.0, 1.0, -1.0], [30.0, -30.0, 2.5]])
    sp = oracle.dt_softplus_fwd(v, bias)
    assert abs(sp[0, 0] - math.log(2.0)) < 1e-15
    assert abs(sp[0, 1] - math.log(1.0 + math.e)) < 1e-15
    # softplus(v) - softplus(-v) = v
    assert abs(sp[0, 1] - sp[0, 2] - 1.0) < 1e-15
    # large arguments: softplus(v) -> v, softplus(-v) -> e^-v
    assert abs(sp[1, 0] - 30.0) < 1e-12
    assert abs(sp[1, 1] - math.exp(-30.0)) / math.exp(-30.0) < 1e-12
    # the bias adds to the pre-activation per head (last axis)
    b = np.array([0.5, -2.0, 1.0])
    np.testing.assert_allclose(oracle.dt_softplus_fwd(v, b), oracle.dt_softplus_fwd(v + b, bias), rtol=0, atol=0)


def test_softplus_gradient_is_sigmoid():
    rng = np.random.default_rng(3)
    raw = rng.standard_normal((2, 5, 3))
    bias = rng.uniform(-4, -2, 3)
    ones = np.ones_like(raw)
    g, gb = oracle.dt_softplus_bwd(raw, bias, ones)
    eps = 1e-6
    fd = (oracle.dt_softplus_fwd(raw + eps, bias) - oracle.dt_softplus_fwd(raw - eps, bias)) / (2 * eps)
    np.testing.assert_allclose(g, fd, rtol=1e-8, atol=1e-12)
    # at v = 0 the sigmoid is exactly 1/2
    g0, _ = oracle.dt_softplus_bwd(np.zeros((1, 1, 2)), np.zeros(2), np.array([[[2.0, -4.0]]]))
    np.testing.assert_array_equal(g0, [[[1.0, -2.0]]])
    # d_dt_bias sums over every row (batch and time), per head
    np.testing.assert_allclose(gb, g.reshape(-1, 3).sum(axis=0), rtol=1e-15)


def test_chain_finite_differences():
    rng = np.random.default_rng(21)
    b, T, H, G, P, N = 2, 6, 4, 2, 2, 3
    p = dict(x=rng.standard_normal((b, T, H, P)), B=rng.standard_normal((b, T, G, N)),
             C=rng.standard_normal((b, T, G, N)), A_log=rng.uniform(0, np.log(16), H),
             D=rng.standard_normal(H), dy=rng.standard_normal((b, T, H, P)))
    raw = rng.standard_normal((b, T, H))
    bias = rng.uniform(-4, -2, H)

    def loss(raw_, bias_):
        dt = oracle.dt_softplus_fwd(raw_, bias_)
        y = oracle.ssd_fwd(p["x"], dt, p["A_log"], p["B"], p["C"], p["D"])["y"]
        return float(np.sum(y * p["dy"]))

    dt = oracle.dt_softplus_fwd(raw, bias)
    g = oracle.ssd_bwd(p["x"], dt, p["A_log"], p["B"], p["C"], p["D"], p["dy"])
    g_raw, g_bias = oracle.dt_softplus_bwd(raw, bias, g["ddt"])
    eps = 1e-6
    scale = max(1.0, float(np.max(np.abs(g_raw))))
    for k in range(raw.size):
        rp, rm = raw.copy(), raw.copy()
        rp.ravel()[k] += eps
        rm.ravel()[k] -= eps
        fd = (loss(rp, bias) - loss(rm, bias)) / (2 * eps)
        assert abs(fd - g_raw.ravel()[k]) / scale < 1e-7, k
    for h in range(H):
        bp, bm = bias.copy(), bias.copy()
        bp[h] += eps
        bm[h] -= eps
        fd = (loss(raw, bp) - loss(raw, bm)) / (2 * eps)
        assert abs(fd - g_bias[h]) / max(1.0, abs(g_bias[h])) < 1e-7, h
