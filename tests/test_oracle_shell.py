"""Pins of the shell oracle (causal depthwise conv + SiLU, RMSNorm-gated).

The conv preactivation is pinned to numpy's convolve per channel and to the
unit-impulse identity; SiLU to scipy's logistic function; RMSNorm-gated to the
formula written directly in numpy; every backward to central finite
differences of the oracle's own forward.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def conv_problem(seed, b=2, T=11, cd=5, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, T, cd)), 0.5 * rng.standard_normal((cd, K)),
            0.1 * rng.standard_normal(cd), rng.standard_normal((b, T, cd)))


def test_conv_matches_numpy_convolve():
    x, w, bias, _ = conv_problem(1)
    pre, act = oracle.conv_fwd(x, w, bias)
    b, T, cd = x.shape
    for bi in range(b):
        for c in range(cd):
            ref = np.convolve(x[bi, :, c], w[c, ::-1])[:T] + bias[c]
            np.testing.assert_allclose(pre[bi, :, c], ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(act, pre * expit(pre), rtol=1e-14)


def test_conv_unit_impulse_is_identity():
    x, w, bias, _ = conv_problem(2)
    w = np.zeros_like(w)
    w[:, -1] = 1.0
    pre, _ = oracle.conv_fwd(x, w, np.zeros_like(bias))
    assert np.array_equal(pre, x)
    # the oldest tap sees the input K-1 steps back, zeros before t = 0
    w2 = np.zeros_like(w)
    w2[:, 0] = 1.0
    pre2, _ = oracle.conv_fwd(x, w2, np.zeros_like(bias))
    assert np.array_equal(pre2[:, 3:], x[:, :-3]) and np.all(pre2[:, :3] == 0)


def test_conv_backward_finite_differences():
    x, w, bias, g = conv_problem(3, b=2, T=6, cd=3, K=4)
    dx, dw, db = oracle.conv_bwd(x, w, bias, g)

    def loss(x_, w_, b_):
        return float(np.sum(g * oracle.conv_fwd(x_, w_, b_)[1]))

    eps = 1e-6
    for arr, grad, which in ((x, dx, 0), (w, dw, 1), (bias, db, 2)):
        for k in range(arr.size):
            args = [x.copy(), w.copy(), bias.copy()]
            args[which].ravel()[k] += eps
            lp = loss(*args)
            args[which].ravel()[k] -= 2 * eps
            lm = loss(*args)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.ravel()[k]) < 1e-7 * max(1.0, abs(fd)), (which, k)


def rms_problem(seed, rows=(2, 3), width=7):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(rows + (width,)), rng.standard_normal(rows + (width,)),
            1.0 + 0.1 * rng.standard_normal(width), rng.standard_normal(rows + (width,)))


def test_rmsnorm_gated_forward_formula():
    y, z, w, _ = rms_problem(4)
    eps = 1e-5
    out, inv = oracle.rmsnorm_fwd(y, z, w, eps)
    inv_ref = 1.0 / np.sqrt(np.mean(y * y, axis=-1) + eps)
    np.testing.assert_allclose(inv, inv_ref, rtol=1e-14)
    np.testing.assert_allclose(out, y * inv_ref[..., None] * w * (z * expit(z)), rtol=1e-13)


def test_rmsnorm_gated_large_z_is_plain_rmsnorm_times_z():
    # silu(z) -> z as z -> +inf: the gate becomes multiplication by z.
    y, z, w, _ = rms_problem(5)
    z = 60.0 + np.abs(z)
    out, inv = oracle.rmsnorm_fwd(y, z, w, 1e-5)
    np.testing.assert_allclose(out, y * inv[..., None] * w * z, rtol=1e-14)


@pytest.mark.parametrize("seed", [6, 7])
def test_rmsnorm_gated_backward_finite_differences(seed):
    y, z, w, g = rms_problem(seed)
    eps_n = 1e-5
    _, inv = oracle.rmsnorm_fwd(y, z, w, eps_n)
    dy, dz, dw = oracle.rmsnorm_bwd(y, z, w, inv, g)

    def loss(y_, z_, w_):
        return float(np.sum(g * oracle.rmsnorm_fwd(y_, z_, w_, eps_n)[0]))

    eps = 1e-6
    for arr, grad, which in ((y, dy, 0), (z, dz, 1), (w, dw, 2)):
        for k in range(arr.size):
            args = [y.copy(), z.copy(), w.copy()]
            args[which].ravel()[k] += eps
            lp = loss(*args)
            args[which].ravel()[k] -= 2 * eps
            lm = loss(*args)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.ravel()[k]) < 1e-7 * max(1.0, abs(fd)), (which, k)


def test_bf16_rounding_matches_torch():
    import torch
    from ssd_inputs import bf16_bits, bf16_to_f32
    rng = np.random.default_rng(8)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties to even both ways
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(a), ref)
    assert np.array_equal(bf16_to_f32(ref), torch.from_numpy(a).to(torch.bfloat16).float().numpy())
