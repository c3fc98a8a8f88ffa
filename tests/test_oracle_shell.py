"""Pins of the shell oracle (causal depthwise conv + SiLU, RMSNorm-gated).

The conv preactivation is pinned to numpy's convolve per channel and to the
unit-impulse identity.  SiLU (v times the logistic function) is pinned by
identities that any correct logistic gate satisfies and a dropped term or a
wrong sign breaks: silu(0) = 0, the odd part silu(v) - silu(-v) = v, the even
part silu(v) + silu(-v) = v tanh(v / 2), the closed values at v = +-ln 3
(the logistic function is 3/4 and 1/4 there) and the limits silu(v)/v -> 1,
silu(-v) -> -v e^-v for large v.  RMSNorm-gated is pinned by what fixes each
of its factors: a constant row c gives inv_rms = 1/sqrt(c^2 + eps) (eps inside
the square root, added to the mean square); a one-hot row gives mean square
v^2 / width (the divisor is the width); at eps = 0 the output is invariant
under y -> alpha y for alpha > 0, odd in y, and y * inv_rms has mean square 1
(checked against numpy's vector norm); the weight scales each column and the
gate is silu(z) per element.  Every backward is pinned to central finite
differences of the oracle's own forward, which the pins above fix.
"""
import numpy as np
import pytest
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


# ---------------------------------------------------------------- SiLU pins
# conv_fwd with a unit impulse on the current tap and no bias returns the
# input unchanged as the preactivation, so its act is silu of the input.

def silu_via_conv(v):
    v = np.asarray(v, np.float64)
    x = v.reshape(1, -1, 1)
    w = np.array([[0.0, 0.0, 0.0, 1.0]])
    pre, act = oracle.conv_fwd(x, w, np.zeros(1))
    assert np.array_equal(pre.ravel(), v.ravel())
    return act.ravel()


def test_silu_zero_and_odd_part():
    rng = np.random.default_rng(11)
    v = np.concatenate([[0.0], rng.standard_normal(64) * 4.0])
    a = silu_via_conv(v)
    b = silu_via_conv(-v)
    assert a[0] == 0.0
    # v s(v) + v s(-v) = v because s(v) + s(-v) = 1
    np.testing.assert_allclose(a - b, v, rtol=1e-14, atol=1e-15)


def test_silu_even_part_is_tanh():
    # v s(v) - v s(-v) = v (2 s(v) - 1) = v tanh(v / 2)
    v = np.linspace(-12.0, 12.0, 97)
    a, b = silu_via_conv(v), silu_via_conv(-v)
    np.testing.assert_allclose(a + b, v * np.tanh(v / 2.0), rtol=1e-13, atol=1e-15)


def test_silu_closed_values_and_limits():
    l3 = np.log(3.0)
    a = silu_via_conv([l3, -l3, 40.0, -40.0])
    # logistic(ln 3) = 3 / (3 + 1), logistic(-ln 3) = 1 / 4
    assert abs(a[0] - 0.75 * l3) <= 1e-15
    assert abs(a[1] + 0.25 * l3) <= 1e-15
    # large v: silu(v) / v -> 1 and silu(-v) -> -v e^-v (relative 1e-17 terms)
    assert abs(a[2] / 40.0 - 1.0) <= 1e-15
    assert abs(a[3] / (-40.0 * np.exp(-40.0)) - 1.0) <= 1e-12


# ------------------------------------------------------ RMSNorm-gated pins

GATE = 0.75 * np.log(3.0)  # silu(ln 3), pinned above


def test_rmsnorm_constant_row_places_eps_inside_the_root():
    # a constant row c: the mean square is c^2, so inv_rms = 1 / sqrt(c^2 + eps)
    width = 40
    for c, eps in ((0.3, 1e-5), (-2.0, 0.25), (1e-3, 1e-5), (0.0, 1e-5)):
        y = np.full((1, width), c)
        z = np.full((1, width), np.log(3.0))
        out, inv = oracle.rmsnorm_fwd(y, z, np.ones(width), eps)
        ref = 1.0 / np.sqrt(c * c + eps)
        assert abs(inv[0] - ref) <= 1e-14 * ref
        np.testing.assert_allclose(out, c * ref * GATE, rtol=1e-14, atol=1e-300)


def test_rmsnorm_one_hot_row_divides_by_width():
    # one nonzero entry v: the mean square is v^2 / width
    for width, v, eps in ((7, 3.0, 0.0), (64, -0.5, 1e-5), (3072, 10.0, 1e-5)):
        y = np.zeros((1, width))
        y[0, width // 2] = v
        _, inv = oracle.rmsnorm_fwd(y, np.zeros((1, width)), np.ones(width), eps)
        ref = 1.0 / np.sqrt(v * v / width + eps)
        assert abs(inv[0] - ref) <= 1e-14 * ref


def test_rmsnorm_scale_invariance_sign_and_unit_mean_square():
    rng = np.random.default_rng(12)
    rows, width = 5, 33
    y = rng.standard_normal((rows, width))
    z = 60.0 + np.abs(rng.standard_normal((rows, width)))  # silu(z) = z to 1e-24 relative
    w = np.ones(width)
    out, inv = oracle.rmsnorm_fwd(y, z, w, 0.0)
    for alpha in (1e-3, 0.5, 7.0, 1e4):
        out_a, _ = oracle.rmsnorm_fwd(alpha * y, z, w, 0.0)
        np.testing.assert_allclose(out_a, out, rtol=1e-13)
    out_n, _ = oracle.rmsnorm_fwd(-y, z, w, 0.0)
    np.testing.assert_allclose(out_n, -out, rtol=0, atol=0)
    # inv_rms from numpy's 2-norm: sqrt(width) / |y|
    np.testing.assert_allclose(inv, np.sqrt(width) / np.linalg.norm(y, axis=-1), rtol=1e-14)
    normalized = out / z
    np.testing.assert_allclose(np.mean(normalized * normalized, axis=-1), 1.0, rtol=1e-13)


def test_rmsnorm_weight_scales_columns_and_gate_is_elementwise():
    rng = np.random.default_rng(13)
    rows, width = 3, 17
    y = rng.standard_normal((rows, width))
    w = 1.0 + rng.standard_normal(width)
    z = rng.standard_normal((rows, width))
    out, inv = oracle.rmsnorm_fwd(y, z, w, 1e-5)
    # the weight multiplies column i only; the gate multiplies element (r, i) only
    out1, inv1 = oracle.rmsnorm_fwd(y, np.full_like(z, np.log(3.0)), np.ones(width), 1e-5)
    np.testing.assert_array_equal(inv, inv1)
    gate = silu_via_conv(z.ravel()).reshape(rows, width)
    np.testing.assert_allclose(out, out1 / GATE * w * gate, rtol=1e-13, atol=1e-15)
