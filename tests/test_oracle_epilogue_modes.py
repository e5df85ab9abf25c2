"""Pins of the oracle's other epilogue modes: SiLU, ReLU, tanh and the factor alpha.

These are wavo's `Epilogue` modes (gpu/mod.rs: Silu, Relu, Tanh, Residual(alpha), GeluResidual and
its test reference `epilogue`). Each is checked against something other than its own formula:
identities between SiLU and tanh, the exponential form of tanh, textbook values, hand examples of
the order (bias, activation, alpha, old output) and a brute-force layer on tiny shapes.
"""
import math

import numpy as np
import pytest

import oracle
import synth

ACTS = [oracle.FLAG_GELU, oracle.FLAG_SILU, oracle.FLAG_RELU, oracle.FLAG_TANH]


def test_silu_equals_half_x_times_one_plus_tanh_half_x():
    # x * sigma(x) == x/2 * (1 + tanh(x/2)): pins SiLU and tanh against each other. (For x far
    # below 0 the right side cancels in 1 + tanh, so the range stops at -10.)
    x = np.linspace(-10, 30, 4001)
    np.testing.assert_allclose(oracle.silu(x), 0.5 * x * (1.0 + oracle.tanh(0.5 * x)), rtol=1e-11, atol=1e-15)


def test_silu_odd_part_and_limits():
    x = np.linspace(-20, 20, 4001)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-13)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-20)
    assert abs(oracle.silu(-800.0)) == 0.0  # exp overflow gives -0, not NaN


def test_tanh_exponential_form_and_values():
    for x in np.linspace(-9, 9, 181):
        e = math.exp(2.0 * x)
        assert oracle.tanh(x) == pytest.approx((e - 1.0) / (e + 1.0), rel=1e-13, abs=1e-15)
    # tanh(1) = (e^2 - 1) / (e^2 + 1), tanh(ln 2) = 3/5 exactly
    assert oracle.tanh(1.0) == pytest.approx(0.7615941559557649, rel=1e-15)
    assert oracle.tanh(math.log(2.0)) == pytest.approx(0.6, rel=1e-15)
    np.testing.assert_array_equal(oracle.tanh(np.array([0.0, 40.0, -40.0])), [0.0, 1.0, -1.0])


def test_silu_value_at_ln3():
    # sigma(ln 3) = 3/4, so silu(ln 3) = 3/4 ln 3
    assert oracle.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)


def test_relu_values():
    np.testing.assert_array_equal(oracle.relu(np.array([-2.5, -0.0, 0.0, 1e-30, 3.0])), [0.0, 0.0, 0.0, 1e-30, 3.0])


def _one_output(flags, v, bias, y_old, alpha):
    # x = [v, 0, ...], w = [1, 0, ...]: the product is exactly v
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = v
    w = np.zeros((1, 32), np.uint16)
    w[0, 0] = 0x3F80
    got, _ = oracle.linear(x, w, oracle.W_BF16, 1, 32, np.array([bias], np.float32), flags,
                           np.array([[y_old]], np.float32), alpha=alpha)
    return got[0, 0]


def test_order_bias_activation_alpha_residual():
    B, R = oracle.FLAG_BIAS, oracle.FLAG_RESIDUAL
    # bias before the activation: relu(-1 + 2) = 1 (relu(-1) + 2 would be 2)
    assert _one_output(B | oracle.FLAG_RELU, -1.0, 2.0, 0.0, 1.0) == 1.0
    # alpha after the activation, before the old output: 5 + 0.5 * relu(3 + 1) = 7
    assert _one_output(B | oracle.FLAG_RELU | R, 3.0, 1.0, 5.0, 0.5) == 7.0
    # wavo Residual(alpha): c + alpha * (a.W^T + b) = 2 + 0.25 * (4 - 8) = 1
    assert _one_output(B | R, 4.0, -8.0, 2.0, 0.25) == 1.0
    # tanh(ln 2) = 3/5, times alpha 10, plus 1 (ln 2 enters rounded to f32: 1e-6 slack)
    assert _one_output(B | oracle.FLAG_TANH | R, math.log(2.0), 0.0, 1.0, 10.0) == pytest.approx(7.0, abs=1e-6)
    # silu(ln 3) = 3/4 ln 3, times -2
    assert _one_output(oracle.FLAG_SILU, math.log(3.0), 0.0, 0.0, -2.0) == pytest.approx(-1.5 * math.log(3.0),
                                                                                         abs=1e-6)


def test_alpha_one_is_the_plain_epilogue_and_two_activations_are_refused():
    g = synth.rng(61)
    x = synth.normal_f32(g, (3, 64), 1.0)
    w = synth.bf16_weight(g, 5, 64, 0.1)
    b = synth.normal_f32(g, (5,), 0.1)
    y_old = synth.normal_f32(g, (3, 5), 1.0)
    for flags in range(8):
        plain, _ = oracle.linear(x, w, oracle.W_BF16, 5, 64, b, flags, y_old)
        one, _ = oracle.linear(x, w, oracle.W_BF16, 5, 64, b, flags, y_old, alpha=1.0)
        assert np.array_equal(plain, one)
    with pytest.raises(ValueError):
        oracle.linear(x, w, oracle.W_BF16, 5, 64, b, oracle.FLAG_GELU | oracle.FLAG_TANH, y_old)


def _brute(x, w_raw, wtype, m, k, bias, act, alpha, y_old):
    w = oracle.decode(w_raw, wtype, m, k)
    n = x.shape[0]
    y = np.zeros((n, m))
    f = {oracle.FLAG_GELU: lambda v: 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))),
         oracle.FLAG_SILU: lambda v: v * 0.5 * (1.0 + math.tanh(0.5 * v)),
         oracle.FLAG_RELU: lambda v: v if v > 0 else 0.0,
         oracle.FLAG_TANH: lambda v: (math.exp(2 * v) - 1.0) / (math.exp(2 * v) + 1.0)}[act]
    for t in range(n):
        for j in range(m):
            v = math.fsum(float(x[t, i]) * w[j][i] for i in range(k)) + float(bias[j])
            y[t, j] = float(y_old[t, j]) + alpha * f(v)
    return y


@pytest.mark.parametrize("wtype", [oracle.W_BF16, oracle.W_Q8_0, oracle.W_Q4_0])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("alpha", [1.0, 0.5, -3.0])
def test_linear_with_each_activation_matches_brute_force(wtype, act, alpha):
    n, m, k = 2, 3, 64
    g = synth.rng(62, wtype, act)
    x = synth.normal_f32(g, (n, k), 1.0)
    raw = synth.weight(g, wtype, m, k, sigma=0.3, dsigma=0.05)
    bias = synth.normal_f32(g, (m,), 0.3)
    y_old = synth.normal_f32(g, (n, m), 1.0)
    flags = oracle.FLAG_BIAS | act | oracle.FLAG_RESIDUAL
    got, _ = oracle.linear(x, raw, wtype, m, k, bias, flags, y_old, alpha=alpha)
    want = _brute(x, raw, wtype, m, k, bias, act, alpha, y_old)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_dual_outputs_repeat_the_first_outputs_with_their_own_bias():
    # wavo Linear.dual: the first `dual` outputs again after the m others, with bias[m + j].
    g = synth.rng(63)
    n, m, k, dual = 3, 5, 64, 2
    x = synth.normal_f32(g, (n, k), 1.0)
    w = synth.bf16_weight(g, m, k, 0.1)
    bias = synth.normal_f32(g, (m + dual,), 0.5)
    y_old = synth.normal_f32(g, (n, m + dual), 1.0)
    flags = oracle.FLAG_BIAS | oracle.FLAG_SILU | oracle.FLAG_RESIDUAL
    got, s = oracle.linear_dual(x, w, oracle.W_BF16, m, k, dual, bias, flags, y_old, alpha=0.5)
    assert got.shape == (n, m + dual) and s.shape == (n, m + dual)
    # brute force, column by column
    wd = oracle.decode(w, oracle.W_BF16, m, k)
    for t in range(n):
        for c in range(m + dual):
            j = c if c < m else c - m
            v = math.fsum(float(x[t, i]) * wd[j, i] for i in range(k)) + float(bias[c])
            want = float(y_old[t, c]) + 0.5 * v * 0.5 * (1.0 + math.tanh(0.5 * v))
            assert got[t, c] == pytest.approx(want, rel=1e-12, abs=1e-12)
    assert np.array_equal(s[:, m:], s[:, :dual])
    # dual = 0 is the plain layer
    plain, _ = oracle.linear(x, w, oracle.W_BF16, m, k, bias[:m], flags, y_old[:, :m], alpha=0.5)
    zero, _ = oracle.linear_dual(x, w, oracle.W_BF16, m, k, 0, bias[:m], flags, y_old[:, :m], alpha=0.5)
    assert np.array_equal(plain, zero)
    with pytest.raises(ValueError):
        oracle.linear_dual(x, w, oracle.W_BF16, m, k, m + 1)
