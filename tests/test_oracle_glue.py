"""Pins of the oracle's MoE-layer glue (SwiGLU, router-weighted combine).

These steps are not on the pages; they are the standard SwiGLU expert MLP
and the weighted sum of routed experts.  Pins: closed forms of the logistic
function, the identity silu(x) - silu(-x) = x, scipy's expit, hand-built
inputs for the gate/up split and one-hot / linearity of the combine."""
import math

import numpy as np
import scipy.special

import oracle


def test_silu_closed_forms_and_limits():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(oracle.silu(np.array([1.0]))[0], 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(oracle.silu(np.array([math.log(3.0)]))[0], 0.75 * math.log(3.0), rel_tol=1e-15)
    big = oracle.silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 800.0
    assert np.isnan(oracle.silu(np.array([np.nan]))[0])


def test_silu_odd_part_identity_and_expit():
    x = np.random.default_rng(0).normal(size=1000) * 6
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)


def test_swiglu_takes_gate_first_then_up():
    gu = np.array([[[2.0, -1.0, 0.0, 3.0, 5.0, 7.0]]])  # gate (2, -1, 0), up (3, 5, 7)
    h = oracle.swiglu(gu)
    assert h.shape == (1, 1, 3)
    expect = [2.0 / (1 + math.exp(-2.0)) * 3.0, -1.0 / (1 + math.exp(1.0)) * 5.0, 0.0]
    np.testing.assert_allclose(h[0, 0], expect, rtol=1e-15)


def test_combine_one_hot_linear_and_nan():
    rng = np.random.default_rng(1)
    yp = rng.normal(size=(3, 4, 5))
    onehot = np.zeros((3, 4))
    onehot[np.arange(3), [2, 0, 3]] = 1.0
    np.testing.assert_array_equal(oracle.combine(yp, onehot), yp[np.arange(3), [2, 0, 3]])
    w1, w2 = rng.normal(size=(3, 4)), rng.normal(size=(3, 4))
    np.testing.assert_allclose(oracle.combine(yp, 2 * w1 - w2), 2 * oracle.combine(yp, w1) - oracle.combine(yp, w2),
                               rtol=1e-12, atol=1e-12)
    hand = oracle.combine(np.array([[[1.0, 2.0], [10.0, 20.0]]]), np.array([[0.25, 0.5]]))
    np.testing.assert_array_equal(hand, [[5.25, 10.5]])
    yp[1, 2, 0] = np.nan
    c = oracle.combine(yp, w1)
    assert np.all(np.isnan(c[1, :1])) and not np.any(np.isnan(c[0]))
