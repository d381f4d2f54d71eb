"""Pins of the output-epilogue oracle (oracle/gla_epilogue_oracle.c): hand
worked cases with exact intermediate values, and invariants of the
definition.  Page: "Beyond the KV cache ...", section "GLA mixer"
(self-augmentation gate, Head RMSNorm per decay tier, SiLU output gate)."""
import math

import numpy as np
import pytest

import oracle

SIG1 = 0.7310585786300049  # sigmoid(1) = SiLU(1)


def one_token(q, k, v, o, a, gamma, g, eps=0.0):
    """Shape single-token single-head arrays for the oracle."""
    q, k, v, o, g = (np.asarray(t, dtype=np.float64)[None, None, None] for t in (q, k, v, o, g))
    return oracle.epilogue(q, k, v, o, np.asarray(a, dtype=np.float64)[None],
                           np.asarray(gamma, dtype=np.float64)[None], eps, g)[0, 0, 0]


def test_zero_balance_gives_half_skip():
    """a = 0: gate = 1/2.  o = (0.5, -1.5), v = (1, 5) -> o' = (1, 1), RMS 1;
    gamma = (2, 3), g = (1, 0): y = (2 sigmoid(1), 0)."""
    y = one_token([0.3], [-0.7], [1.0, 5.0], [0.5, -1.5], [0.0], [2.0, 3.0], [1.0, 0.0])
    assert y[0] == pytest.approx(2 * SIG1, rel=1e-15)
    assert y[1] == 0.0


def test_gate_is_sigmoid_of_scaled_dot():
    """q . (a * k) = ln 3 -> gate = 3/4.  o = (1, -0.5), v = (0, 2) -> o' = (1, 1);
    a gate of 1/4 (sign flipped) would give o' = (1, 0) instead."""
    y = one_token([math.log(3.0)], [1.0], [0.0, 2.0], [1.0, -0.5], [1.0], [1.0, 1.0], [1.0, 1.0])
    np.testing.assert_allclose(y, [SIG1, SIG1], rtol=1e-14)
    # the per-channel scale multiplies element-wise: a = (2, 0) ignores channel 1
    y2 = one_token([math.log(3.0) / 2, 9.0], [1.0, 9.0], [0.0, 2.0], [1.0, -0.5], [2.0, 0.0],
                   [1.0, 1.0], [1.0, 1.0])
    np.testing.assert_allclose(y2, [SIG1, SIG1], rtol=1e-14)


def test_rmsnorm_uses_mean_square_plus_eps():
    """o' = (3, 4): mean square 12.5; with eps = 3.5 the scale is 1 / sqrt(16) = 1/4."""
    y = one_token([0.0], [0.0], [0.0, 0.0], [3.0, 4.0], [0.0], [1.0, 1.0], [1.0, 1.0], eps=3.5)
    np.testing.assert_allclose(y, [0.75 * SIG1, 1.0 * SIG1], rtol=1e-14)


def test_cancellation_gives_zero():
    r = np.random.default_rng(1)
    o = r.standard_normal(6)
    y = one_token(r.standard_normal(3), r.standard_normal(3), -2.0 * o, o, [0.0] * 3, r.standard_normal(6),
                  r.standard_normal(6), eps=1e-6)
    assert np.all(y == 0.0)


def test_scale_invariance_without_eps():
    r = np.random.default_rng(2)
    B, H, T, dk, dv = 1, 2, 5, 4, 6
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
    v, o, g = (r.standard_normal((B, H, T, dv)) for _ in range(3))
    a, gam = r.standard_normal((H, dk)), r.standard_normal((H, dv))
    y = oracle.epilogue(q, k, v, o, a, gam, 0.0, g)
    y7 = oracle.epilogue(q, k, 7.0 * v, 7.0 * o, a, gam, 0.0, g)
    np.testing.assert_allclose(y7, y, rtol=1e-12, atol=1e-14)


def test_head_weights_are_per_head():
    r = np.random.default_rng(3)
    B, H, T, dk, dv = 1, 3, 4, 2, 5
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
    v, o, g = (r.standard_normal((B, H, T, dv)) for _ in range(3))
    a = r.standard_normal((H, dk))
    gam = np.ones((H, dv))
    y1 = oracle.epilogue(q, k, v, o, a, gam, 1e-6, g)
    gam2 = gam.copy()
    gam2[1] *= 3.0
    y3 = oracle.epilogue(q, k, v, o, a, gam2, 1e-6, g)
    np.testing.assert_allclose(y3[:, 1], 3.0 * y1[:, 1], rtol=1e-14)
    np.testing.assert_array_equal(y3[:, [0, 2]], y1[:, [0, 2]])


def test_planted_mistake_is_caught():
    """Dropping the epsilon (a plausible slip) changes a tiny-output case."""
    y = one_token([0.0], [0.0], [0.0, 0.0], [1e-4, 0.0], [0.0], [1.0, 1.0], [1.0, 1.0], eps=1e-8)
    y0 = one_token([0.0], [0.0], [0.0, 0.0], [1e-4, 0.0], [0.0], [1.0, 1.0], [1.0, 1.0], eps=0.0)
    assert abs(y[0] - y0[0]) > 1e-3 * abs(y0[0])
