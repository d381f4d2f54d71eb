"""Pins of the convolution oracle (oracle/gla_conv_oracle.c) against facts
that do not come from the oracle itself: a library correlation, SiLU values
and identities, tap placement on impulse inputs, and the chaining of the
carried window.  Page: "Beyond the KV cache ...", section "i14 and Laplace 3B
architecture", paragraph "Normalization and convolution"."""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gated_linear_attention_gla_amd import inputs


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_matches_library_correlation():
    """z equals numpy's valid-mode correlation of [window, x] with the taps
    (per channel), and y = z * expit(z) with scipy's logistic function."""
    B, T, D = 2, 37, 5
    x, w, b, win = rnd(1, B, T, D), rnd(2, D, 4), rnd(3, D), rnd(4, B, 3, D)
    y, st = oracle.conv1d(x, w, b, win)
    for bi in range(B):
        for c in range(D):
            xp = np.concatenate([win[bi, :, c], x[bi, :, c]])
            z = np.correlate(xp, w[c], mode="valid") + b[c]
            assert z.shape == (T,)
            np.testing.assert_allclose(y[bi, :, c], z * expit(z), rtol=1e-13, atol=1e-13)


def test_silu_known_values():
    # SiLU(1) = sigmoid(1) = 0.7310585786300049; SiLU(0) = 0;
    # SiLU(z) - SiLU(-z) = z for every z
    D = 3
    w = np.zeros((D, 4))
    w[:, 3] = 1.0
    x = np.array([[[1.0, 0.0, 2.5], [-2.5, 7.0, -7.0]]])
    y, _ = oracle.conv1d(x, w)
    assert y[0, 0, 0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert y[0, 0, 1] == 0.0
    assert y[0, 0, 2] - y[0, 1, 0] == pytest.approx(2.5, rel=1e-14)
    assert y[0, 1, 1] - y[0, 1, 2] == pytest.approx(7.0, rel=1e-14)


def test_current_token_tap_is_last():
    """Taps (0, 0, 0, 1): the output at t depends on x[t] only."""
    x = rnd(5, 1, 9, 2)
    w = np.tile([0.0, 0.0, 0.0, 1.0], (2, 1))
    y, st = oracle.conv1d(x, w, None, rnd(6, 1, 3, 2))
    np.testing.assert_allclose(y, x * expit(x), rtol=1e-14)


def test_oldest_tap_reaches_three_tokens_back():
    """Taps (1, 0, 0, 0): y[t] = SiLU(x[t-3]), the first three outputs from the window."""
    x, win = rnd(7, 1, 8, 3), rnd(8, 1, 3, 3)
    w = np.tile([1.0, 0.0, 0.0, 0.0], (3, 1))
    y, _ = oracle.conv1d(x, w, None, win)
    xp = np.concatenate([win, x], axis=1)
    np.testing.assert_allclose(y, xp[:, :8] * expit(xp[:, :8]), rtol=1e-14)


def test_missing_window_is_zero():
    x, w = rnd(9, 2, 6, 4), rnd(10, 4, 4)
    y0, s0 = oracle.conv1d(x, w)
    y1, s1 = oracle.conv1d(x, w, None, np.zeros((2, 3, 4)))
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(s0, s1)


def test_window_out_is_last_three_inputs():
    x, w, win = rnd(11, 2, 10, 4), rnd(12, 4, 4), rnd(13, 2, 3, 4)
    _, st = oracle.conv1d(x, w, None, win)
    np.testing.assert_array_equal(st, x[:, -3:])
    # fewer than three tokens: the window keeps its newest entries
    _, st2 = oracle.conv1d(x[:, :2], w, None, win)
    np.testing.assert_array_equal(st2, np.concatenate([win[:, 2:], x[:, :2]], axis=1))
    _, st0 = oracle.conv1d(x[:, :0], w, None, win)
    np.testing.assert_array_equal(st0, win)


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_chained_calls_equal_one_call(split):
    x, w, b, win = rnd(14, 2, 11, 6), rnd(15, 6, 4), rnd(16, 6), rnd(17, 2, 3, 6)
    y, st = oracle.conv1d(x, w, b, win)
    ya, sa = oracle.conv1d(x[:, :split], w, b, win)
    yb, sb = oracle.conv1d(x[:, split:], w, b, sa)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(sb, st)


def test_decode_steps_equal_prefill():
    x, w, b, win = rnd(18, 3, 7, 8), rnd(19, 8, 4), rnd(20, 8), rnd(21, 3, 3, 8)
    y, st = oracle.conv1d(x, w, b, win)
    s = win.copy()
    for t in range(7):
        yt, s = oracle.conv1d_step(x[:, t], w, b, s)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(s, st)


def test_planted_tap_reversal_is_caught():
    """A reversed tap order (a plausible mistake) changes the result."""
    x, w = rnd(22, 1, 9, 3), rnd(23, 3, 4)
    y, _ = oracle.conv1d(x, w)
    yr, _ = oracle.conv1d(x, w[:, ::-1])
    assert np.max(np.abs(y - yr)) > 1e-3


def test_seeded_conv_inputs_are_stored_values():
    c = inputs.conv_inputs(3, 1, 4, 8, "bf16")
    assert np.array_equal(c["x"], inputs.round_bf16(c["x"]))
    assert np.array_equal(c["w"], inputs.round_f32(c["w"]))
    assert c["state"].shape == (1, 3, 8)
