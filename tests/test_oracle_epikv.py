"""Pins of the oracle's attention-free (hidden-state change) score."""
import math

import numpy as np
import pytest

from oracle import epikv_g, rolling_z, epikv_score


def test_g_hand_example():
    h = np.array([[0.0, 0.0], [3.0, 4.0], [3.0, 4.0], [0.0, 0.0], [1.0, 0.0]])
    assert epikv_g(h).tolist() == [0.0, 5.0, 0.0, 5.0, 1.0]


def _trace_with_steps(gvals, d=3):
    """h(t) = h(t-1) + g(t) e_0, so ||h(t) - h(t-1)|| = g(t)."""
    h = np.zeros((len(gvals), d))
    for t in range(1, len(gvals)):
        h[t] = h[t - 1]
        h[t, 0] += gvals[t]
    return h


def test_constant_steps_give_zero():
    g = epikv_g(_trace_with_steps([0.0] + [0.7] * 400))
    assert np.allclose(g[1:], 0.7)
    assert np.all(np.abs(rolling_z(g, 256, 1e-6)) < 1e-6)


def test_linear_ramp_closed_form():
    """For g(u) = a + b u over a full window of W values, the newest value sits
    b (W-1)/2 above the mean and sigma = b sqrt((W^2-1)/12), so
    z = sqrt(3 (W-1)/(W+1)) = 1.72530... at W = 256."""
    W = 256
    g = np.array([0.0] + [5.0 + 2.0 * u for u in range(1, 1000)])
    z = rolling_z(g, W, 1e-6)
    want = math.sqrt(3 * (W - 1) / (W + 1))
    assert want == pytest.approx(1.72530, abs=1e-5)
    assert np.allclose(z[W:], want, rtol=1e-8)
    assert z[0] == 0.0 and z[1] == 0.0                  # window {1}: sigma = 0
    assert z[2] == pytest.approx(1.0, abs=1e-6)         # window {1, 2}: one sigma above the mean


def test_affine_invariance_and_window_truncation():
    rng = np.random.default_rng(0)
    g = np.concatenate([[0.0], rng.gamma(2.0, 1.0, 700)])
    z = rolling_z(g, 64, 1e-9)
    z2 = rolling_z(3.5 * g + 11.0, 64, 1e-9)
    assert np.allclose(z[1:], z2[1:], atol=1e-6)
    t = 30                                              # warm-up: window is {1..t}
    u = g[1:t + 1]
    assert z[t] == pytest.approx((g[t] - u.mean()) / (u.std() + 1e-9), rel=1e-12)
    t = 500                                             # full window {t-63..t}
    u = g[t - 63:t + 1]
    assert z[t] == pytest.approx((g[t] - u.mean()) / (u.std() + 1e-9), rel=1e-12)


def test_score_is_difference_of_the_two_layers():
    rng = np.random.default_rng(1)
    a = np.cumsum(rng.standard_normal((300, 8)), axis=0)
    b = np.cumsum(rng.standard_normal((300, 8)), axis=0)
    s = epikv_score(a, b, 32, 1e-6)
    assert np.allclose(s, -epikv_score(b, a, 32, 1e-6))
    assert np.allclose(epikv_score(a, a, 32, 1e-6), 0.0)
    assert s[0] == 0.0


def test_rolling_mean_closed_forms():
    """EPIKV part 2's g_bar over the window {max(1, t-W+1) .. t}: for the ramp
    g(u) = a + b u the warm-up mean is a + b (t+1)/2 and the full-window mean
    a + b (t - (W-1)/2); a constant stays constant."""
    from oracle import rolling_mean
    W, a, b = 64, 5.0, 2.0
    g = np.array([0.0] + [a + b * u for u in range(1, 400)])
    m = rolling_mean(g, W)
    assert m[0] == 0.0
    for t in (1, 2, 30, W):
        assert m[t] == pytest.approx(a + b * (t + 1) / 2, rel=1e-14)
    for t in (W + 1, 200, 399):
        assert m[t] == pytest.approx(a + b * (t - (W - 1) / 2), rel=1e-14)
    assert np.allclose(rolling_mean(np.array([0.0] + [0.7] * 100), 16)[1:], 0.7)


def test_mean_form_score():
    from oracle import rolling_mean
    rng = np.random.default_rng(2)
    a = np.cumsum(rng.standard_normal((300, 8)), axis=0)
    b = np.cumsum(rng.standard_normal((300, 8)), axis=0)
    s = epikv_score(a, b, 32, 1e-6, form="mean")
    assert np.allclose(s, rolling_mean(epikv_g(a), 32) - rolling_mean(epikv_g(b), 32))
    assert np.allclose(s, -epikv_score(b, a, 32, 1e-6, form="mean"))
    # steps of constant size c in layer a and 2c in layer b: s = -c after t = 0
    ha = _trace_with_steps([0.0] + [0.5] * 100)
    hb = _trace_with_steps([0.0] + [1.0] * 100)
    sm = epikv_score(ha, hb, 16, 1e-6, form="mean")
    assert sm[0] == 0.0 and np.allclose(sm[1:], -0.5)
