"""Pins of the oracle's storage rounding and rotary embedding."""
import math

import numpy as np
import pytest
import torch

from oracle import round_bf16, to_storage, rope



def test_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38 / 4])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_direct_rounding_avoids_double_rounding():
    # 1 + 2^-8 is the midpoint between the bf16 values 1 and 1 + 2^-7; a value a
    # hair above it rounds to float32 *onto* the midpoint, but must round up.
    above = 1.0 + 2.0 ** -8 + 2.0 ** -30
    below = 1.0 + 2.0 ** -8 - 2.0 ** -30
    assert round_bf16(np.array([above]))[0] == 1.0 + 2.0 ** -7
    assert round_bf16(np.array([below]))[0] == 1.0
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0             # tie -> even
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6   # tie -> even (up)
    assert round_bf16(np.array([-above]))[0] == -(1.0 + 2.0 ** -7)


def test_bf16_rejects_non_finite():
    with pytest.raises(ValueError):
        round_bf16(np.array([np.nan]))


def test_to_storage_f32():
    assert to_storage(np.array([1.0 + 2.0 ** -30]), "f32")[0] == 1.0


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((5, 64))
    assert np.array_equal(rope(x, np.zeros(5), 1e4), x)


def test_rope_two_dims_is_plane_rotation():
    # d = 2: a single pair with frequency theta^0 = 1, angle = p radians.
    for p in (1, 2, 7, 100):
        out = rope(np.array([1.0, 0.0]), p, 1e4)
        assert np.allclose(out, [math.cos(p), math.sin(p)], atol=1e-15)
        out = rope(np.array([0.0, 1.0]), p, 1e4)
        assert np.allclose(out, [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_half_split_pairing_and_frequencies():
    # d = 8, theta = 1e4: pair i couples dims (i, i + 4) with frequency 1e4^(-i/4).
    d, theta, p = 8, 1e4, 3
    for i in range(4):
        e = np.zeros(d)
        e[i] = 1.0
        out = rope(e, p, theta)
        f = theta ** (-i / 4)
        want = np.zeros(d)
        want[i] = math.cos(p * f)
        want[i + 4] = math.sin(p * f)
        assert np.allclose(out, want, atol=1e-15), i


def test_rope_preserves_norm_and_composes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 128))
    pos = rng.integers(0, 70000, 7)
    y = rope(x, pos, 1e6)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(rope(rope(x, pos, 1e6), 11, 1e6), rope(x, pos + 11, 1e6), atol=1e-10)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = rope(q, 900, 5e5) @ rope(k, 37, 5e5)
    for shift in (1, 100, 30000):
        assert abs(rope(q, 900 + shift, 5e5) @ rope(k, 37 + shift, 5e5) - base) < 1e-9
