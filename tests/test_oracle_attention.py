"""Pins of the oracle's decode attention over a compacted cache."""
import math

import numpy as np
import pytest
import torch

from oracle import decode_attention, hole_fill


def test_single_row_and_uniform_logits():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 8))
    out, lse = decode_attention(rng.standard_normal((1, 8)), v, rng.standard_normal((3, 8)))
    assert np.allclose(out, np.repeat(v, 3, axis=0), rtol=1e-15)
    k, v = rng.standard_normal((20, 8)), rng.standard_normal((20, 8))
    out, lse = decode_attention(k, v, np.zeros((2, 8)))         # zero query: uniform weights
    assert np.allclose(out, v.mean(axis=0), rtol=1e-13)
    assert np.allclose(lse, math.log(20), rtol=1e-15)


def test_two_rows_closed_form():
    """Logits a and b: weight of row 0 = 1 / (1 + e^(b - a))."""
    k = np.array([[2.0, 0.0], [0.0, 1.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    q = np.array([[1.5, -0.5]])
    a, b = 3.0 / math.sqrt(2), -0.5 / math.sqrt(2)
    w0 = 1.0 / (1.0 + math.exp(b - a))
    out, lse = decode_attention(k, v, q)
    assert out[0].tolist() == pytest.approx([w0, 1 - w0], rel=1e-14)
    assert lse[0] == pytest.approx(math.log(math.exp(a) + math.exp(b)), rel=1e-14)


def test_dense_softmax_and_row_order_invariance():
    rng = np.random.default_rng(1)
    k, v, q = rng.standard_normal((300, 64)) * 2, rng.standard_normal((300, 64)), rng.standard_normal((4, 64)) * 2
    out, lse = decode_attention(k, v, q)
    p = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(k).T / 8.0, dim=1)
    assert np.allclose(out, (p @ torch.from_numpy(v)).numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(q) @ torch.from_numpy(k).T / 8.0, dim=1).numpy())
    # the in-place (hole-filled) layout of a kept set attends exactly like the ordered one
    kept = np.sort(rng.choice(300, 220, replace=False))
    src = hole_fill(kept, 300)
    o1, l1 = decode_attention(k[kept], v[kept], q)
    o2, l2 = decode_attention(k[src], v[src], q)
    assert np.allclose(o1, o2, rtol=1e-13) and np.allclose(l1, l2, rtol=1e-14)
    # linear in V
    o3, _ = decode_attention(k, 2.0 * v + 1.0, q)
    assert np.allclose(o3, 2.0 * out + 1.0, rtol=1e-13)
