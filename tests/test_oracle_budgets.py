"""Pins of the oracle's head entropy and budget allocation."""
import math

import numpy as np
import pytest

from oracle import normalized_entropy, waterfill, largest_remainder, head_budgets, layer_wave_budgets


def test_entropy_closed_forms():
    assert normalized_entropy(np.ones(100)) == pytest.approx(1.0, abs=1e-14)
    assert normalized_entropy(np.eye(1, 50)[0]) == 0.0
    assert normalized_entropy(np.array([1.0, 1.0, 0.0, 0.0])) == pytest.approx(0.5, abs=1e-15)
    # pi = (1/2, 1/4, 1/4): H = 1.5 ln 2, over ln 3
    assert normalized_entropy(np.array([2.0, 1.0, 1.0])) == pytest.approx(1.5 * math.log(2) / math.log(3), rel=1e-14)
    assert normalized_entropy(np.array([3.0, 3.0]) * 7) == pytest.approx(1.0)   # scale-free


def _bisect(total, w, lo, hi):
    """Independent solver: bisection on lam for sum(clip(lam w, lo_g, hi)) = total."""
    w, hi = np.asarray(w, float), np.asarray(hi, float)
    lo_g = np.minimum(lo, hi)
    a, b = 0.0, 1.0
    while np.clip(b * w, lo_g, hi).sum() < total:
        b *= 2
    for _ in range(200):
        m = 0.5 * (a + b)
        if np.clip(m * w, lo_g, hi).sum() < total:
            a = m
        else:
            b = m
    return np.clip(b * w, lo_g, hi)


def test_waterfill_hand_examples():
    assert np.allclose(waterfill(100, [1, 1, 2], 0, [1e9] * 3), [25, 25, 50])
    assert np.allclose(waterfill(100, [1, 1, 8], 20, [1e9] * 3), [20, 20, 60])
    assert np.allclose(waterfill(150, [1, 1, 8], 0, [100, 100, 40]), [55, 55, 40])
    assert np.allclose(waterfill(90, [0, 0, 0], 10, [100] * 3), [30, 30, 30])     # all-zero weights: equal
    assert np.allclose(waterfill(500, [1, 2], 0, [100, 100]), [100, 100])         # total >= sum(hi)
    with pytest.raises(ValueError):
        waterfill(100, [1, 1], 64, [1000, 1000])


def test_waterfill_weightless_heads_hand_examples():
    """Heads of weight 0 stay at their floor while a common factor can still
    meet the total; once every weighted head is at its cap, the rest of the
    total is split equally over the weightless heads (the limit of equal tiny
    weights).  ReasonAlloc, Core Mechanism: the layer total is kept."""
    # weighted heads below their caps: the weightless head keeps its floor
    assert np.allclose(waterfill(600, [0, 1, 1], 64, [1000, 1000, 1000]), [64, 268, 268])
    assert np.allclose(waterfill(300, [0, 2, 1], 50, [1000, 1000, 1000]), [50, 500 / 3, 250 / 3])
    # weighted heads capped: the weightless head takes what is left
    assert np.allclose(waterfill(600, [0, 0.5, 0.5], 64, [1000, 100, 100]), [400, 100, 100])
    # two weightless heads share the rest equally, one of them then capped
    assert np.allclose(waterfill(700, [0, 0, 1], 64, [500, 300, 100]), [300, 300, 100])
    assert np.allclose(waterfill(850, [0, 0, 1], 64, [500, 300, 100]), [450, 300, 100])
    # the boundary between the two regimes: weighted heads exactly at their caps
    assert np.allclose(waterfill(264, [0, 1, 1], 64, [1000, 100, 100]), [64, 100, 100])


def test_waterfill_weightless_heads_match_bisection():
    """Independent check of both regimes: bisection on the unmodified weights
    where a common factor meets the total (total <= sum of the weighted heads'
    caps + the weightless heads' floors), else bisection with every zero weight
    replaced by the same tiny weight (the limit the oracle's equal split of the
    rest stands for)."""
    rng = np.random.default_rng(5)
    n_split = 0
    for _ in range(300):
        G = int(rng.integers(2, 10))
        w = rng.random(G) ** 2 + 0.05
        zero = rng.random(G) < 0.4
        zero[int(rng.integers(G))] = True
        if zero.all():
            zero[0] = False
        w[zero] = 0.0
        hi = rng.integers(80, 3000, G).astype(float)
        lo = 64.0
        lo_g = np.minimum(lo, hi)
        total = float(rng.uniform(lo_g.sum(), hi.sum()))
        x = waterfill(total, w, lo, hi)
        assert abs(x.sum() - total) < 1e-6
        if total <= hi[~zero].sum() + lo_g[zero].sum():
            assert np.allclose(x, _bisect(total, w, lo, hi), rtol=1e-9, atol=1e-7)
            assert np.allclose(x[zero], lo_g[zero])
        else:
            n_split += 1
            eps = np.where(zero, 1e-12, w)
            assert np.allclose(x, _bisect(total, eps, lo, hi), rtol=1e-7, atol=1e-5)
            assert np.allclose(x[~zero], hi[~zero])
    assert n_split > 20


def test_waterfill_matches_bisection():
    rng = np.random.default_rng(0)
    for _ in range(300):
        G = int(rng.integers(1, 12))
        w = rng.random(G) ** 3
        w[rng.random(G) < 0.1] = 0.0
        hi = rng.integers(10, 3000, G).astype(float)
        lo = 64.0
        lo_sum = np.minimum(lo, hi).sum()
        total = float(rng.uniform(lo_sum, hi.sum() * 1.05))
        x = waterfill(total, w, lo, hi)
        assert abs(x.sum() - min(total, hi.sum())) < 1e-6
        assert np.all(x >= np.minimum(lo, hi) - 1e-9) and np.all(x <= hi + 1e-9)
        if np.all(w > 0) and total < hi.sum():
            assert np.allclose(x, _bisect(total, w, lo, hi), rtol=1e-9, atol=1e-7)


def test_largest_remainder_rule():
    assert largest_remainder(np.array([1.5, 1.5, 1.0]), 4).tolist() == [2, 1, 1]   # tie -> lower index
    assert largest_remainder(np.array([0.2, 0.7, 2.1]), 3).tolist() == [0, 1, 2]
    assert largest_remainder(np.array([3.0, 4.0]), 7).tolist() == [3, 4]
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = rng.random(8) * 100
        tot = int(round(x.sum()))
        x *= tot / x.sum()
        b = largest_remainder(x, tot)
        assert b.sum() == tot and np.all(np.abs(b - x) < 1)


def test_head_budgets_invariants():
    rng = np.random.default_rng(2)
    for _ in range(200):
        seg = rng.integers(100, 9000, 8)
        E = rng.random(8)
        total = int(rng.integers(8 * 64, 8 * 2200))
        b = head_budgets(E, seg, total, 64)
        assert b.sum() == min(total, seg.sum())
        assert np.all(b >= np.minimum(64, seg)) and np.all(b <= seg)
    eq = head_budgets(np.full(8, 0.7), np.full(8, 8000), 8 * 1001, 64)
    assert eq.max() - eq.min() <= 1 and eq.sum() == 8008


def test_layer_wave_budgets_shape():
    b = layer_wave_budgets(32, 16.0, 6.0, 32 * 1024, 64)
    assert b.sum() == 32768 and b.min() >= 64
    assert int(np.argmax(b)) == 16
    assert all(b[16 - k] == b[16 + k] for k in range(1, 16))      # symmetric about the centre
    assert all(b[i] <= b[i + 1] for i in range(16))                # rises to the peak
    l = np.arange(32)
    w = np.exp(-((l - 16.0) ** 2) / 72.0)
    x = _bisect(32768.0, w, 64.0, np.full(32, 1e9))
    assert np.all(np.abs(b - x) < 1)
    assert b[0] == 64                                              # raw share 62.7 < 64 is floored


def test_inverse_entropy_weights_favour_focused_heads():
    """ReasonAlloc, Key Concepts: low-entropy heads gain budget.  With weights
    1 - E = (0.9, 0.5, 0.1) and room everywhere the split is 180/100/20."""
    from oracle import head_weights
    E = np.array([0.1, 0.5, 0.9])
    assert np.allclose(head_weights(E, inverse=True), [0.9, 0.5, 0.1])
    assert np.array_equal(head_weights(E), E)
    b = head_budgets(head_weights(E, inverse=True), [1000, 1000, 1000], 300, 0)
    assert b.tolist() == [180, 100, 20]
    b2 = head_budgets(head_weights(E), [1000, 1000, 1000], 300, 0)
    assert b2.tolist() == [20, 100, 180]
