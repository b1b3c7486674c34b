"""Pins of the oracle's selection, compaction and farthest-point sampling."""
import itertools
import math

import numpy as np
import pytest

from oracle import select_kept, compact_rows, fps, fps_acceptable


def _beats(s32, a, b):
    return (s32[a] > s32[b]) or (s32[a] == s32[b] and a < b)


def test_select_brute_force_order():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(20, 60))
        P, R = 4, 16
        budget = int(rng.integers(P + R, n + 3))
        s = rng.random(n) * (10.0 ** -rng.integers(0, 8))
        s[rng.random(n) < 0.3] = s[0]                          # plenty of exact ties
        kept = select_kept(s, n, budget, P, R)
        assert len(kept) == min(budget, n)
        assert np.all(np.diff(kept) > 0)
        ks = set(kept.tolist())
        assert set(range(P)) <= ks and set(range(n - R, n)) <= ks
        cand = range(P, n - R)
        for a in cand:
            for b in cand:
                if a in ks and b not in ks:
                    assert _beats(s, a, b)


def test_select_hand_example_ties_to_lower_slot():
    s = np.array([0, 0, 0, 0, .5, .9, .5, .5, .1, .5, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0], float)
    n = len(s)                      # candidates are slots 4..9
    kept = select_kept(s, n, 4 + 16 + 3, 4, 16)
    assert kept.tolist() == [0, 1, 2, 3, 4, 5, 6] + list(range(10, 26))


def test_select_edge_cases():
    s = np.arange(30.0)
    assert select_kept(s, 30, 30, 4, 16).tolist() == list(range(30))
    assert select_kept(s, 30, 99, 4, 16).tolist() == list(range(30))
    assert select_kept(s, 10, 25, 4, 16).tolist() == list(range(10))    # short segment keeps all
    for n, budget in ((30, 19), (10, 5)):                                # budget below P + R
        with pytest.raises(ValueError):
            select_kept(s, n, budget, 4, 16)
    assert select_kept(s, 30, 20, 4, 16).tolist() == list(range(4)) + list(range(14, 30))


def test_compact_is_a_stable_gather():
    rows = np.arange(40).reshape(20, 2)
    kept = np.array([0, 3, 4, 19])
    assert compact_rows(rows, kept).tolist() == [[0, 1], [6, 7], [8, 9], [38, 39]]


def _angle_points(deg):
    return np.array([[math.cos(math.radians(a)), math.sin(math.radians(a))] for a in deg])


def test_fps_hand_example_on_the_circle():
    # angles 0, 10, 90, 180, 100 degrees.  From row 0 the farthest is 180 (index 3);
    # then 90 (distance 1 to both picks) beats 100 (min(1-cos100, 1-cos80) = 0.826).
    X = _angle_points([0, 10, 90, 180, 100])
    assert fps(X, 3).tolist() == [0, 3, 2]
    assert fps(X, 5).tolist()[:3] == [0, 3, 2]


def _fps_from_scratch(X, k):
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    picks = [0]
    for _ in range(k - 1):
        best, arg = -1.0, -1
        for r in range(len(X)):
            if r in picks:
                continue
            dmin = min(float(1.0 - U[r] @ U[p]) for p in picks)
            if dmin > best:
                best, arg = dmin, r
        picks.append(arg)
    return picks


def test_fps_incremental_equals_recompute():
    rng = np.random.default_rng(1)
    for _ in range(30):
        X = rng.standard_normal((20, 12))
        assert fps(X, 10).tolist() == _fps_from_scratch(X, 10)


def test_fps_properties():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((32, 128))
    p = fps(X, 16)
    assert len(set(p.tolist())) == 16 and p[0] == 0
    assert np.array_equal(fps(2.0 * X, 16), p)                 # scale-free (exact power of two)
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    radii = [min(1 - U[r] @ U[q] for q in p[:i]) for i, r in enumerate(p) if i > 0]
    assert all(radii[i] >= radii[i + 1] - 1e-12 for i in range(len(radii) - 1))
    ok, _ = fps_acceptable(X, p, 2e-3)
    assert ok
    bad = p.copy()
    # replace the last pick with the unpicked row nearest to the picked set
    rest = [r for r in range(32) if r not in set(p.tolist())]
    dmin = [min(1 - U[r] @ U[q] for q in p[:-1]) for r in rest]
    bad[-1] = rest[int(np.argmin(dmin))]
    assert not fps_acceptable(X, bad, 2e-3)[0]


def test_fps_gonzalez_two_approximation_exhaustive():
    """FPS (Gonzalez 1985) is a 2-approximation of k-center in any metric; the
    angle between vectors is a metric and 1 - cos is monotone in it, so the FPS
    picks' angular covering radius is at most twice the optimum over all
    C(16, 8) = 12,870 subsets."""
    rng = np.random.default_rng(3)
    for trial in range(3):
        centers = rng.standard_normal((3, 64))
        X = centers[rng.integers(0, 3, 16)] + 0.5 * rng.standard_normal((16, 64))
        U = X / np.linalg.norm(X, axis=1, keepdims=True)
        ang = np.arccos(np.clip(U @ U.T, -1, 1))
        p = fps(X, 8)
        r_fps = ang[:, p].min(axis=1).max()
        best = min(ang[:, list(c)].min(axis=1).max() for c in itertools.combinations(range(16), 8))
        assert r_fps <= 2 * best + 1e-12


def test_fps_duplicates_and_zero_rows():
    X = np.zeros((6, 4))
    X[:, 0] = 1.0
    X[5] = 0.0                                     # zero norm row: treated as distance 1 from all
    p = fps(X, 3)
    assert p.tolist() == [0, 5, 1]


def test_hole_fill_hand_example_and_invariants():
    """n = 10, survivors {0, 2, 3, 5, 7, 9}: K = 6, holes 1 and 4 take movers 7
    and 9."""
    from oracle import hole_fill
    assert hole_fill([0, 2, 3, 5, 7, 9], 10).tolist() == [0, 7, 2, 3, 9, 5]
    assert hole_fill(list(range(6)), 10).tolist() == list(range(6))      # nothing to move
    assert hole_fill([4, 5, 6, 7], 8).tolist() == [4, 5, 6, 7]           # every survivor moves
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(1, 80))
        K = int(rng.integers(0, n + 1))
        kept = np.sort(rng.choice(n, K, replace=False))
        src = hole_fill(kept, n)
        assert sorted(src.tolist()) == kept.tolist()                      # a permutation of the survivors
        stay = kept[kept < K]
        assert np.all(src[stay] == stay)                                  # survivors below K do not move
        moved = int((src != np.arange(K)).sum())
        assert moved == int((kept >= K).sum()) <= min(K, n - K)
        # the movers fill the holes in ascending order of both
        holes = np.setdiff1d(np.arange(K), kept)
        assert np.all(np.diff(src[holes]) > 0) and np.all(src[holes] >= K)
