"""Pins of the oracle's observation scores (logits, softmax, max aggregation)."""
import math

import numpy as np
import pytest
import torch

from oracle import segment_probabilities, segment_scores, layer_scores, visible_mask, rope, to_storage


def _brute(k, kpos, q, qpos, causal):
    """Dense masked attention through torch.softmax in float64."""
    logits = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(k.shape[1])
    if causal:
        mask = torch.from_numpy(kpos)[None, :] <= torch.from_numpy(qpos)[:, None]
        logits = logits.masked_fill(~mask, float("-inf"))
    return torch.softmax(logits, dim=1).numpy()


def test_probabilities_match_dense_softmax():
    rng = np.random.default_rng(0)
    for causal in (True, False):
        k = rng.standard_normal((37, 16)) * 2
        kpos = np.arange(37)
        q = rng.standard_normal((9, 16)) * 2
        qpos = np.array([30, 31, 32, 33, 34, 35, 36, 37, 37])
        p = segment_probabilities(k, kpos, q, qpos, causal)
        assert np.allclose(p, _brute(k, kpos, q, qpos, causal), rtol=1e-12, atol=1e-300)
        s = segment_scores(k, kpos, q, qpos, causal)
        assert np.allclose(s, _brute(k, kpos, q, qpos, causal).max(axis=0), rtol=1e-12)


def test_rows_sum_to_one_and_mask_is_causal():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((50, 8))
    kpos = np.arange(50)
    qpos = np.array([10, 25, 49, 60])
    p = segment_probabilities(k, kpos, rng.standard_normal((4, 8)), qpos)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-13)
    assert np.all(p[0, 11:] == 0) and np.all(p[0, :11] > 0)
    assert np.all(p[3] > 0)


def test_identical_keys_and_zero_query_give_uniform_rows():
    k = np.tile(np.random.default_rng(2).standard_normal(16), (20, 1))
    p = segment_probabilities(k, np.arange(20), np.random.default_rng(3).standard_normal((3, 16)),
                              np.array([4, 19, 19]))
    assert np.allclose(p[0, :5], 1 / 5) and np.allclose(p[1], 1 / 20)
    k2 = np.random.default_rng(4).standard_normal((20, 16))
    p2 = segment_probabilities(k2, np.arange(20), np.zeros((1, 16)), np.array([19]))
    assert np.allclose(p2, 1 / 20, rtol=1e-14)


def test_large_logits_do_not_overflow():
    k = np.array([[1.0, 0.0], [0.0, 1.0]]) * 100.0
    q = np.array([[100.0, 0.0]])
    p = segment_probabilities(k, np.arange(2), q, np.array([5]))
    # logits 100*100/sqrt2 and 0: second probability is exp(-7071.07) -> 0
    assert p[0, 0] == 1.0 and p[0, 1] == 0.0


def test_max_aggregation_properties():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((64, 16))
    q = rng.standard_normal((12, 16))
    qpos = rng.integers(40, 70, 12)
    p = segment_probabilities(k, np.arange(64), q, qpos)
    s = segment_scores(k, np.arange(64), q, qpos)
    assert np.all(s[None, :] >= p)                             # aggregate >= every query's score
    perm = rng.permutation(12)
    assert np.array_equal(segment_scores(k, np.arange(64), q[perm], qpos[perm]), s)
    one = segment_scores(k, np.arange(64), q[:1], qpos[:1])    # one query: exactly its row
    assert np.allclose(one, p[0], rtol=1e-13, atol=0)


def test_layer_scores_gqa_mapping_and_rotation():
    """Segment (b, g) is scored by query heads g*G .. g*G+G-1 only, rotated to q_pos."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d, n, no = 2, 4, 2, 16, 30, 3
    theta = 1e4
    k = to_storage(rng.standard_normal((B * Hkv * n, d)), "bf16")
    kpos = np.tile(np.arange(n), B * Hkv)
    seg_off = np.arange(B * Hkv) * n
    seg_len = np.full(B * Hkv, n)
    q = to_storage(rng.standard_normal((B, Hq, no, d)), "bf16")
    qpos = np.array([[28, 29, 30], [27, 29, 30]])
    out = layer_scores(k, kpos, seg_off, seg_len, q, qpos, np.array([no, 2]), Hkv, theta, "bf16")
    for b in range(B):
        nob = no if b == 0 else 2
        for g in range(Hkv):
            o = (b * Hkv + g) * n
            per_head = []
            for h in (2 * g, 2 * g + 1):
                qr = to_storage(rope(q[b, h, :nob], qpos[b, :nob], theta), "bf16")
                per_head.append(segment_probabilities(k[o:o + n], kpos[o:o + n], qr, qpos[b, :nob]))
            want = np.concatenate(per_head).max(axis=0)
            assert np.array_equal(out[o:o + n], want)


def test_visible_mask_shapes():
    m = visible_mask(np.arange(5), np.array([2, 4]))
    assert m.tolist() == [[True, True, True, False, False], [True] * 5]


def test_mean_aggregation_hand_example_and_row_sum_invariant():
    """Mean over observation rows (BeaconKV experiments, max vs mean ablation).
    Two keys with equal logits for row 0, and a row 1 at position 0 that sees
    only key 0: probabilities [0.5, 0.5] and [1, 0], so mean = [0.75, 0.25] and
    max = [1, 0.5]."""
    k = np.array([[1.0, 0.0], [1.0, 0.0]])
    q = np.array([[2.0, 0.0], [3.0, 0.0]])
    kpos, qpos = np.array([0, 1]), np.array([1, 0])
    assert np.allclose(segment_scores(k, kpos, q, qpos, True, "mean"), [0.75, 0.25], rtol=1e-15)
    assert np.allclose(segment_scores(k, kpos, q, qpos, True, "max"), [1.0, 0.5], rtol=1e-15)
    # each row's probabilities sum to 1 (0 for a row that sees nothing), so the
    # mean scores sum to (rows that see a key) / (all rows)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((40, 16))
    kpos = np.arange(40) + 10
    qpos = np.array([5, 12, 30, 49, 49, 60, 9])          # rows 0 and 6 see no key
    s = segment_scores(k, kpos, rng.standard_normal((7, 16)), qpos, True, "mean")
    assert s.sum() == pytest.approx(5 / 7, rel=1e-13)
    # one row: mean and max agree; mean never exceeds max
    q1 = rng.standard_normal((1, 16))
    assert np.allclose(segment_scores(k, kpos, q1, [60], True, "mean"), segment_scores(k, kpos, q1, [60]))
    q3 = rng.standard_normal((5, 16)) * 3
    assert np.all(segment_scores(k, kpos, q3, [45, 50, 60, 60, 60], True, "mean")
                  <= segment_scores(k, kpos, q3, [45, 50, 60, 60, 60]) + 1e-15)
    # and matches the dense softmax's column means
    brute = _brute(k, kpos, q3, np.array([45, 50, 60, 60, 60]), True).mean(axis=0)
    assert np.allclose(segment_scores(k, kpos, q3, [45, 50, 60, 60, 60], True, "mean"), brute, rtol=1e-12)


def test_empty_segment_has_no_scores():
    """A segment without keys scores nothing, and the layer's other segments
    score as they would alone: the softmax and the maximum run over no key."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 8))
    assert segment_scores(np.zeros((0, 8)), np.zeros(0, dtype=np.int64), q, np.full(2, 9)).shape == (0,)
    k = rng.standard_normal((5, 8))
    pos = np.arange(5)
    qo = np.broadcast_to(q, (3, 1, 2, 8)).copy()           # three requests, one head, the same two rows
    s = layer_scores(np.concatenate([k, k]), np.concatenate([pos, pos]), np.array([0, 5, 5]), np.array([5, 0, 5]),
                     qo, np.full((3, 2), 9), np.array([2, 2, 2]), 1, 1e4, "f64")
    assert np.array_equal(s[:5], s[5:]) and np.all(s > 0)
