"""Pins of the oracle's sentence-redundancy score (SkipKV §4.1)."""
import math

import numpy as np
import pytest

from oracle import pss_later_max, sentence_means, skipkv_token_scores


def test_sentence_means_hand_example():
    h = np.array([[1.0, 0.0], [3.0, 0.0], [0.0, 2.0], [0.0, 4.0], [2.0, 2.0], [5.0, 5.0]])
    e = sentence_means(h, [0, 2, 4, 5])
    assert e.tolist() == [[2.0, 0.0], [0.0, 3.0], [2.0, 2.0]]
    assert sentence_means(h, [0, 2, 2, 6]).tolist() == [[2.0, 0.0], [0.0, 0.0], [1.75, 3.25]]   # empty sentence


def test_pss_closed_forms():
    e = np.array([[2.0, 0.0], [0.0, 3.0], [2.0, 2.0], [-1.0, 0.0]])
    p = pss_later_max(e)
    # 0 vs later: cos 0, 1/sqrt2, -1 -> 1/sqrt2; 1 vs later: 1/sqrt2, 0; 2 vs 3: -1/sqrt2; 3: none
    assert p[0] == pytest.approx(1 / math.sqrt(2), rel=1e-15)
    assert p[1] == pytest.approx(1 / math.sqrt(2), rel=1e-15)
    assert p[2] == pytest.approx(-1 / math.sqrt(2), rel=1e-15)
    assert p[3] == -1.0
    # scale invariance; an exact repeat of a later sentence gives 1
    assert np.allclose(pss_later_max(e * np.array([[3.0], [0.5], [7.0], [2.0]])), p, rtol=1e-14)
    assert pss_later_max(np.array([[1.0, 2.0, 3.0], [0.0, 1.0, 0.0], [2.0, 4.0, 6.0]]))[0] == pytest.approx(1.0)
    assert pss_later_max(np.array([[0.0, 0.0], [1.0, 0.0]]))[0] == 0.0          # zero mean


def test_token_scores_follow_their_sentence():
    starts = [0, 3, 5, 9]
    sc = skipkv_token_scores(np.array([0.97, -0.2, 0.5]), starts, 12)
    assert sc[:3] == pytest.approx([0.03] * 3)
    assert sc[3:5].tolist() == [1.0, 1.0]          # negative similarity counts as 0
    assert sc[5:9].tolist() == [0.5] * 4
    assert sc[9:].tolist() == [1.0] * 3             # after the last complete sentence


def test_token_scores_end_to_end_hand_example():
    """Hidden states -> sentence means -> later-sentence PSS -> token scores, by hand:
    sentences A = tokens 0-1 (mean (1, 0)), B = tokens 2-4 (mean (0, 2)),
    C = tokens 5-6 (mean (3, 3)), D = tokens 7-8 (mean (2, 0)); tokens 9-10
    follow the last complete sentence.  A's later sentences: cos(A, B) = 0,
    cos(A, C) = 1/sqrt2, cos(A, D) = 1 -> A repeats D and scores 0.  B: cos(B, C)
    = 1/sqrt2, cos(B, D) = 0 -> 1 - 1/sqrt2.  C: cos(C, D) = 1/sqrt2 -> 1 - 1/sqrt2.
    D has no later sentence -> 1."""
    h = np.array([[1.0, 0.0], [1.0, 0.0],
                  [0.0, 1.0], [0.0, 2.0], [0.0, 3.0],
                  [2.0, 4.0], [4.0, 2.0],
                  [1.0, 0.0], [3.0, 0.0],
                  [9.0, -9.0], [-5.0, 1.0]])
    starts = [0, 2, 5, 7, 9]
    e = sentence_means(h, starts)
    assert e.tolist() == [[1.0, 0.0], [0.0, 2.0], [3.0, 3.0], [2.0, 0.0]]
    sc = skipkv_token_scores(pss_later_max(e), starts, len(h))
    r = 1.0 - 1.0 / math.sqrt(2.0)
    assert sc[0:2] == pytest.approx([0.0, 0.0], abs=1e-15)
    assert sc[2:5] == pytest.approx([r] * 3, rel=1e-14)
    assert sc[5:7] == pytest.approx([r] * 2, rel=1e-14)
    assert sc[7:].tolist() == [1.0] * 4


def test_token_scores_invariants():
    """On random sentences: scores lie in [0, 1], are shared by a sentence's
    tokens, are 1 for the last sentence and after it, do not change when the
    hidden dimensions are permuted or a sentence's tokens are scaled by one
    positive factor, and a sentence whose mean equals a later one's scores 0."""
    rng = np.random.default_rng(7)
    T, d = 60, 8
    h = rng.standard_normal((T, d))
    starts = [0, 4, 11, 12, 20, 33, 41, 52]
    sc = skipkv_token_scores(pss_later_max(sentence_means(h, starts)), starts, T)
    assert np.all((sc >= 0.0) & (sc <= 1.0))
    for a, b in zip(starts[:-1], starts[1:]):
        assert np.all(sc[a:b] == sc[a])
    assert np.all(sc[starts[-2]:] == 1.0)
    perm = rng.permutation(d)
    assert np.allclose(skipkv_token_scores(pss_later_max(sentence_means(h[:, perm], starts)), starts, T), sc,
                       rtol=0, atol=1e-12)
    h2 = h.copy()
    h2[20:33] *= 3.5                                     # one sentence's tokens scaled: its mean scales, cosines do not
    assert np.allclose(skipkv_token_scores(pss_later_max(sentence_means(h2, starts)), starts, T), sc,
                       rtol=0, atol=1e-12)
    h3 = h.copy()
    h3[33:41] = h3[4:11].mean(axis=0)                    # sentence 5's mean equals sentence 1's -> sentence 1 repeats it
    sc3 = skipkv_token_scores(pss_later_max(sentence_means(h3, starts)), starts, T)
    assert sc3[4:11] == pytest.approx([0.0] * 7, abs=1e-12)
