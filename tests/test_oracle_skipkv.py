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
