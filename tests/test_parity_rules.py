"""CPU checks of the comparison rules themselves: a plausible mistake in a
GPU result must fail them (a budget rounded the wrong way, a swapped kept slot
far from the cut)."""
import numpy as np

import oracle
from tests.parity import budgets_match, kept_matches


def test_budgets_rule_accepts_exact_and_near_ties_only():
    n = np.array([4000, 4000, 4000, 4000])
    E = np.array([0.31, 0.23, 0.19, 0.27])
    total = 4001
    want = oracle.head_budgets(oracle.head_weights(E), n, total, 64)
    assert want.tolist() == [1241, 920, 760, 1080]        # shares 1240.31 920.23 760.19 1080.27
    assert budgets_match(want, E, E, n, total, 64)[0]
    # the extra token at the second-largest remainder (0.27 vs 0.31): rejected
    assert not budgets_match(np.array([1240, 920, 760, 1081]), E, E, n, total, 64)[0]
    # a wrong sum, a budget above the length or below the floor: rejected
    assert not budgets_match(want + np.array([1, 0, 0, 0]), E, E, n, total, 64)[0]
    assert not budgets_match(np.array([4001, 0, 0, 0]), E, E, n, total, 64)[0]
    assert not budgets_match(np.array([1241 + 960 - 63, 63, 760, 1080 + 897]), E, E, n, total, 64)[0]


def test_budgets_rule_allows_a_swap_at_a_true_tie():
    # two heads with equal weights and shares x.5: the rounding of the two is a tie
    n = np.array([1000, 1000, 1000])
    E = np.array([0.5, 0.25, 0.25])
    total = 401
    x = oracle.waterfill(float(total), E, 0.0, n.astype(float))
    assert np.allclose(x, [200.5, 100.25, 100.25])
    want = oracle.largest_remainder(x, total)
    assert want.tolist() == [201, 100, 100]
    assert budgets_match(want, E, E, n, total, 0)[0]
    # heads 1 and 2 tie with each other, not with head 0 (0.5 vs 0.25): moving a
    # token from 0 to 1 is an error
    assert not budgets_match(np.array([200, 101, 100]), E, E, n, total, 0)[0]
    E2 = np.array([0.5, 0.5, 0.5])
    x2 = oracle.waterfill(400.0, E2, 0.0, n.astype(float))
    w2 = oracle.largest_remainder(x2, 400)
    assert w2.tolist() == [134, 133, 133]
    assert budgets_match(np.array([133, 134, 133]), E2, E2, n, 400, 0)[0]   # all three tie at 1/3


def test_budgets_rule_widens_with_the_entropy_difference():
    n = np.array([3000, 3000])
    e_orc = np.array([0.4, 0.6])
    e_gpu = e_orc * (1 + np.array([2e-4, -2e-4]))
    total = 2001
    ok, _ = budgets_match(oracle.head_budgets(oracle.head_weights(e_gpu), n, total, 0), e_gpu, e_orc, n, total, 0)
    assert ok


def test_kept_rule_rejects_a_swap_far_from_the_cut():
    rng = np.random.default_rng(3)
    s = rng.random(200) + 1.0
    want = oracle.select_kept(s, 200, 120, 4, 16)
    assert kept_matches(want, s, 200, 120, 4, 16)[0]
    dropped = np.setdiff1d(np.arange(4, 184), want)
    worst = dropped[np.argmin(s[dropped])]
    bad = np.sort(np.concatenate([want[want != want[np.argmax(s[want] * (want >= 4) * (want < 184))]], [worst]]))
    assert not kept_matches(bad, s, 200, 120, 4, 16)[0]
