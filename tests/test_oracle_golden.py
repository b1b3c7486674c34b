"""The oracle against its stored worked example (tests/golden/): fixed
integer-pattern inputs, every output recomputed and compared — integers
exactly, stored fp32 values to one ulp, float64 results to 1e-12 — so that
any change of the oracle's arithmetic is caught here.  The stored values are
also checked against what the method fixes about them on their own."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_golden  # noqa: E402

STORED = json.load(open(os.path.join(HERE, "golden", "oracle_worked_example.json")))["outputs"]


def _v(name):
    return np.asarray(STORED[name]["value"])


def test_every_output_cites_its_passage():
    assert all(o["cite"] for o in STORED.values())


def test_oracle_reproduces_the_worked_example():
    got = make_golden.compute(make_golden.inputs())
    assert set(got) == set(STORED)
    for name in ("kept", "compacted_pos", "head_budgets", "layer_wave_budgets", "fps_picks"):
        np.testing.assert_array_equal(np.asarray(got[name]), _v(name), err_msg=name)
    for name in ("k_cache", "q_rot"):
        np.testing.assert_allclose(got[name], _v(name), rtol=1.2e-7, atol=0, err_msg=name)
    for name in ("scores", "entropy"):
        np.testing.assert_allclose(got[name], _v(name), rtol=1e-12, atol=0, err_msg=name)


def test_stored_values_satisfy_the_method():
    x = make_golden.inputs()
    kept, scores = _v("kept"), _v("scores")
    n, P, R, K = x["n"], x["n_prefix"], x["n_recent"], x["budget"]
    assert len(kept) == K and np.all(np.diff(kept) > 0)
    assert set(range(P)) | set(range(n - R, n)) <= set(kept.tolist())
    cand = [j for j in range(P, n - R)]
    chosen = [j for j in cand if j in set(kept.tolist())]
    evicted = [j for j in cand if j not in set(kept.tolist())]
    assert min(scores[chosen]) >= max(scores[evicted])
    np.testing.assert_array_equal(_v("compacted_pos"), np.asarray(x["key_pos"])[kept])
    assert np.all((scores > 0) & (scores <= 1)) and 0 < float(_v("entropy")) <= 1
    hb = _v("head_budgets")
    assert hb.sum() == 1000 and hb.min() >= 64 and np.all(hb <= [500, 100, 800, 300])
    lw = _v("layer_wave_budgets")
    assert lw.sum() == 32 * 1024 and lw.min() == 64 and int(np.argmax(lw)) == 16
    picks = _v("fps_picks")
    assert picks[0] == 0 and len(set(picks.tolist())) == x["fps_keep"]
