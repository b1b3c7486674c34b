"""The one-call eviction trigger (kv_evict_score_select_compact) against the
oracle and against the two-call form (kv_evict_score, kv_evict_select_compact).

Cases span several 1024-key chunks with ragged tails, both head sizes, the
single-kernel path and the two-call fallback (fp32 caches, segments longer
than the on-chip selection, a forced VALU scorer), per-segment budgets with
the degenerate ones (K >= n, K below the protected slots, K above the output
capacity), repeated calls on the same workspace, and the report of a segment
whose work-groups did not meet within the barrier's poll bound."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
from tests.gpu_side import alloc_out, cache_of, device_layer, obs_of, score_layer, score_select_compact, \
    select_compact
from tests.oracle_side import oracle_cache_keys, oracle_layer_scores
from tests.parity import assert_scores_close, kept_matches
from workloads import get_workload, make_layer

pytestmark = pytest.mark.gpu

CASES = {
    # single-kernel path
    "qwen3-4b-1l": (get_workload("qwen3-4b-1l"), 1792),
    "llama-ragged": (get_workload("r1-llama-8b").scaled(batch=3, len_lo=700, len_hi=3300, n_layers=1), 640),
    "long-9216": (get_workload("long-65k").scaled(batch=1, len_lo=9216, len_hi=9216), 2048),
    "d64-bf16": (get_workload("tiny-f32").scaled(dtype="bf16", batch=3, len_lo=1500, len_hi=5120), 1000),
    "qwen-short": (get_workload("qwen3-4b-1l").scaled(batch=2, len_lo=333, len_hi=333), 300),
    "d64-long": (get_workload("tiny-f32").scaled(dtype="bf16", batch=1, len_lo=6000, len_hi=8704), 3000),
    "non-causal": (get_workload("qwen3-4b-1l").scaled(batch=2, len_lo=500, len_hi=900, causal=0), 480),
    # two-call fallback
    "tiny-f32": (get_workload("tiny-f32"), 448),
    "long-9217": (get_workload("long-65k").scaled(batch=1, len_lo=9217, len_hi=9500), 2048),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


_cache = {}


def _case(name):
    if name not in _cache:
        w, budget = CASES[name]
        L = make_layer(w, 0)
        D = device_layer(L, w)
        _cache[name] = (w, budget, L, D, oracle_layer_scores(L, w, oracle_cache_keys(L, w)))
    return _cache[name]


def _ints(t, w):
    return t.view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()


def _check_segments(w, L, D, out, s_orc, budgets):
    """Every segment against the oracle: length, kept slots (tie band allowed),
    and a byte-exact gather of the kept rows."""
    kept, seg_len = out["kept"].cpu().numpy(), out["seg_len"].cpu().numpy()
    k_in, v_in, k_out, v_out = _ints(D["k"], w), _ints(D["v"], w), _ints(out["k"], w), _ints(out["v"], w)
    pos_in, pos_out = D["pos"].cpu().numpy(), out["pos"].cpu().numpy()
    cap = out["cap"]
    for s in range(len(L["seg_len"])):
        o, n, K = int(L["seg_off"][s]), int(L["seg_len"][s]), int(budgets[s])
        if K < n and K < w.n_prefix + w.n_recent or min(K, n) > cap:
            assert seg_len[s] == -1, (s, seg_len[s])
            continue
        m = min(K, n)
        assert seg_len[s] == m, (s, seg_len[s], m)
        oo = s * cap
        ks = kept[oo:oo + m]
        ok, _, msg = kept_matches(ks, s_orc[o:o + n], n, K, w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
        assert np.array_equal(k_out[oo:oo + m], k_in[o + ks])
        assert np.array_equal(v_out[oo:oo + m], v_in[o + ks])
        assert np.array_equal(pos_out[oo:oo + m], pos_in[o + ks])


@pytest.mark.parametrize("name", list(CASES))
def test_one_call_trigger_matches_oracle(name):
    w, budget, L, D, s_orc = _case(name)
    out = alloc_out(D, w, budget)
    scores = score_select_compact(D, w, out, uniform=budget)
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy(), s_orc, what=f"{name} scores")
    _check_segments(w, L, D, out, s_orc, [budget] * len(L["seg_len"]))


@pytest.mark.parametrize("name", ["qwen3-4b-1l", "llama-ragged", "d64-bf16"])
def test_one_call_trigger_agrees_with_two_calls(name):
    """Same kept rows as score + select_compact wherever the two score vectors
    order the candidates alike; scores within fp32 rounding of each other."""
    w, budget, L, D, s_orc = _case(name)
    out1 = alloc_out(D, w, budget)
    s1 = score_select_compact(D, w, out1, uniform=budget)
    s2, _ = score_layer(D, w)
    out2 = alloc_out(D, w, budget)
    select_compact(D, w, s2, out2, uniform=budget)
    torch.cuda.synchronize()
    a, b = s1.cpu().numpy(), s2.cpu().numpy()
    assert_scores_close(a, b, rtol=2e-5, what="one-call vs two-call scores")
    assert torch.equal(out1["seg_len"], out2["seg_len"])
    k1, k2 = out1["kept"].cpu().numpy(), out2["kept"].cpu().numpy()
    cap = out1["cap"]
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        m = min(budget, n)
        same = np.array_equal(k1[s * cap:s * cap + m], k2[s * cap:s * cap + m])
        if not same:   # only candidates tied within rounding may swap
            ok, _, msg = kept_matches(k1[s * cap:s * cap + m], b[o:o + n].astype(np.float64), n, budget,
                                      w.n_prefix, w.n_recent, rtol=2e-5)
            assert ok, msg


def test_per_segment_budgets_and_degenerate_segments():
    w, _, L, D, s_orc = _case("llama-ragged")
    S = len(L["seg_len"])
    lens = [int(x) for x in L["seg_len"]]
    cap = 1500
    rng = np.random.default_rng(11)
    bud = rng.integers(w.n_prefix + w.n_recent, cap + 1, size=S)
    bud[0] = lens[0]             # keep everything (K == n) ... if it fits
    bud[1] = lens[1] + 50        # K > n: every row kept
    bud[2] = w.n_prefix + w.n_recent - 1   # below the protected slots: rejected
    bud[3] = w.n_prefix + w.n_recent       # exactly the protected slots
    bud[4] = cap + 1             # above the output capacity: rejected unless n <= cap
    bud[5] = 0                   # rejected (n > 0)
    budget = torch.tensor(bud, dtype=torch.int32, device="cuda")
    out = alloc_out(D, w, cap)
    score_select_compact(D, w, out, budget=budget)
    torch.cuda.synchronize()
    _check_segments(w, L, D, out, s_orc, bud)


def test_without_kept_index_and_repeated_calls():
    """kept_idx omitted gives the same output cache; a second call on the same
    workspace (queue and arrival counters re-zeroed on the stream) repeats it."""
    w, budget, L, D, s_orc = _case("llama-ragged")
    out1 = alloc_out(D, w, budget)
    score_select_compact(D, w, out1, uniform=budget)
    out2 = alloc_out(D, w, budget)
    cin, obs = cache_of(D, w), obs_of(D, w)
    cout = kv.make_cache(out2["k"], out2["v"], out2["pos"], out2["seg_off"], out2["seg_len"], w.n_kv_heads, budget)
    nbytes = kv.kv_evict_score_select_compact_workspace(cin, obs, cout, False)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    scores = torch.empty(D["k"].shape[0], dtype=torch.float32, device="cuda")
    for _ in range(2):
        for t in (out2["k"], out2["v"]):
            t.zero_()
        kv.kv_evict_score_select_compact(cin, obs, scores, None, w.n_prefix, w.n_recent, cout, uniform_budget=budget,
                                         ws=ws)
        torch.cuda.synchronize()
        for key in ("k", "v", "pos", "seg_len"):
            assert torch.equal(out1[key], out2[key]), key


def test_segments_with_bad_metadata_are_rejected():
    """A segment longer than max_seg_len, or reaching past the cache, gets
    seg_len -1 and no rows; the other segments are unaffected."""
    w, budget, L, D, s_orc = _case("qwen-short")
    D2 = dict(D)
    D2["seg_len"] = D["seg_len"].clone()
    D2["seg_len"][1] = D["max_len"] + 1
    D2["seg_off"] = D["seg_off"].clone()
    D2["seg_off"][3] = D["k"].shape[0] - 10
    out = alloc_out(D2, w, budget)
    score_select_compact(D2, w, out, uniform=budget)
    torch.cuda.synchronize()
    lens = out["seg_len"].cpu().numpy()
    assert lens[1] == -1 and lens[3] == -1
    assert torch.all(out["kept"][budget:2 * budget] == -5)
    good = [s for s in range(len(lens)) if s not in (1, 3)]
    kept = out["kept"].cpu().numpy()
    for s in good:
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        assert lens[s] == min(budget, n)
        ok, _, msg = kept_matches(kept[s * budget:s * budget + lens[s]], s_orc[o:o + n], n, budget, w.n_prefix,
                                  w.n_recent)
        assert ok, msg


def test_one_call_rejects_bad_arguments_before_launch():
    w, budget, L, D, _ = _case("qwen-short")
    out = alloc_out(D, w, budget)
    cin, obs = cache_of(D, w), obs_of(D, w)
    scores = torch.empty(D["k"].shape[0], dtype=torch.float32, device="cuda")
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, budget)
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact(cin, obs, scores, None, 4, 16, cout, uniform_budget=19)
    assert ei.value.name == "KVE_EBUDGET"
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact(cin, obs, scores, None, 4, 16, cout, uniform_budget=budget + 1)
    assert ei.value.name == "KVE_EBUDGET"
    # scores over the output keys
    bad = out["k"].view(torch.float32).view(-1)[:D["k"].shape[0]]
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact(cin, obs, bad, None, 4, 16, cout, uniform_budget=budget)
    assert ei.value.name == "KVE_EALIAS"
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact(cin, obs, scores, None, 4, 16, cout, uniform_budget=budget,
                                         ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "KVE_EWORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(out["seg_len"] == -9)   # nothing ran


def test_forced_valu_scorer_takes_the_two_call_path(kve_overrides):
    kve_overrides(score_impl="valu")
    w, budget, L, D, s_orc = _case("qwen-short")
    out = alloc_out(D, w, budget)
    scores = score_select_compact(D, w, out, uniform=budget)
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy(), s_orc)
    _check_segments(w, L, D, out, s_orc, [budget] * len(L["seg_len"]))


def test_barrier_timeout_reports_failed_segments(kve_overrides):
    """With the segment barrier's poll bound forced down to one poll (the
    failure handling path, driven from the host), a segment whose work-groups
    do not all arrive at once is reported failed (seg_len -1) rather than
    selected from partial row statistics; every kernel exits, and a segment
    that did meet is exact.  A later call with the default bound is whole."""
    w, budget, L, D, s_orc = _case("llama-ragged")
    kve_overrides(spin_limit=1)
    out = alloc_out(D, w, budget)
    score_select_compact(D, w, out, uniform=budget)
    torch.cuda.synchronize()
    lens = out["seg_len"].cpu().numpy()
    kept = out["kept"].cpu().numpy()
    k_in, k_out = _ints(D["k"], w), _ints(out["k"], w)
    cap = out["cap"]
    for s in range(len(lens)):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        if lens[s] == -1:
            continue
        assert lens[s] == min(budget, n), (s, lens[s])
        ks = kept[s * cap:s * cap + lens[s]]
        ok, _, msg = kept_matches(ks, s_orc[o:o + n], n, budget, w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
        assert np.array_equal(k_out[s * cap:s * cap + lens[s]], k_in[o + ks])
    kve_overrides(spin_limit=0)
    out2 = alloc_out(D, w, budget)
    score_select_compact(D, w, out2, uniform=budget)
    torch.cuda.synchronize()
    _check_segments(w, L, D, out2, s_orc, [budget] * len(L["seg_len"]))
