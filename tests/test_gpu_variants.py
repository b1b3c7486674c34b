"""Variants of the step on the GPU against the oracle: mean aggregation of
the observation rows (BeaconKV's max-vs-mean ablation), inverse-entropy head
budgets (ReasonAlloc, Key Concepts), the EPIKV rolling-mean score (part 2) and
the Initial+Recent observation set (BeaconKV's Table 3 alternative, which
changes only the caller's query set)."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import alloc_out, device_layer, score_layer, score_select_compact, select_compact
from tests.oracle_side import np64, oracle_cache_keys, oracle_layer_scores
from tests.parity import assert_scores_close, budgets_match, kept_matches
from workloads import get_workload, initial_recent_obs, make_layer, make_traces

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-f32": get_workload("tiny-f32"),
    "qwen3-4b-1l": get_workload("qwen3-4b-1l").scaled(batch=3),
    "llama-ragged": get_workload("r1-llama-8b").scaled(batch=3, len_lo=700, len_hi=1100, n_layers=1),
    "non-causal": get_workload("qwen3-4b-1l").scaled(batch=2, len_lo=500, len_hi=900, causal=0),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


_cache = {}


def _case(name):
    if name not in _cache:
        w = CASES[name]
        L = make_layer(w, 0)
        D = device_layer(L, w)
        k = oracle_cache_keys(L, w)
        _cache[name] = (w, L, D, k, oracle_layer_scores(L, w, k, aggregate="mean"))
    return _cache[name]


@pytest.mark.parametrize("impl", ["mfma", "fused", "valu"])
@pytest.mark.parametrize("name", list(CASES))
def test_mean_aggregation_scores_and_entropy(name, impl, kve_overrides):
    w, L, D, _, s_orc = _case(name)
    if impl != "mfma":
        if w.dtype != "bf16":
            pytest.skip("fp32 caches always use the VALU path")
        kve_overrides(score_impl=impl)
    scores, ent = score_layer(D, w, entropy=True, aggregate=kv.KVE_AGG_MEAN)
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy(), s_orc, what=f"{name}/{impl} mean scores")
    e = ent.cpu().numpy()
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        want = oracle.normalized_entropy(s_orc[o:o + n])
        assert abs(e[s] - want) <= 2e-3 * max(abs(want), 1e-3), (s, e[s], want)


@pytest.mark.parametrize("name", ["qwen3-4b-1l", "llama-ragged"])
def test_mean_aggregation_one_call_trigger(name):
    w, L, D, _, s_orc = _case(name)
    budget = 600
    out = alloc_out(D, w, budget)
    scores = score_select_compact(D, w, out, uniform=budget, aggregate=kv.KVE_AGG_MEAN)
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy(), s_orc, what="one-call mean scores")
    kept, lens = out["kept"].cpu().numpy(), out["seg_len"].cpu().numpy()
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        m = min(budget, n)
        assert lens[s] == m
        ok, _, msg = kept_matches(kept[s * budget:s * budget + m], s_orc[o:o + n], n, budget, w.n_prefix, w.n_recent)
        assert ok, msg


@pytest.mark.parametrize("inverse", [0, 1])
def test_entropy_budgets_both_directions(inverse):
    """Scores with head entropy -> budgets with weight E or 1 - E -> variable-K
    selection; the direction decides which heads gain."""
    w, L, D, _, _ = _case("llama-ragged")
    k = oracle_cache_keys(L, w)
    s_orc = oracle_layer_scores(L, w, k)
    scores, ent = score_layer(D, w, entropy=True)
    total = torch.full((w.batch,), int(w.n_kv_heads * 500), dtype=torch.int32, device="cuda")
    bud = torch.zeros(w.batch * w.n_kv_heads, dtype=torch.int32, device="cuda")
    kv.kv_evict_entropy_budgets(ent, inverse, total, D["seg_len"], w.batch, w.n_kv_heads, 24, bud)
    out = alloc_out(D, w, int(max(L["lengths"])))
    select_compact(D, w, scores, out, budget=bud)
    torch.cuda.synchronize()
    g_bud, g_ent = bud.cpu().numpy(), ent.cpu().numpy()
    kept, lens, cap = out["kept"].cpu().numpy(), out["seg_len"].cpu().numpy(), out["cap"]
    for b in range(w.batch):
        segs = list(range(b * w.n_kv_heads, (b + 1) * w.n_kv_heads))
        n = [int(L["seg_len"][s]) for s in segs]
        E = np.array([oracle.normalized_entropy(s_orc[int(L["seg_off"][s]):int(L["seg_off"][s]) + n[i]])
                      for i, s in enumerate(segs)])
        got = g_bud[segs]
        ok, msg = budgets_match(got, g_ent[segs], E, n, int(w.n_kv_heads * 500), 24, bool(inverse))
        assert ok, f"request {b}: {msg}"
        # the direction: the most focused head gets at least as much as the most diffuse one under 1 - E
        e = g_ent[segs]
        lo, hi = int(np.argmin(e)), int(np.argmax(e))
        if inverse:
            assert got[lo] >= got[hi]
        else:
            assert got[hi] >= got[lo]
        for i, s in enumerate(segs):
            assert lens[s] == got[i]
            o = int(L["seg_off"][s])
            ok, _, msg = kept_matches(kept[s * cap:s * cap + got[i]], s_orc[o:o + n[i]], n[i], int(got[i]), 4, 16)
            assert ok, msg


def test_epikv_rolling_mean_form():
    w = get_workload("long-65k")
    B, T, Dm, W = 2, 1500, 1024, 128
    h = make_traces(w, T=T, d_model=Dm, batch=B)
    hd = h.cuda()
    scores = torch.zeros(B, T, dtype=torch.float32, device="cuda")
    kv.epikv_score(hd[0], hd[1], W, w.epikv_eps, scores, form=kv.KVE_EPIKV_MEAN)
    torch.cuda.synchronize()
    hn = np64(h)
    for b in range(B):
        ga, gb = oracle.epikv_g(hn[0, b]), oracle.epikv_g(hn[1, b])
        want = oracle.epikv_score(hn[0, b], hn[1, b], W, w.epikv_eps, form="mean")
        scale = np.maximum(oracle.rolling_mean(ga, W), oracle.rolling_mean(gb, W))
        err = np.abs(scores[b].cpu().numpy().astype(np.float64) - want)
        assert np.all(err <= 1e-4 * scale + 1e-6), float((err / (scale + 1e-12)).max())


def test_initial_recent_observation_set():
    """Initial+Recent: the first queries of the sequence at their own positions
    stand in for the beacons; only the caller's query set changes."""
    w = get_workload("qwen3-4b-1l").scaled(batch=2, len_lo=1200, len_hi=1500)
    L = make_layer(w, 0)
    q_obs, q_pos, n_obs = initial_recent_obs(L, w, 16)
    L2 = dict(L, q_obs=q_obs, q_pos=q_pos, n_obs=n_obs)
    D = device_layer(L2, w)
    k = oracle_cache_keys(L2, w)
    s_orc = oracle_layer_scores(L2, w, k)
    scores, _ = score_layer(D, w)
    budget = 1000
    out = alloc_out(D, w, budget)
    select_compact(D, w, scores, out, uniform=budget)
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy(), s_orc, what="initial+recent scores")
    kept = out["kept"].cpu().numpy()
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        ok, _, msg = kept_matches(kept[s * budget:(s + 1) * budget], s_orc[o:o + n], n, budget, w.n_prefix,
                                  w.n_recent)
        assert ok, msg
    # the initial rows see only the first keys: keys beyond position 15 get no
    # mass from them, so late keys' scores come from the recent rows alone
    assert int(q_pos[:, :16].max()) == 15
