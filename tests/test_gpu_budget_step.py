"""The one-kernel trigger with ReasonAlloc's entropy-driven head budgets
(kv_evict_score_budget_select_compact) against the oracle (scores, head
entropies, head budgets, kept sets and moved bytes) and against the three calls
it stands for (kv_evict_score with entropies, kv_evict_entropy_budgets,
kv_evict_select_compact); failure reporting driven from the host."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import alloc_out, cache_of, device_layer, obs_of, score_layer, select_compact
from tests.oracle_side import np64, oracle_cache_keys, oracle_layer_scores
from tests.parity import assert_scores_close, budgets_match, kept_matches
from workloads import get_workload, make_layer

pytestmark = pytest.mark.gpu

CASES = {
    # 4 requests x 8 heads, ragged lengths: four request-layers of eight heads
    "llama-ragged": get_workload("r1-llama-8b").scaled(batch=4, len_lo=700, len_hi=3300, n_layers=1),
    # d = 64, fewer heads per request-layer
    "d64": get_workload("tiny-f32").scaled(dtype="bf16", batch=5, len_lo=900, len_hi=2500),
    # segments of at most 256 keys: one work-group per segment (no first barrier)
    "short": get_workload("r1-llama-8b").scaled(batch=6, len_lo=100, len_hi=256, n_layers=1),
}
FLOOR = 24


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
        _cache[name] = (w, L, D, oracle_layer_scores(L, w, k))
    return _cache[name]


def _totals(w, L, frac):
    """Request-layer totals: a fraction of each request's cached rows over its heads."""
    n = np.asarray(L["lengths"], dtype=np.int64)
    return (np.maximum(FLOOR * w.n_kv_heads, (frac * n).astype(np.int64) * w.n_kv_heads)).astype(np.int32)


def _one_call(D, w, L, totals, inverse):
    S = D["seg_off"].numel()
    scores = torch.zeros(D["k"].shape[0], dtype=torch.float32, device="cuda")
    ent = torch.zeros(S, dtype=torch.float32, device="cuda")
    bud = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    out = alloc_out(D, w, D["max_len"])
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, out["cap"])
    tot = torch.from_numpy(totals).to("cuda")
    kv.kv_evict_score_budget_select_compact(cache_of(D, w), obs_of(D, w), scores, ent, tot, FLOOR, w.n_prefix,
                                            w.n_recent, cout, inverse=inverse, budget_out=bud, kept_idx=out["kept"])
    torch.cuda.synchronize()
    return scores, ent, bud, out


def _ints(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("form", ["one-kernel", "three-call"])
@pytest.mark.parametrize("inverse", [0, 1])
@pytest.mark.parametrize("name", list(CASES))
def test_entropy_budget_trigger_matches_oracle(name, inverse, form, kve_overrides):
    """form three-call: the entry point's own fallback (taken for fp32 caches,
    long segments or many heads), forced here by selecting the single-read
    scoring kernel."""
    if form == "three-call":
        kve_overrides(score_impl="fused")
    w, L, D, s_orc = _case(name)
    totals = _totals(w, L, 0.3)
    scores, ent, bud, out = _one_call(D, w, L, totals, inverse)
    assert_scores_close(scores.cpu().numpy(), s_orc)
    g_ent, g_bud = ent.cpu().numpy(), bud.cpu().numpy()
    lens, kept, cap = out["seg_len"].cpu().numpy(), out["kept"].cpu().numpy(), out["cap"]
    k_in, v_in, p_in = _ints(D["k"]), _ints(D["v"]), D["pos"].cpu().numpy()
    k_out, v_out, p_out = _ints(out["k"]), _ints(out["v"]), out["pos"].cpu().numpy()
    H = w.n_kv_heads
    for b in range(w.batch):
        segs = list(range(b * H, (b + 1) * H))
        n = np.array([int(L["seg_len"][s]) for s in segs])
        E = np.array([oracle.normalized_entropy(s_orc[int(L["seg_off"][s]):int(L["seg_off"][s]) + n[i]])
                      for i, s in enumerate(segs)])
        assert np.all(np.abs(g_ent[segs] - E) <= 2e-3 * np.maximum(np.abs(E), 1e-3)), (g_ent[segs], E)
        got = g_bud[segs]
        ok, msg = budgets_match(got, g_ent[segs], E, n, int(totals[b]), FLOOR, bool(inverse))
        assert ok, f"request {b}: {msg}"
        for i, s in enumerate(segs):
            K = int(got[i])
            assert lens[s] == min(K, n[i]), (s, lens[s], K)
            o = int(L["seg_off"][s])
            ks = kept[s * cap:s * cap + lens[s]]
            ok, _, msg = kept_matches(ks, s_orc[o:o + n[i]], int(n[i]), K, w.n_prefix, w.n_recent)
            assert ok, f"segment {s}: {msg}"
            rows = slice(s * cap, s * cap + lens[s])
            assert np.array_equal(k_out[rows], k_in[o + ks]) and np.array_equal(v_out[rows], v_in[o + ks])
            assert np.array_equal(p_out[rows], p_in[o + ks])


@pytest.mark.parametrize("name", list(CASES))
def test_entropy_budget_trigger_agrees_with_three_calls(name):
    w, L, D, _ = _case(name)
    totals = _totals(w, L, 0.2)
    scores, ent, bud, out = _one_call(D, w, L, totals, 0)
    s3, e3 = score_layer(D, w, entropy=True)
    b3 = torch.zeros_like(bud)
    kv.kv_evict_entropy_budgets(e3, 0, torch.from_numpy(totals).to("cuda"), D["seg_len"], w.batch, w.n_kv_heads,
                                FLOOR, b3)
    out3 = alloc_out(D, w, D["max_len"])
    select_compact(D, w, s3, out3, budget=b3)
    torch.cuda.synchronize()
    e1, e2 = ent.cpu().numpy(), e3.cpu().numpy()
    assert np.all(np.abs(e1 - e2) <= 1e-5 * np.maximum(np.abs(e2), 1e-3))
    g1, g2 = bud.cpu().numpy(), b3.cpu().numpy()
    H = w.n_kv_heads
    for b in range(w.batch):
        segs = slice(b * H, (b + 1) * H)
        n = D["seg_len"][segs].cpu().numpy()
        # each form's budgets follow the budget rule from its own entropies and from the other's
        for gb, ea, eb in ((g1, e1, e2), (g2, e2, e1)):
            ok, msg = budgets_match(gb[segs], ea[segs], eb[segs], n, int(totals[b]), FLOOR)
            assert ok, f"request {b}: {msg}"
    same = np.flatnonzero(g1 == g2)
    assert len(same) >= len(g1) - 2 * w.batch
    a, c = scores.cpu().numpy(), s3.cpu().numpy()
    assert_scores_close(a, c, rtol=2e-5, what="one-call vs three-call scores")
    cap = out["cap"]
    k1, k2 = out["kept"].cpu().numpy(), out3["kept"].cpu().numpy()
    l1, l2 = out["seg_len"].cpu().numpy(), out3["seg_len"].cpu().numpy()
    for s in same:
        assert l1[s] == l2[s]
        if not np.array_equal(k1[s * cap:s * cap + l1[s]], k2[s * cap:s * cap + l2[s]]):
            # only candidates tied within rounding may swap
            o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
            ok, _, msg = kept_matches(k1[s * cap:s * cap + l1[s]], c[o:o + n].astype(np.float64), n, int(g1[s]),
                                      w.n_prefix, w.n_recent, rtol=2e-5)
            assert ok, msg


@pytest.mark.parametrize("name", ["llama-ragged", "short"])
def test_entropy_budget_trigger_floors_exceed_total_and_failed_meetings(name, kve_overrides):
    """A request-layer whose floors exceed its total gets -1 in every head
    (as kv_evict_entropy_budgets); with the meeting poll bound forced to one
    poll from the host, request-layers whose work-groups did not meet report
    -1 and the others are exact; the default bound is whole again."""
    w, L, D, s_orc = _case(name)
    totals = _totals(w, L, 0.3)
    totals[1] = FLOOR * w.n_kv_heads - 5                      # below the floors
    H = w.n_kv_heads

    def check(allow_failed):
        scores, ent, bud, out = _one_call(D, w, L, totals, 0)
        lens, kept, cap = out["seg_len"].cpu().numpy(), out["kept"].cpu().numpy(), out["cap"]
        g_bud = bud.cpu().numpy()
        assert np.all(lens[H:2 * H] == -1)
        if not allow_failed:
            assert np.all(g_bud[H:2 * H] == -1)
        for s in range(len(lens)):
            if s // H == 1 or (allow_failed and lens[s] == -1):
                continue
            n, o = int(L["seg_len"][s]), int(L["seg_off"][s])
            K = int(g_bud[s])
            assert lens[s] == min(K, n)
            ok, _, msg = kept_matches(kept[s * cap:s * cap + lens[s]], s_orc[o:o + n], n, K, w.n_prefix, w.n_recent)
            assert ok, f"segment {s}: {msg}"

    check(False)
    kve_overrides(spin_limit=1)
    check(True)
    kve_overrides(spin_limit=0)
    check(False)


@pytest.mark.parametrize("name", ["llama-ragged", "short"])
def test_entropy_budget_trigger_degenerate_heads(name):
    """A request-layer with an empty head and a head shorter than the
    protected rows: the empty head gets budget 0 and length 0, the short one
    keeps every row, and the other heads share the total as the oracle's
    budgets (computed with the same lengths) say."""
    w, L, D, s_full = _case(name)
    H = w.n_kv_heads
    D2 = dict(D)
    D2["seg_len"] = D["seg_len"].clone()
    D2["seg_len"][1] = 0
    D2["seg_len"][2] = 10
    # the oracle's scores of the ten-row head (its own softmax over those rows)
    k_orc = oracle_cache_keys(L, w)
    o2 = int(L["seg_off"][2])
    qp = L["q_pos"][0].cpu().numpy()
    q = np64(L["q_obs"][0])
    rows = [oracle.to_storage(oracle.rope(q[hh], qp, w.rope_theta), w.dtype)
            for hh in range(2 * w.group, 3 * w.group)]
    s2 = oracle.segment_scores(k_orc[o2:o2 + 10], L["pos"][o2:o2 + 10].cpu().numpy(), np.concatenate(rows),
                               np.tile(qp, w.group))
    totals = _totals(w, L, 0.3)
    scores, ent, bud, out = _one_call(D2, w, L, totals, 0)
    g_ent, g_bud = ent.cpu().numpy(), bud.cpu().numpy()
    lens, kept, cap = out["seg_len"].cpu().numpy(), out["kept"].cpu().numpy(), out["cap"]
    n = np.array([int(D2["seg_len"][s]) for s in range(H)])
    seg_scores = [s_full[int(L["seg_off"][s]):int(L["seg_off"][s]) + n[s]] for s in range(H)]
    seg_scores[2] = s2
    E = np.array([oracle.normalized_entropy(x) if len(x) else 0.0 for x in seg_scores])
    assert np.all(np.abs(g_ent[:H] - E) <= 2e-3 * np.maximum(np.abs(E), 1e-3)), (g_ent[:H], E)
    want = oracle.head_budgets(oracle.head_weights(E, False), n, int(totals[0]), FLOOR)
    assert g_bud[1] == 0 and g_bud[2] == 10 and want[1] == 0 and want[2] == 10
    ok, msg = budgets_match(g_bud[:H], g_ent[:H], E, n, int(totals[0]), FLOOR)
    assert ok, msg
    assert lens[1] == 0 and lens[2] == 10
    assert np.array_equal(kept[2 * cap:2 * cap + 10], np.arange(10))
    for s in [0] + list(range(3, H)):
        ok, _, msg = kept_matches(kept[s * cap:s * cap + lens[s]], seg_scores[s], int(n[s]), int(g_bud[s]),
                                  w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
