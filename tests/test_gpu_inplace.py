"""In-place hole-filling compaction against the oracle, both as the
select/compact call after kv_evict_score (kv_evict_select_compact_inplace) and
as the one-call trigger (kv_evict_score_select_compact_inplace, one kernel for
bf16 segments up to the on-chip selection size, the two calls otherwise): the
survivors are the oracle's kept set (ties within tolerance), their layout is
exactly oracle.hole_fill of that set, the moved rows are byte-exact copies,
and rows beyond the new length are untouched."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import cache_of, device_layer, obs_of, score_layer
from tests.oracle_side import np64, oracle_cache_keys, oracle_layer_scores
from tests.parity import kept_matches
from workloads import get_workload, make_layer

pytestmark = pytest.mark.gpu

CASES = {
    "qwen3-4b-1l": (get_workload("qwen3-4b-1l").scaled(batch=4), 1792),
    "llama-ragged": (get_workload("r1-llama-8b").scaled(batch=3, len_lo=700, len_hi=1100, n_layers=1), 640),
    "long-5k": (get_workload("long-65k").scaled(batch=1, len_lo=5000, len_hi=5000), 1024),
    "tiny-f32": (get_workload("tiny-f32"), 448),
    "d64-bf16": (get_workload("tiny-f32").scaled(dtype="bf16", batch=3, len_lo=900, len_hi=2100), 700),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def _ints(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _run(w, L, D, budgets, uniform, alias, one_call=False):
    """Score, then compact in place on a copy of the cache (or both in one
    call); returns the copy and the new lengths."""
    C = dict(D, k=D["k"].clone(), v=D["v"].clone(), pos=D["pos"].clone(), seg_len=D["seg_len"].clone())
    new_len = C["seg_len"] if alias else torch.full_like(C["seg_len"], -9)
    if one_call:
        scores = torch.empty(C["k"].shape[0], dtype=torch.float32, device="cuda")
        kv.kv_evict_score_select_compact_inplace(cache_of(C, w), obs_of(C, w), scores, budgets, w.n_prefix,
                                                 w.n_recent, new_len, uniform_budget=uniform)
    else:
        scores, _ = score_layer(D, w)
        kv.kv_evict_select_compact_inplace(cache_of(C, w), scores, budgets, w.n_prefix, w.n_recent, new_len,
                                           uniform_budget=uniform)
    torch.cuda.synchronize()
    return C, new_len.cpu().numpy()


def _check(w, L, D, C, new_len, budgets_np, s_orc):
    k0, v0, p0 = _ints(D["k"]), _ints(D["v"]), D["pos"].cpu().numpy()
    k1, v1, p1 = _ints(C["k"]), _ints(C["v"]), C["pos"].cpu().numpy()
    moved = 0
    for s in range(len(L["seg_len"])):
        o, n, K = int(L["seg_off"][s]), int(L["seg_len"][s]), int(budgets_np[s])
        if K < n and K < w.n_prefix + w.n_recent:
            assert new_len[s] == -1
            assert np.array_equal(p1[o:o + n], p0[o:o + n])
            continue
        m = min(K, n)
        assert new_len[s] == m, (s, new_len[s], m)
        src = p1[o:o + m] - p0[o]                  # positions are the slots in these segments
        kept = np.sort(src)
        ok, _, msg = kept_matches(kept, s_orc[o:o + n], n, K, w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
        assert np.array_equal(src, oracle.hole_fill(kept, n)), f"segment {s}: layout"
        assert np.array_equal(k1[o:o + m], k0[o + src]) and np.array_equal(v1[o:o + m], v0[o + src])
        assert np.array_equal(k1[o + m:o + n], k0[o + m:o + n]) and np.array_equal(p1[o + m:o + n], p0[o + m:o + n])
        moved += int((src != np.arange(m)).sum())
    return moved


@pytest.mark.parametrize("one_call", [False, True])
@pytest.mark.parametrize("alias", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_inplace_matches_oracle(name, alias, one_call):
    w, budget = CASES[name]
    L = make_layer(w, 0)
    assert all(np.array_equal(L["pos"][int(L["seg_off"][s]):int(L["seg_off"][s]) + int(L["seg_len"][s])].numpy(),
                              np.arange(int(L["seg_len"][s]))) for s in range(len(L["seg_len"])))
    D = device_layer(L, w)
    s_orc = oracle_layer_scores(L, w, oracle_cache_keys(L, w))
    C, new_len = _run(w, L, D, None, budget, alias, one_call)
    moved = _check(w, L, D, C, new_len, np.full(len(L["seg_len"]), budget), s_orc)
    bound = sum(min(budget, int(n) - budget) for n in L["seg_len"] if int(n) > budget)
    assert 0 < moved <= bound
    print(f"{name}: {moved} rows moved of {int(L['seg_len'].sum())} (at most {bound})")


@pytest.mark.parametrize("one_call", [False, True])
def test_inplace_per_segment_budgets_and_degenerate_segments(one_call):
    w, _ = CASES["llama-ragged"]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    s_orc = oracle_layer_scores(L, w, oracle_cache_keys(L, w))
    S = len(L["seg_len"])
    lens = [int(x) for x in L["seg_len"]]
    rng = np.random.default_rng(5)
    bud = rng.integers(w.n_prefix + w.n_recent, 1200, size=S)
    bud[0] = lens[0]                       # K == n
    bud[1] = lens[1] + 7                   # K > n
    bud[2] = w.n_prefix + w.n_recent - 1   # rejected
    bud[3] = w.n_prefix + w.n_recent       # only the protected slots survive
    bud[4] = lens[4] - 1                   # one eviction
    budget = torch.tensor(bud, dtype=torch.int32, device="cuda")
    C, new_len = _run(w, L, D, budget, 0, False, one_call)
    _check(w, L, D, C, new_len, bud, s_orc)


def test_inplace_rejects_overlaps():
    w, budget = CASES["llama-ragged"]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    scores = D["k"].view(torch.float32).view(-1)[:D["k"].shape[0]]    # scores inside the key rows
    nl = torch.zeros_like(D["seg_len"])
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_select_compact_inplace(cache_of(D, w), scores, None, 4, 16, nl, uniform_budget=budget)
    assert ei.value.name == "KVE_EALIAS"
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_select_compact_inplace(cache_of(D, w), torch.zeros(D["k"].shape[0], device="cuda"), None, 4, 16,
                                           nl, uniform_budget=19)
    assert ei.value.name == "KVE_EBUDGET"


def test_one_call_inplace_rejects_bad_arguments():
    w, budget = CASES["llama-ragged"]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    cache, obs = cache_of(D, w), obs_of(D, w)
    nl = torch.full_like(D["seg_len"], -9)
    bad = D["k"].view(torch.float32).view(-1)[:D["k"].shape[0]]      # scores inside the key rows
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact_inplace(cache, obs, bad, None, 4, 16, nl, uniform_budget=budget)
    assert ei.value.name == "KVE_EALIAS"
    scores = torch.empty(D["k"].shape[0], dtype=torch.float32, device="cuda")
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact_inplace(cache, obs, scores, None, 4, 16, nl, uniform_budget=19)
    assert ei.value.name == "KVE_EBUDGET"
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score_select_compact_inplace(cache, obs, scores, None, 4, 16, nl, uniform_budget=budget,
                                                 ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "KVE_EWORKSPACE"
    with pytest.raises(kv.KveError) as ei:                            # new_len over the scores
        kv.kv_evict_score_select_compact_inplace(cache, obs, scores, None, 4, 16, scores[:nl.numel()].view(torch.int32),
                                                 uniform_budget=budget)
    assert ei.value.name == "KVE_EALIAS"
    torch.cuda.synchronize()
    assert torch.all(nl == -9)                                        # nothing ran


def test_chained_inplace_triggers_protect_by_slot():
    """Two in-place one-call triggers with fewer appended tokens than the
    protected recent window in between.  After hole filling, slot order no
    longer follows position, and the next trigger protects its last n_recent
    slots (BeaconKV's protected recent span, read by slot): with A < n_recent
    appended tokens that window holds the A new tokens and the last
    n_recent - A slots of the hole-filled region, whatever their positions.
    The GPU's second trigger equals the oracle's selection by slot on the
    oracle's own layout (scores within 2e-3, kept sets up to the tie band), and
    it keeps exactly those protected slots."""
    from workloads import make_append
    w, K = get_workload("qwen3-4b-1l").scaled(batch=2), 1792
    A = 8
    assert A < w.n_recent
    L = make_layer(w, 0)
    D = device_layer(L, w)
    n = int(L["lengths"][0])
    # trigger 1 on the GPU (in place, one call)
    C = dict(D, k=D["k"].clone(), v=D["v"].clone(), pos=D["pos"].clone(), seg_len=D["seg_len"].clone())
    sc1 = torch.empty(C["k"].shape[0], dtype=torch.float32, device="cuda")
    kv.kv_evict_score_select_compact_inplace(cache_of(C, w), obs_of(C, w), sc1, None, w.n_prefix, w.n_recent,
                                             C["seg_len"], uniform_budget=K)
    torch.cuda.synchronize()
    assert torch.all(C["seg_len"] == K)
    # append A tokens at slots K .. K+A-1 (positions n .. n+A-1), queries moved to step n + A
    full = make_append(w.scaled(append=w.n_recent_q), 0, 1, [n] * w.batch)   # the first A of its tokens
    ap = {k: full[k][:, :, :A].contiguous() for k in ("k_pre", "v", "pos")}
    S = w.batch * w.n_kv_heads
    new_k = torch.empty(S * A, w.head_dim, dtype=torch.bfloat16, device="cuda")
    kv.kv_rope_apply(ap["k_pre"].reshape(-1, w.head_dim).contiguous().cuda(), new_k,
                     ap["pos"].reshape(-1).contiguous().cuda(), w.rope_theta)
    rows = (torch.arange(S, device="cuda") * n).view(S, 1) + K + torch.arange(A, device="cuda").view(1, A)
    C["k"][rows.view(-1)] = new_k
    C["v"][rows.view(-1)] = ap["v"].reshape(-1, w.head_dim).cuda()
    C["pos"][rows.view(-1)] = ap["pos"].reshape(-1).cuda()
    C["seg_len"].fill_(K + A)
    t2 = n + A
    C["q_pos"] = torch.cat([torch.arange(t2 - w.n_recent_q, t2, dtype=torch.int32).expand(w.batch, -1),
                            torch.full((w.batch, w.n_beacon), t2, dtype=torch.int32)], 1).contiguous().cuda()
    k_before = C["k"].clone()
    pos_before = C["pos"].cpu().numpy()
    sc2 = torch.empty(C["k"].shape[0], dtype=torch.float32, device="cuda")
    new_len = torch.full_like(C["seg_len"], -9)
    kv.kv_evict_score_select_compact_inplace(cache_of(C, w), obs_of(C, w), sc2, None, w.n_prefix, w.n_recent,
                                             new_len, uniform_budget=K)
    torch.cuda.synchronize()
    assert torch.all(new_len == K)
    # the oracle's own chain for each segment
    k_orc = oracle_cache_keys(L, w)
    s1 = oracle_layer_scores(L, w, k_orc)
    qp2 = C["q_pos"].cpu().numpy()
    pos_after = C["pos"].cpu().numpy()
    k_now, k_prev = _ints(C["k"]), _ints(k_before)
    checked = 0
    for s in range(S):
        b, g = divmod(s, w.n_kv_heads)
        o = int(L["seg_off"][s])
        kept1 = oracle.select_kept(s1[o:o + n], n, K, w.n_prefix, w.n_recent)
        src = oracle.hole_fill(kept1, n)
        lay_pos = np.concatenate([np.arange(n)[src], ap["pos"][b, g].numpy()])   # trigger-1 positions are the slots
        if not np.array_equal(pos_before[s * n:s * n + K + A], lay_pos):
            continue                                   # trigger 1 resolved a near-tie the other way
        kn = oracle.to_storage(oracle.rope(np64(ap["k_pre"][b, g]), ap["pos"][b, g].numpy(), w.rope_theta), w.dtype)
        lay_k = np.concatenate([k_orc[o:o + n][src], kn])
        q = np64(L["q_obs"][b])
        qrows = [oracle.to_storage(oracle.rope(q[h], qp2[b], w.rope_theta), w.dtype)
                 for h in range(g * w.group, (g + 1) * w.group)]
        s2 = oracle.segment_scores(lay_k, lay_pos, np.concatenate(qrows), np.tile(qp2[b], w.group))
        got2 = sc2[s * n:s * n + K + A].cpu().numpy()
        assert np.all(np.abs(got2 - s2) <= np.maximum(2e-3 * np.abs(s2), 1e-30)), f"segment {s}: scores"
        # the GPU's kept slots of trigger 2, from where each kept position sat before it
        at = {int(p): j for j, p in enumerate(pos_before[s * n:s * n + K + A])}
        kept2 = np.sort([at[int(p)] for p in pos_after[s * n:s * n + K]])
        ok, _, msg = kept_matches(kept2, s2, K + A, K, w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
        prot = np.arange(K + A - w.n_recent, K + A)
        assert np.all(np.isin(prot, kept2)), f"segment {s}: a protected slot was evicted"
        # the protected window reaches back into the hole-filled region
        assert np.any(lay_pos[prot] < n)
        assert np.array_equal(oracle.hole_fill(kept2, K + A), np.array([at[int(p)] for p in pos_after[s * n:s * n + K]]))
        assert np.array_equal(k_now[s * n:s * n + K], k_prev[s * n + np.array([at[int(p)] for p in pos_after[s * n:s * n + K]])])
        checked += 1
    assert checked >= S - 2, f"only {checked} of {S} segments checked"
