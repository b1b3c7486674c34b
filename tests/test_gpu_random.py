"""A seeded sweep of random shapes through the one-call trigger
(kv_evict_score_select_compact) and the two-call form (kv_evict_score,
kv_evict_select_compact), each against the oracle.

Every case draws its own configuration: dtype (bf16, or fp32 through the
plain-VALU path), head size 64 or 128, 1-8 KV heads with GQA groups of 1-8,
1-3 requests of ragged lengths from 0 to 6000 keys (some shorter than the
protected slots), ragged observation-row counts (some requests with a single
row), prefix and recent window of 0 or 4 and 0 or 16, causal or not, max or
mean aggregation, three RoPE bases, positions starting anywhere below 60,000,
and a uniform or a per-segment budget.  Scores must match within the parity tolerance, kept
sets inside the tie band, and the gathered rows byte for byte."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import device_layer
from tests.oracle_side import np64
from tests.parity import assert_scores_close, budgets_match, kept_matches
from workloads import random_layer, random_rows

pytestmark = pytest.mark.gpu

N_CASES = 64


def _config(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "f32" if r.random() < 0.2 else "bf16"
    d = int(r.choice([64, 128]))
    n_kv = int(r.choice([1, 2, 3, 8]))
    group = int(r.choice([1, 2, 4, 8]))
    max_rows = 256 if dtype == "bf16" else (96 if d == 128 else 192)   # fp32 rows live in the VALU path's LDS
    max_obs = int(r.integers(1, max_rows // group + 1))
    B = int(r.integers(1, 4))
    lengths = [int(x) for x in r.choice([0, 1, 5, 19, 20, 21, 300, 1023, 1025, 2900, 4096, 6000], size=B)]
    if max(lengths) == 0:
        lengths[0] = 300
    n_obs = [int(max_obs if r.random() < 0.5 else r.integers(1, max_obs + 1)) for _ in range(B)]
    P = int(r.choice([0, 4]))
    R = int(r.choice([0, 16]))
    causal = bool(r.random() < 0.8)
    theta = float(r.choice([1e4, 5e5, 1e6]))
    n_recent_q = int(r.choice([0, 8, 16]))
    per_seg = bool(r.random() < 0.4)
    aggregate = "mean" if r.random() < 0.2 else "max"
    longest = max(lengths) if max(lengths) > 0 else 1
    if per_seg:
        budget = [int(r.integers(P + R, max(P + R + 1, longest + 40))) for _ in range(B * n_kv)]
    else:
        budget = int(r.integers(P + R, max(P + R + 1, longest)))
    return dict(dtype=dtype, d=d, n_kv=n_kv, group=group, max_obs=max_obs, lengths=lengths, n_obs=n_obs, P=P, R=R,
                causal=causal, theta=theta, n_recent_q=n_recent_q, budget=budget, aggregate=aggregate)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


class _W:
    """The few workload fields the device-side helpers read."""

    def __init__(self, c):
        self.dtype, self.rope_theta, self.causal, self.n_kv_heads = c["dtype"], c["theta"], int(c["causal"]), c["n_kv"]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shapes_one_call_and_two_calls_match_oracle(seed):
    c = _config(seed)
    L = random_layer(seed, c["dtype"], c["d"], c["n_kv"], c["group"], c["lengths"], c["max_obs"], c["n_obs"],
                     c["n_recent_q"])
    L["k_pre"] = L["k_pre"] * 2.0                       # logits spread wider than N(0, 1)
    w = _W(c)
    D = device_layer(L, w)
    S, cap = len(L["seg_len"]), max(max(c["lengths"]), 1)
    k_orc = oracle.to_storage(oracle.rope(np64(L["k_pre"]), L["pos"].numpy(), c["theta"]), c["dtype"])
    s_orc = oracle.layer_scores(k_orc, L["pos"].numpy(), L["seg_off"].numpy(), L["seg_len"].numpy(),
                                np64(L["q_obs"]), L["q_pos"].numpy(), L["n_obs"].numpy(), c["n_kv"], c["theta"],
                                c["dtype"], c["causal"], c["aggregate"])
    bud = c["budget"] if isinstance(c["budget"], list) else [c["budget"]] * S
    budget_t = torch.tensor(bud, dtype=torch.int32, device="cuda") if isinstance(c["budget"], list) else None
    uniform = 0 if budget_t is not None else c["budget"]
    cache = kv.make_cache(D["k"], D["v"], D["pos"], D["seg_off"], D["seg_len"], c["n_kv"], cap)
    obs = kv.make_obs(D["q_obs"], D["q_pos"], D["n_obs"], c["theta"], c["causal"],
                      kv.KVE_AGG_MEAN if c["aggregate"] == "mean" else kv.KVE_AGG_MAX)
    results = {}
    for form in ("one-call", "two-call"):
        out = {"k": torch.zeros(S * cap, c["d"], dtype=D["k"].dtype, device="cuda"),
               "v": torch.zeros(S * cap, c["d"], dtype=D["v"].dtype, device="cuda"),
               "pos": torch.full((S * cap,), -7, dtype=torch.int32, device="cuda"),
               "seg_off": torch.arange(S, dtype=torch.int64, device="cuda") * cap,
               "seg_len": torch.full((S,), -9, dtype=torch.int32, device="cuda"),
               "kept": torch.full((S * cap,), -5, dtype=torch.int32, device="cuda")}
        cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], c["n_kv"], cap)
        scores = torch.zeros(max(D["k"].shape[0], 1), dtype=torch.float32, device="cuda")
        if form == "one-call":
            kv.kv_evict_score_select_compact(cache, obs, scores, budget_t, c["P"], c["R"], cout, kept_idx=out["kept"],
                                             uniform_budget=uniform)
        else:
            kv.kv_evict_score(cache, obs, scores)
            kv.kv_evict_select_compact(cache, scores, budget_t, c["P"], c["R"], cout, kept_idx=out["kept"],
                                       uniform_budget=uniform)
        torch.cuda.synchronize()
        results[form] = (scores.cpu().numpy()[:D["k"].shape[0]], out)
    esz = torch.int16 if c["dtype"] == "bf16" else torch.int32
    k_in, v_in, pos_in = D["k"].view(esz).cpu().numpy(), D["v"].view(esz).cpu().numpy(), D["pos"].cpu().numpy()
    for form, (sc, out) in results.items():
        assert_scores_close(sc, s_orc, what=f"case {seed} {form} scores {c}")
        kept, lens = out["kept"].cpu().numpy(), out["seg_len"].cpu().numpy()
        k_out, v_out, p_out = out["k"].view(esz).cpu().numpy(), out["v"].view(esz).cpu().numpy(), out["pos"].cpu().numpy()
        for s in range(S):
            o, n, K = int(L["seg_off"][s]), int(L["seg_len"][s]), bud[s]
            if K < n and K < c["P"] + c["R"] or min(K, n) > cap:
                assert lens[s] == -1, (seed, form, s, lens[s])
                continue
            m = min(K, n)
            assert lens[s] == m, (seed, form, s, lens[s], m, c)
            oo = s * cap
            ks = kept[oo:oo + m]
            ok, _, msg = kept_matches(ks, s_orc[o:o + n], n, K, c["P"], c["R"])
            assert ok, f"case {seed} {form} segment {s}: {msg} ({c})"
            assert np.array_equal(k_out[oo:oo + m], k_in[o + ks])
            assert np.array_equal(v_out[oo:oo + m], v_in[o + ks])
            assert np.array_equal(p_out[oo:oo + m], pos_in[o + ks])


def _inputs(seed):
    """The random layer of case `seed` on the device, the oracle's scores of it."""
    c = _config(seed)
    L = random_layer(seed, c["dtype"], c["d"], c["n_kv"], c["group"], c["lengths"], c["max_obs"], c["n_obs"],
                     c["n_recent_q"])
    L["k_pre"] = L["k_pre"] * 2.0
    D = device_layer(L, _W(c))
    k_orc = oracle.to_storage(oracle.rope(np64(L["k_pre"]), L["pos"].numpy(), c["theta"]), c["dtype"])
    s_orc = oracle.layer_scores(k_orc, L["pos"].numpy(), L["seg_off"].numpy(), L["seg_len"].numpy(),
                                np64(L["q_obs"]), L["q_pos"].numpy(), L["n_obs"].numpy(), c["n_kv"], c["theta"],
                                c["dtype"], c["causal"], c["aggregate"])
    cap = max(max(c["lengths"]), 1)
    obs = kv.make_obs(D["q_obs"], D["q_pos"], D["n_obs"], c["theta"], c["causal"],
                      kv.KVE_AGG_MEAN if c["aggregate"] == "mean" else kv.KVE_AGG_MAX)
    return c, L, D, s_orc, cap, obs


def _ints(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("seed", range(0, N_CASES, 2))
def test_random_shapes_inplace_match_oracle(seed):
    """Hole filling in place, one call and two calls, on the same random shapes:
    the survivors are the oracle's kept set (tie band), laid out exactly as
    oracle.hole_fill, moved rows byte-exact, rows past the new length untouched;
    the new lengths go to a separate array or to the cache's own lengths."""
    c, L, D, s_orc, cap, obs = _inputs(seed)
    S = len(L["seg_len"])
    bud = c["budget"] if isinstance(c["budget"], list) else [c["budget"]] * S
    budget_t = torch.tensor(bud, dtype=torch.int32, device="cuda") if isinstance(c["budget"], list) else None
    uniform = 0 if budget_t is not None else c["budget"]
    k0, v0, p0 = _ints(D["k"]), _ints(D["v"]), D["pos"].cpu().numpy()
    for one_call in (True, False):
        alias = bool((seed // 2 + one_call) % 2)
        C = dict(D, k=D["k"].clone(), v=D["v"].clone(), pos=D["pos"].clone(), seg_len=D["seg_len"].clone())
        cache = kv.make_cache(C["k"], C["v"], C["pos"], C["seg_off"], C["seg_len"], c["n_kv"], cap)
        new_len = C["seg_len"] if alias else torch.full_like(C["seg_len"], -9)
        scores = torch.zeros(max(D["k"].shape[0], 1), dtype=torch.float32, device="cuda")
        if one_call:
            kv.kv_evict_score_select_compact_inplace(cache, obs, scores, budget_t, c["P"], c["R"], new_len,
                                                     uniform_budget=uniform)
        else:
            kv.kv_evict_score(cache, obs, scores)
            kv.kv_evict_select_compact_inplace(cache, scores, budget_t, c["P"], c["R"], new_len,
                                               uniform_budget=uniform)
        torch.cuda.synchronize()
        nl = new_len.cpu().numpy()
        k1, v1, p1 = _ints(C["k"]), _ints(C["v"]), C["pos"].cpu().numpy()
        for s in range(S):
            o, n, K = int(L["seg_off"][s]), int(L["seg_len"][s]), bud[s]
            if K < n and K < c["P"] + c["R"]:
                assert nl[s] == -1, (seed, one_call, s, nl[s])
                continue
            m = min(K, n)
            assert nl[s] == m, (seed, one_call, s, nl[s], m, c)
            if m == 0:
                continue
            src = (p1[o:o + m] - p0[o]).astype(np.int64)        # positions rise by one per slot
            kept = np.sort(src)
            ok, _, msg = kept_matches(kept, s_orc[o:o + n], n, K, c["P"], c["R"])
            assert ok, f"case {seed} one_call={one_call} segment {s}: {msg} ({c})"
            assert np.array_equal(src, oracle.hole_fill(kept, n)), (seed, s, "layout")
            assert np.array_equal(k1[o:o + m], k0[o + src]) and np.array_equal(v1[o:o + m], v0[o + src])
            assert np.array_equal(k1[o + m:o + n], k0[o + m:o + n]) and np.array_equal(p1[o + m:o + n], p0[o + m:o + n])


@pytest.mark.parametrize("seed", range(1, N_CASES, 2))
def test_random_shapes_entropy_budgets_match_oracle(seed):
    """The one-call trigger with entropy-driven head budgets on the random
    shapes (its three-call fallback where they do not fit one kernel): scores,
    head entropies, head budgets under the largest-remainder contract, kept
    sets and gathered rows against the oracle."""
    c, L, D, s_orc, cap, obs = _inputs(seed)
    r = np.random.default_rng(5000 + seed)
    S, H, B = len(L["seg_len"]), c["n_kv"], len(c["lengths"])
    floor = int(r.choice([0, 16, 64]))
    inverse = int(r.random() < 0.3)
    n_all = np.array([int(x) for x in L["seg_len"]], dtype=np.int64)
    totals = []
    for b in range(B):
        n = n_all[b * H:(b + 1) * H]
        totals.append(max(int(np.minimum(floor, n).sum()), int(r.uniform(0.05, 1.2) * n.sum())))
    tot = torch.tensor(totals, dtype=torch.int32, device="cuda")
    scores = torch.zeros(max(D["k"].shape[0], 1), dtype=torch.float32, device="cuda")
    ent = torch.zeros(S, dtype=torch.float32, device="cuda")
    bud = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    out = {"k": torch.zeros(S * cap, c["d"], dtype=D["k"].dtype, device="cuda"),
           "v": torch.zeros(S * cap, c["d"], dtype=D["v"].dtype, device="cuda"),
           "pos": torch.full((S * cap,), -7, dtype=torch.int32, device="cuda"),
           "seg_off": torch.arange(S, dtype=torch.int64, device="cuda") * cap,
           "seg_len": torch.full((S,), -9, dtype=torch.int32, device="cuda"),
           "kept": torch.full((S * cap,), -5, dtype=torch.int32, device="cuda")}
    cache = kv.make_cache(D["k"], D["v"], D["pos"], D["seg_off"], D["seg_len"], H, cap)
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], H, cap)
    kv.kv_evict_score_budget_select_compact(cache, obs, scores, ent, tot, floor, c["P"], c["R"], cout,
                                            inverse=inverse, budget_out=bud, kept_idx=out["kept"])
    torch.cuda.synchronize()
    assert_scores_close(scores.cpu().numpy()[:D["k"].shape[0]], s_orc, what=f"case {seed} scores {c}")
    g_ent, g_bud = ent.cpu().numpy(), bud.cpu().numpy()
    lens, kept = out["seg_len"].cpu().numpy(), out["kept"].cpu().numpy()
    k_in, v_in, p_in = _ints(D["k"]), _ints(D["v"]), D["pos"].cpu().numpy()
    k_out, v_out, p_out = _ints(out["k"]), _ints(out["v"]), out["pos"].cpu().numpy()
    for b in range(B):
        segs = list(range(b * H, (b + 1) * H))
        n = n_all[segs]
        E = np.array([oracle.normalized_entropy(s_orc[int(L["seg_off"][s]):int(L["seg_off"][s]) + n[i]])
                      for i, s in enumerate(segs)])
        assert np.all(np.abs(g_ent[segs] - E) <= 2e-3 * np.maximum(np.abs(E), 1e-3)), (seed, g_ent[segs], E)
        ok, msg = budgets_match(g_bud[segs], g_ent[segs], E, n, totals[b], floor, bool(inverse))
        assert ok, f"case {seed} request {b}: {msg} ({c}, floor {floor}, total {totals[b]})"
        for i, s in enumerate(segs):
            K = int(g_bud[s])
            o = int(L["seg_off"][s])
            if K < n[i] and K < c["P"] + c["R"]:
                assert lens[s] == -1, (seed, s, lens[s], K)
                continue
            assert lens[s] == min(K, n[i]), (seed, s, lens[s], K)
            ks = kept[s * cap:s * cap + lens[s]]
            ok, _, msg = kept_matches(ks, s_orc[o:o + n[i]], int(n[i]), K, c["P"], c["R"])
            assert ok, f"case {seed} segment {s}: {msg}"
            rows = slice(s * cap, s * cap + lens[s])
            assert np.array_equal(k_out[rows], k_in[o + ks]) and np.array_equal(v_out[rows], v_in[o + ks])
            assert np.array_equal(p_out[rows], p_in[o + ks])


@pytest.mark.parametrize("seed", range(32))
def test_random_fps_buffers_match_oracle(seed):
    """Continual FPS on random buffers: bf16 (Gram matrix on the matrix cores)
    or fp32, head size 64 or 128, capacities 1-64, k_keep 1..cap, full and
    partly filled buffers, in place or not: every full buffer's picks pass the
    oracle's farthest-point check and its rows are those picks in ascending
    order; the others pass through unchanged."""
    r = np.random.default_rng(7000 + seed)
    dt = "f32" if r.random() < 0.3 else "bf16"
    d = int(r.choice([64, 128]))
    cap_max = 64 if (dt == "bf16" or d == 64) else 32          # fp32: cap * d * 4 bytes per wave in LDS
    cap = int(r.integers(1, cap_max + 1))
    keep = int(r.integers(1, cap + 1))
    n_buf = int(r.integers(1, 50))
    X = random_rows(seed, (n_buf, cap, d), dt).cuda()
    cnt = torch.full((n_buf,), cap, dtype=torch.int32)
    for i in r.choice(n_buf, size=min(n_buf, 3), replace=False):
        cnt[int(i)] = int(r.integers(0, cap))                    # not full: passes through
    cnt = cnt.cuda()
    in_place = bool(r.random() < 0.5)
    q_in, c_in = X.clone(), cnt.clone()
    q_out = q_in if in_place else torch.full_like(X, 3)
    c_out = c_in if in_place else torch.full_like(cnt, -3)
    picks = torch.full((n_buf, keep), -9, dtype=torch.int32, device="cuda")
    kv.beacon_fps_update(q_in, q_out, c_in, c_out, keep, picks)
    torch.cuda.synchronize()
    Xn, P, Co = np64(X), picks.cpu().numpy(), c_out.cpu().numpy()
    raw_in = X.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    raw_out = q_out.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    cn = cnt.cpu().numpy()
    for p in range(n_buf):
        if cn[p] != cap:
            assert Co[p] == cn[p] and np.all(P[p] == -1), (seed, p)
            assert np.array_equal(raw_out[p, :cn[p]], raw_in[p, :cn[p]]), (seed, p)
            continue
        assert Co[p] == keep, (seed, p, Co[p])
        ok, step = oracle.fps_acceptable(Xn[p], P[p], 2e-3)
        assert ok, f"case {seed} ({dt}, d {d}, cap {cap}, keep {keep}) buffer {p}: step {step}, picks {P[p].tolist()}"
        assert np.array_equal(raw_out[p, :keep], raw_in[p, np.sort(P[p])]), (seed, p)
