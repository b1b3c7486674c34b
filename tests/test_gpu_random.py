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
from tests.parity import assert_scores_close, kept_matches
from workloads import random_layer

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
