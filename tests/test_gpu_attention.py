"""Decode attention over the (compacted) cache against the oracle: ragged
segments, several 1024-row chunks with a ragged tail, both head sizes, both
storage dtypes, GQA groups 1/2/4/8, empty segments, and the in-place
(hole-filled) layout attending like the ordered one."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import cache_of, device_layer, score_layer
from tests.oracle_side import np64
from workloads import get_workload, make_layer

pytestmark = pytest.mark.gpu

CASES = {
    "qwen3-4b-1l": get_workload("qwen3-4b-1l").scaled(batch=3),
    "llama-ragged": get_workload("r1-llama-8b").scaled(batch=3, len_lo=700, len_hi=3300, n_layers=1),
    "tiny-f32": get_workload("tiny-f32"),
    "d64-bf16-g1": get_workload("tiny-f32").scaled(dtype="bf16", n_q_heads=2, batch=2, len_lo=900, len_hi=2100),
    "g8": get_workload("qwen3-4b-1l").scaled(batch=2, n_q_heads=64, len_lo=1500, len_hi=2600),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def _queries(w, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (torch.randn(w.batch, w.n_q_heads, w.head_dim, generator=g) * 1.5).to(dt)


def _check(D, w, q, seg_len=None):
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.n_q_heads), float("nan"), device="cuda")
    kv.kv_decode_attention(cache_of(D, w), q.cuda(), out, lse)
    torch.cuda.synchronize()
    K, V = np64(D["k"]), np64(D["v"])
    qn = np64(q)
    lens = (seg_len if seg_len is not None else D["seg_len"]).cpu().numpy()
    offs = D["seg_off"].cpu().numpy()
    o_g, l_g = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            s = b * w.n_kv_heads + g
            o, n = int(offs[s]), int(lens[s])
            heads = slice(g * w.group, (g + 1) * w.group)
            want, wl = oracle.decode_attention(K[o:o + n], V[o:o + n], qn[b, heads])
            if n == 0:
                assert np.all(o_g[b, heads] == 0) and np.all(np.isneginf(l_g[b, heads]))
                continue
            scale = np.abs(want).max(axis=1, keepdims=True) + 1e-6
            assert np.all(np.abs(o_g[b, heads] - want) <= 1e-4 * scale), (b, g)
            assert np.allclose(l_g[b, heads], wl, rtol=0, atol=1e-4), (b, g)
    return out, lse


@pytest.mark.parametrize("name", list(CASES))
def test_decode_attention_matches_oracle(name):
    w = CASES[name]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    _check(D, w, _queries(w, 11))


def test_decode_attention_empty_and_short_segments():
    w = CASES["llama-ragged"]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    lens = D["seg_len"].clone()
    for s, v in ((0, 0), (3, 1), (5, 1023), (6, 1025), (9, 2048)):
        lens[s] = min(v, int(lens[s]))
    D2 = dict(D, seg_len=lens)
    _check(D2, w, _queries(w, 12), seg_len=lens)


def test_decode_attention_hole_filled_layout_matches_ordered():
    """Attention over the in-place compacted cache equals attention over the
    ordered (out-of-place) compaction of the same survivors."""
    w = CASES["qwen3-4b-1l"]
    L = make_layer(w, 0)
    D = device_layer(L, w)
    budget = 1500
    scores, _ = score_layer(D, w)
    # ordered compaction
    S = D["seg_off"].numel()
    ko = torch.zeros(S * budget, w.head_dim, dtype=D["k"].dtype, device="cuda")
    vo, po = torch.zeros_like(ko), torch.zeros(S * budget, dtype=torch.int32, device="cuda")
    offo = torch.arange(S, dtype=torch.int64, device="cuda") * budget
    leno = torch.zeros(S, dtype=torch.int32, device="cuda")
    cout = kv.make_cache(ko, vo, po, offo, leno, w.n_kv_heads, budget)
    kv.kv_evict_select_compact(cache_of(D, w), scores, None, w.n_prefix, w.n_recent, cout, uniform_budget=budget)
    # in place on a copy
    C = dict(D, k=D["k"].clone(), v=D["v"].clone(), pos=D["pos"].clone(), seg_len=D["seg_len"].clone())
    kv.kv_evict_select_compact_inplace(cache_of(C, w), scores, None, w.n_prefix, w.n_recent, C["seg_len"],
                                       uniform_budget=budget)
    q = _queries(w, 13).cuda()
    o1 = torch.empty(w.batch, w.n_q_heads, w.head_dim, device="cuda")
    o2 = torch.empty_like(o1)
    l1 = torch.empty(w.batch, w.n_q_heads, device="cuda")
    l2 = torch.empty_like(l1)
    kv.kv_decode_attention(cout, q, o1, l1)
    kv.kv_decode_attention(cache_of(C, w), q, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(leno, C["seg_len"])
    assert torch.allclose(o1, o2, rtol=1e-4, atol=1e-5) and torch.allclose(l1, l2, atol=1e-4)
    # and both match the oracle on the ordered cache
    Dc = {"k": ko, "v": vo, "seg_off": offo, "seg_len": leno, "pos": po, "max_len": budget}
    _check(Dc, w, q.cpu())
