"""Sentence-redundancy score (SkipKV §4.1) on the GPU against the oracle, and
its token scores driving the protected top-K selection for every KV head."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import alloc_out, device_layer, select_compact
from tests.parity import kept_matches
from workloads import get_workload, make_layer, make_sentences

pytestmark = pytest.mark.gpu
TAU = 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


def _run(h, st, ns):
    B, T, _ = h.shape
    max_sent = st.shape[1] - 1
    pss = torch.full((B, max_sent), float("nan"), device="cuda")
    marks = torch.full((B, max_sent), -3, dtype=torch.int32, device="cuda")
    tok = torch.full((B, T), float("nan"), device="cuda")
    kv.skipkv_sentence_scores(h.cuda(), st.cuda(), ns.cuda(), TAU, pss, tok, marks=marks)
    torch.cuda.synchronize()
    return pss.cpu().numpy(), marks.cpu().numpy(), tok.cpu().numpy()


@pytest.mark.parametrize("T,d_model,seed", [(1500, 512, 3), (4100, 1024, 4), (3000, 4096, 5)])
def test_sentence_scores_match_oracle(T, d_model, seed):
    h, st, ns = make_sentences(2, T, d_model, seed=seed)
    pss, marks, tok = _run(h, st, ns)
    for b in range(2):
        n = int(ns[b])
        starts = st[b, :n + 1].numpy()
        hb = h[b].float().numpy().astype(np.float64)
        want = oracle.pss_later_max(oracle.sentence_means(hb, starts))
        assert np.allclose(pss[b, :n], want, rtol=0, atol=2e-5), float(np.abs(pss[b, :n] - want).max())
        assert np.all(pss[b, n:] == -1.0)
        # the tau decision in fp32 on both sides; a mismatch only inside the rounding band
        want_m = (want.astype(np.float32) >= np.float32(TAU)).astype(np.int32)
        diff = np.nonzero(marks[b, :n] != want_m)[0]
        assert np.all(np.abs(want[diff] - TAU) <= 2e-5), diff
        assert np.all(marks[b, n:] == 0)
        want_t = oracle.skipkv_token_scores(want, starts, T)
        assert np.allclose(tok[b], want_t, rtol=0, atol=2e-5)


def test_degenerate_sentences():
    """An empty sentence has a zero embedding (cosine 0 with everything); a
    request with no complete sentence scores 1 everywhere."""
    h, st, ns = make_sentences(3, 600, 256, seed=9)
    st = st.clone()
    ns = ns.clone()
    st[0, 2] = st[0, 1]           # sentence 1 of request 0 becomes empty
    ns[2] = 0
    pss, marks, tok = _run(h, st, ns)
    for b in range(2):
        n = int(ns[b])
        starts = st[b, :n + 1].numpy()
        want = oracle.pss_later_max(oracle.sentence_means(h[b].float().numpy().astype(np.float64), starts))
        assert np.allclose(pss[b, :n], want, atol=2e-5)
        assert np.allclose(tok[b], oracle.skipkv_token_scores(want, starts, 600), atol=2e-5)
    assert np.all(tok[2] == 1.0) and np.all(pss[2] == -1.0) and np.all(marks[2] == 0)


def test_token_scores_drive_selection_for_every_head():
    w = get_workload("r1-llama-8b").scaled(batch=2, len_lo=1500, len_hi=1500, n_layers=1)
    L = make_layer(w, 0)
    D = device_layer(L, w)
    h, st, ns = make_sentences(2, 1500, 1024, seed=6)
    pss, _, tok = _run(h, st, ns)
    scores = torch.from_numpy(tok).cuda()
    score_off = (torch.arange(2 * w.n_kv_heads, device="cuda") // w.n_kv_heads * 1500).to(torch.int64)
    budget = 1100
    out = alloc_out(D, w, budget)
    select_compact(D, w, scores.view(-1), out, uniform=budget, score_off=score_off)
    torch.cuda.synchronize()
    kept = out["kept"].cpu().numpy()
    for b in range(2):
        n = int(ns[b])
        starts = st[b, :n + 1].numpy()
        want = oracle.skipkv_token_scores(
            oracle.pss_later_max(oracle.sentence_means(h[b].float().numpy().astype(np.float64), starts)), starts, 1500)
        for g in range(w.n_kv_heads):
            s = b * w.n_kv_heads + g
            ok, _, msg = kept_matches(kept[s * budget:(s + 1) * budget], want, 1500, budget, 4, 16, rtol=2e-5,
                                      floor=2e-5)
            assert ok, msg
