"""Whole-step invariants of the oracle on generator inputs."""
import numpy as np

import oracle
from workloads import get_workload, make_layer
from tests.oracle_side import oracle_cache_keys, oracle_layer_scores, np64


def test_tiny_step_invariants():
    w = get_workload("tiny-f32")
    L = make_layer(w, 0)
    k = oracle_cache_keys(L, w)
    sc = oracle_layer_scores(L, w, k)
    pos = L["pos"].numpy()
    q = np64(L["q_obs"])
    for s in range(w.batch * w.n_kv_heads):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        g = s % w.n_kv_heads
        kept = oracle.select_kept(sc[o:o + n], n, w.budget, w.n_prefix, w.n_recent)
        assert len(kept) == w.budget
        assert set(range(w.n_prefix)) <= set(kept) and set(range(n - w.n_recent, n)) <= set(kept)
        out = oracle.compact_rows(k[o:o + n], kept)
        assert np.all(np.diff(pos[o:o + n][kept]) > 0) and out.shape == (w.budget, w.head_dim)
        # the aggregate is at least every single query's probability
        for h in range(g * w.group, (g + 1) * w.group):
            qr = oracle.to_storage(oracle.rope(q[0, h], L["q_pos"][0].numpy(), w.rope_theta), w.dtype)
            p = oracle.segment_probabilities(k[o:o + n], pos[o:o + n], qr, L["q_pos"][0].numpy())
            assert np.all(sc[o:o + n][None, :] >= p)
    # FPS on every head's buffer: 16 -> 8 distinct picks
    for r in range(w.n_q_heads):
        p = oracle.fps(np64(L["fps_buf"][r]), w.fps_keep)
        assert len(set(p.tolist())) == w.fps_keep


def test_scores_reflect_the_clustered_structure():
    """Beacons aimed at clusters {0, 1} must rank those clusters' keys high."""
    w = get_workload("tiny-f32")
    L = make_layer(w, 0)
    sc = oracle_layer_scores(L, w)
    assert np.all(sc > 0) and np.all(sc <= 1)


def test_budget_pipeline_sums_to_layer_budget():
    w = get_workload("r1-llama-8b").scaled(batch=2, len_lo=300, len_hi=400, n_layers=4,
                                          wave_total=4 * 256, min_per_head=24)
    table = oracle.layer_wave_budgets(w.n_layers, 2.0, 1.0, w.wave_total, w.min_per_head)
    assert table.sum() == w.wave_total
    L = make_layer(w, 1)
    sc = oracle_layer_scores(L, w)
    for b in range(w.batch):
        ent, lens = [], []
        for g in range(w.n_kv_heads):
            s = b * w.n_kv_heads + g
            o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
            ent.append(oracle.normalized_entropy(sc[o:o + n]))
            lens.append(n)
        bud = oracle.head_budgets(np.array(ent), np.array(lens), w.n_kv_heads * table[1], w.min_per_head)
        assert bud.sum() == w.n_kv_heads * table[1]
        assert np.all(bud >= w.min_per_head)
