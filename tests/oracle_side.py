"""Helpers that run the CPU oracle on generator output (tests and bench only)."""
import numpy as np
import torch

import oracle


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_cache_keys(layer, w):
    """Post-RoPE keys as stored: the oracle rotates the generator's pre-RoPE
    keys to their positions and rounds to the storage dtype."""
    return oracle.to_storage(oracle.rope(np64(layer["k_pre"]), layer["pos"].cpu().numpy(), w.rope_theta), w.dtype)


def oracle_layer_scores(layer, w, k=None, aggregate="max"):
    k = oracle_cache_keys(layer, w) if k is None else k
    return oracle.layer_scores(
        k, layer["pos"].cpu().numpy(), layer["seg_off"].cpu().numpy(), layer["seg_len"].cpu().numpy(),
        np64(layer["q_obs"]), layer["q_pos"].cpu().numpy(), layer["n_obs"].cpu().numpy(),
        w.n_kv_heads, w.rope_theta, w.dtype, bool(w.causal), aggregate)


def segment_chain(w, layer, b, g, n_triggers, device="cuda"):
    """The oracle's own sequence of eviction triggers for one segment (layer,
    request b, KV head g) of a multi-trigger workload, built the way the
    benchmark builds its trigger states: trigger 0 from the generator; trigger
    i+1 = the oracle's kept rows of trigger i, then the generator's appended
    tokens; the group's observation queries = the newest queries (recent rows)
    and the beacon buffer (the oracle's FPS survivors of trigger i, then the
    newest queries), recent rows at t-Rq .. t-1 and beacons at t.  Returns one
    dict per trigger: stored keys k, values v, positions pos (float64 / int),
    oracle scores, kept slots, per query head the pre-RoPE observation rows q,
    the FPS buffer and picks, and the rows' positions q_pos."""
    from workloads import make_append, make_layer
    G, Hkv, Hq, Rq, Nb, A = w.group, w.n_kv_heads, w.n_q_heads, w.n_recent_q, w.n_beacon, w.append
    L = make_layer(w, layer, device=device)
    n = L["lengths"][b]
    s = b * Hkv + g
    o = int(L["seg_off"][s])
    pos = L["pos"][o:o + n].cpu().numpy().astype(np.int64)
    k = oracle.to_storage(oracle.rope(np64(L["k_pre"][o:o + n]), pos, w.rope_theta), w.dtype)
    v = np64(L["v"][o:o + n])
    heads = list(range(g * G, (g + 1) * G))
    q = {h: np64(L["q_obs"][b, h]) for h in heads}
    qp = L["q_pos"][b].cpu().numpy().astype(np.int64)
    buf = {h: np64(L["fps_buf"][b * Hq + h]) for h in heads}
    t = int(pos.max()) + 1
    del L
    out = []
    for trig in range(n_triggers):
        rows = np.concatenate([oracle.to_storage(oracle.rope(q[h], qp, w.rope_theta), w.dtype) for h in heads])
        sc = oracle.segment_scores(k, pos, rows, np.tile(qp, G), bool(w.causal))
        kept = oracle.select_kept(sc, len(k), w.budget, w.n_prefix, w.n_recent)
        picks = {h: oracle.fps(buf[h], w.fps_keep) for h in heads}
        out.append({"k": k, "v": v, "pos": pos, "scores": sc, "kept": kept, "buf": dict(buf), "picks": picks, "t": t,
                    "q": dict(q), "q_pos": qp})
        if trig + 1 == n_triggers:
            break
        ap = make_append(w, layer, trig + 1, [t] * w.batch, device=device)
        apos = ap["pos"][b, g].cpu().numpy().astype(np.int64)
        knew = oracle.to_storage(oracle.rope(np64(ap["k_pre"][b, g]), apos, w.rope_theta), w.dtype)
        k = np.concatenate([k[kept], knew])
        v = np.concatenate([v[kept], np64(ap["v"][b, g])])
        pos = np.concatenate([pos[kept], apos])
        t += A
        for h in heads:
            qn = np64(ap["q_new"][b, h])
            buf[h] = np.concatenate([buf[h][np.sort(picks[h])], qn])
            q[h] = np.concatenate([qn, buf[h]])
        qp = np.concatenate([np.arange(t - Rq, t), np.full(Nb, t)])
    return out
