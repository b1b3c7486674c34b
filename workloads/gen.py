"""Seeded generators for the eviction-step inputs.

Everything here is random-number drawing and layout.  Keys are returned
*before* the rotary embedding (``k_pre``, fp32) together with their positions;
each side under test applies the rotation itself.  Queries are returned
pre-RoPE in the storage dtype, as a model would hand them over.

Layout conventions (shared by the oracle tests, the GPU tests and the bench):
  * a layer's cache is a list of segments, one per (request b, KV head g),
    segment s = b * n_kv_heads + g, rows packed back to back; ``seg_off[s]`` is
    the first row, ``seg_len[s]`` the number of valid rows;
  * observation queries are ``[batch, n_q_heads, n_obs, d]``: rows
    ``[0, n_recent_q)`` are the recent queries, the rest are beacons;
    ``q_pos[b, i]`` is the position each row is rotated to;
  * query head h belongs to KV head h // group.
"""
import math

import torch

from .specs import Workload

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _g(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _seed(w: Workload, layer: int, stream: int, trigger: int = 0):
    return w.seed_base * 1_000_003 + layer * 10_007 + trigger * 101 + stream


def request_lengths(w: Workload):
    """Per-request cache lengths, uniform in [len_lo, len_hi] (fixed per workload)."""
    if w.len_lo == w.len_hi:
        return [w.len_lo] * w.batch
    g = _g("cpu", _seed(w, 0, 99))
    return [int(x) for x in torch.randint(w.len_lo, w.len_hi + 1, (w.batch,), generator=g)]


def _centers(w: Workload, layer: int, device):
    g = _g(device, _seed(w, layer, 1))
    return torch.randn(w.batch, w.n_kv_heads, w.n_clusters, w.head_dim, generator=g, device=device)


def _assign(w: Workload, n: int, shape_prefix, g, device, late_only=False):
    """Cluster label per position: early positions use the early clusters."""
    E, C = w.early_clusters, w.n_clusters
    if late_only and E > 0:
        return torch.randint(E, C, (*shape_prefix, n), generator=g, device=device)
    if w.early_frac <= 0 or E == 0:
        return torch.randint(0, C, (*shape_prefix, n), generator=g, device=device)
    n_early = int(w.early_frac * n)
    a = torch.empty(*shape_prefix, n, dtype=torch.int64, device=device)
    a[..., :n_early] = torch.randint(0, E, (*shape_prefix, n_early), generator=g, device=device)
    a[..., n_early:] = torch.randint(E, C, (*shape_prefix, n - n_early), generator=g, device=device)
    return a


def _globalise(w: Workload, labels, g, device):
    """Re-aim a fraction of query labels at an early cluster ("global" queries)."""
    if w.global_frac <= 0:
        return labels
    hit = torch.rand(labels.shape, generator=g, device=device) < w.global_frac
    pool = w.early_clusters if w.early_clusters > 0 else w.n_clusters
    alt = torch.randint(0, pool, labels.shape, generator=g, device=device)
    return torch.where(hit, alt, labels)


def _near(centers_bg, labels, sigma, g, device):
    """centers_bg [..., C, d], labels [..., m] -> centers[label] + sigma * N(0, I)."""
    d = centers_bg.shape[-1]
    idx = labels.unsqueeze(-1).expand(*labels.shape, d)
    base = torch.gather(centers_bg, -2, idx)
    return base + sigma * torch.randn(base.shape, generator=g, device=device)


def make_layer(w: Workload, layer: int = 0, device="cpu", lengths=None):
    """Inputs of one layer at its first eviction trigger (step t = n per request)."""
    dt = _DT[w.dtype]
    lengths = list(lengths) if lengths is not None else request_lengths(w)
    B, Hkv, Hq, G, d = w.batch, w.n_kv_heads, w.n_q_heads, w.group, w.head_dim
    Rq, Nb = w.n_recent_q, w.n_beacon
    centers = _centers(w, layer, device)
    g = _g(device, _seed(w, layer, 2))
    k_parts, v_parts, p_parts = [], [], []
    q_obs = torch.empty(B, Hq, Rq + Nb, d, dtype=dt, device=device)
    q_pos = torch.empty(B, Rq + Nb, dtype=torch.int32, device=device)
    fps_rows = w.fps_cap if w.fps_cap else 0
    fps_buf = torch.zeros(B * Hq, max(fps_rows, 1), d, dtype=dt, device=device)
    for b, n in enumerate(lengths):
        assign = _assign(w, n, (Hkv,), g, device)                      # [Hkv, n]
        k = _near(centers[b], assign, w.key_sigma, g, device)          # [Hkv, n, d]
        v = torch.randn(Hkv, n, d, generator=g, device=device)
        k_parts.append(k.reshape(Hkv * n, d))
        v_parts.append(v.reshape(Hkv * n, d).to(dt))
        p_parts.append(torch.arange(n, dtype=torch.int32, device=device).repeat(Hkv))
        # recent queries: rows i at tau_i = n - Rq + i, near the cluster of the key there
        tau = torch.arange(n - Rq, n, device=device)
        lab_r = assign[:, tau].unsqueeze(1).expand(Hkv, G, Rq)
        lab_r = _globalise(w, lab_r, g, device)
        qr = _near(centers[b].unsqueeze(1).expand(Hkv, G, w.n_clusters, d), lab_r, w.key_sigma, g, device)
        # beacons
        if w.beacon_mode == "c01":
            lab_b = torch.randint(0, 2, (Hkv, G, Nb), generator=g, device=device)
        else:
            u = torch.randint(0, n, (Hkv, G, Nb), generator=g, device=device)
            lab_b = torch.gather(assign.unsqueeze(1).expand(Hkv, G, n), 2, u)
            lab_b = _globalise(w, lab_b, g, device)
        qb = _near(centers[b].unsqueeze(1).expand(Hkv, G, w.n_clusters, d), lab_b, w.key_sigma, g, device)
        q_obs[b, :, :Rq] = qr.reshape(Hq, Rq, d).to(dt)
        q_obs[b, :, Rq:] = qb.reshape(Hq, Nb, d).to(dt)
        q_pos[b, :Rq] = tau.to(torch.int32)
        q_pos[b, Rq:] = n
        if fps_rows:
            if w.fps_buf_mode == "beacons":
                buf = q_obs[b, :, Rq:]
            else:
                buf = torch.cat([q_obs[b, :, Rq:], q_obs[b, :, :Rq]], dim=1)
            assert buf.shape[1] == fps_rows
            fps_buf[b * Hq:(b + 1) * Hq] = buf
    seg_len = torch.tensor([n for n in lengths for _ in range(Hkv)], dtype=torch.int32)
    seg_off = torch.zeros(B * Hkv, dtype=torch.int64)
    seg_off[1:] = torch.cumsum(seg_len.to(torch.int64), 0)[:-1]
    return {
        "k_pre": torch.cat(k_parts), "v": torch.cat(v_parts), "pos": torch.cat(p_parts),
        "seg_off": seg_off.to(device), "seg_len": seg_len.to(device),
        "q_obs": q_obs, "q_pos": q_pos,
        "n_obs": torch.full((B,), Rq + Nb, dtype=torch.int32, device=device),
        "fps_buf": fps_buf, "fps_count": torch.full((B * Hq,), fps_rows, dtype=torch.int32, device=device),
        "lengths": lengths,
    }


def make_append(w: Workload, layer: int, trigger: int, t_start, device="cpu"):
    """Tokens decoded between two triggers: ``w.append`` new keys per segment at
    positions t_start[b] .. t_start[b] + append - 1 (late clusters), their values,
    and the newest ``n_recent_q`` queries per query head (pre-RoPE, storage dtype),
    which become the next trigger's recent queries and enter the beacon buffer."""
    dt = _DT[w.dtype]
    B, Hkv, Hq, G, d, A, Rq = w.batch, w.n_kv_heads, w.n_q_heads, w.group, w.head_dim, w.append, w.n_recent_q
    centers = _centers(w, layer, device)
    g = _g(device, _seed(w, layer, 3, trigger))
    assign = _assign(w, A, (B, Hkv), g, device, late_only=True)                  # [B, Hkv, A]
    k = _near(centers, assign, w.key_sigma, g, device)                            # [B, Hkv, A, d]
    v = torch.randn(B, Hkv, A, d, generator=g, device=device).to(dt)
    t0 = torch.as_tensor(t_start, dtype=torch.int64, device=device).view(B, 1, 1)
    pos = (t0 + torch.arange(A, device=device).view(1, 1, A)).expand(B, Hkv, A).to(torch.int32)
    lab = assign[:, :, A - Rq:].unsqueeze(2).expand(B, Hkv, G, Rq)
    lab = _globalise(w, lab, g, device)
    q = _near(centers.unsqueeze(2).expand(B, Hkv, G, w.n_clusters, d), lab, w.key_sigma, g, device)
    q = q.reshape(B, Hq, Rq, d).to(dt)
    return {"k_pre": k, "v": v, "pos": pos, "q_new": q}


def make_traces(w: Workload, device="cpu", T=None, d_model=None, batch=None, chunk=256):
    """Hidden-state traces h_l(t) for the two monitored layers, bf16
    ``[2, batch, T, d_model]``: a mean-reverting random walk
    h(t) = 0.995 h(t-1) + a_t xi_t, xi ~ N(0, I/d_model),
    a_t = exp(0.5 N(0,1)) (1 + t/T) (heavy-tailed steps with a positional trend)."""
    T = T or w.len_hi
    D = d_model or w.d_model
    B = batch or w.batch
    L = len(w.trace_layers) or 2
    rho = 0.995
    out = torch.empty(L, B, T, D, dtype=torch.bfloat16, device=device)
    g = _g(device, _seed(w, 0, 7))
    tt = torch.arange(T, device=device, dtype=torch.float32)
    carry = torch.zeros(L, B, D, device=device)
    for t0 in range(0, T, chunk):
        c = min(chunk, T - t0)
        a = torch.exp(0.5 * torch.randn(L, B, c, 1, generator=g, device=device)) * (1.0 + tt[t0:t0 + c] / T).view(1, 1, c, 1)
        x = a * torch.randn(L, B, c, D, generator=g, device=device) / math.sqrt(D)
        s = torch.arange(c, device=device, dtype=torch.float32)
        up = torch.pow(torch.tensor(rho, device=device), -s).view(1, 1, c, 1)
        dn = torch.pow(torch.tensor(rho, device=device), s).view(1, 1, c, 1)
        h = dn * torch.cumsum(x * up, dim=2) + (rho * dn) * carry.unsqueeze(2)
        out[:, :, t0:t0 + c] = h.to(torch.bfloat16)
        carry = h[:, :, -1]
    return out


def initial_recent_obs(L, w: Workload, n_initial: int, device="cpu"):
    """Observation set of the Initial+Recent alternative that the BeaconKV page
    ablates against (section 打分时的 RoPE 对齐, Table 3): the first n_initial
    queries of the sequence, at their own positions 0 .. n_initial-1, in place
    of the beacons, followed by the layer's recent queries.  An initial query
    of head h is the pre-RoPE key of its KV head at that position plus noise
    (the same construction as the recent queries, which sit near the key at
    their position).  Returns (q_obs [B, Hq, n_initial + Rq, d], q_pos, n_obs)."""
    dt = _DT[w.dtype]
    B, Hkv, Hq, G, d, Rq = w.batch, w.n_kv_heads, w.n_q_heads, w.group, w.head_dim, w.n_recent_q
    g = _g("cpu", _seed(w, 0, 7))
    k_pre = L["k_pre"].to("cpu")
    seg_off = L["seg_off"].to("cpu")
    init = torch.empty(B, Hq, n_initial, d)
    for b in range(B):
        for h in range(Hq):
            o = int(seg_off[b * Hkv + h // G])
            init[b, h] = k_pre[o:o + n_initial] + w.key_sigma * torch.randn(n_initial, d, generator=g)
    q_obs = torch.cat([init.to(dt), L["q_obs"][:, :, :Rq].to("cpu")], dim=2).to(device)
    q_pos = torch.cat([torch.arange(n_initial, dtype=torch.int32).expand(B, n_initial),
                       L["q_pos"][:, :Rq].to("cpu")], dim=1).contiguous().to(device)
    n_obs = torch.full((B,), n_initial + Rq, dtype=torch.int32, device=device)
    return q_obs, q_pos, n_obs


def make_sentences(batch: int, T: int, d_model: int, seed: int = 0, len_lo: int = 6, len_hi: int = 40,
                   repeat_frac: float = 0.25, near_frac: float = 0.1, noise: float = 0.5, common: float = 0.5):
    """Last-layer hidden states with sentence structure, for the sentence
    redundancy score (SkipKV page, §4.1 and observation 2: reasoning traces
    revisit earlier sentences).  Sentence lengths are uniform in [len_lo,
    len_hi]; the tokens after the last complete sentence form an unfinished
    one.  Each sentence has a topic vector (entries N(0, 1)): a fresh one, the
    topic of a random earlier sentence (probability repeat_frac: that earlier
    sentence gets a near-duplicate successor), or a blend 0.97 old + 0.25 new
    (probability near_frac: similarities around 0.95).  A token is its
    sentence's topic plus a component shared by the whole request (scale
    `common`) plus N(0, noise^2) per entry.
    Returns (h bf16 [B, T, d_model], starts int32 [B, max_sent + 1], n_sent int32 [B])."""
    g = torch.Generator().manual_seed(seed)
    hs, all_starts, n_sent = [], [], []
    for _ in range(batch):
        shared = common * torch.randn(d_model, generator=g)
        starts, topics = [0], []
        while True:
            L = int(torch.randint(len_lo, len_hi + 1, (1,), generator=g))
            if starts[-1] + L > T:
                break
            starts.append(starts[-1] + L)
            u = float(torch.rand(1, generator=g))
            if topics and u < repeat_frac:
                topics.append(topics[int(torch.randint(0, len(topics), (1,), generator=g))].clone())
            elif topics and u < repeat_frac + near_frac:
                old = topics[int(torch.randint(0, len(topics), (1,), generator=g))]
                topics.append(0.97 * old + 0.25 * torch.randn(d_model, generator=g))
            else:
                topics.append(torch.randn(d_model, generator=g))
        h = noise * torch.randn(T, d_model, generator=g) + shared
        for i, t in enumerate(topics):
            h[starts[i]:starts[i + 1]] += t
        tail_topic = torch.randn(d_model, generator=g)
        h[starts[-1]:] += tail_topic
        hs.append(h.to(torch.bfloat16))
        all_starts.append(starts)
        n_sent.append(len(starts) - 1)
    max_sent = max(n_sent)
    st = torch.zeros(batch, max_sent + 1, dtype=torch.int32)
    for b, s in enumerate(all_starts):
        st[b, :len(s)] = torch.tensor(s, dtype=torch.int32)
        st[b, len(s):] = s[-1]
    return torch.stack(hs), st, torch.tensor(n_sent, dtype=torch.int32)


def random_layer(seed: int, dtype: str, head_dim: int, n_kv_heads: int, group: int, lengths, max_obs: int, n_obs,
                 n_recent_q: int, device="cpu"):
    """Unstructured inputs of one layer for shape sweeps: keys, values and
    queries standard normal (keys pre-RoPE), request b's keys at positions
    start_b .. start_b + n_b - 1 (start_b random in [0, 60000)), its first
    n_recent_q observation rows at the n_recent_q positions before step
    t_b = start_b + n_b and the rest at t_b; rows at or past n_obs[b] exist in
    the tensor but are not observation rows.  Same layout as make_layer."""
    dt = _DT[dtype]
    g = _g(device, 7_000_003 + seed)
    B, Hkv, Hq, d = len(lengths), n_kv_heads, n_kv_heads * group, head_dim
    starts = torch.randint(0, 60000, (B,), generator=g, device=device)
    k_parts, v_parts, p_parts = [], [], []
    for b, n in enumerate(lengths):
        k_parts.append(torch.randn(Hkv * n, d, generator=g, device=device))
        v_parts.append(torch.randn(Hkv * n, d, generator=g, device=device).to(dt))
        p_parts.append((int(starts[b]) + torch.arange(n, dtype=torch.int32, device=device)).repeat(Hkv))
    q_obs = torch.randn(B, Hq, max_obs, d, generator=g, device=device).to(dt)
    q_pos = torch.empty(B, max_obs, dtype=torch.int32, device=device)
    for b, n in enumerate(lengths):
        t = int(starts[b]) + n
        r = min(n_recent_q, max_obs)
        q_pos[b, :r] = torch.arange(t - r, t, dtype=torch.int32, device=device)
        q_pos[b, r:] = t
    seg_len = torch.tensor([n for n in lengths for _ in range(Hkv)], dtype=torch.int32)
    seg_off = torch.zeros(B * Hkv, dtype=torch.int64)
    seg_off[1:] = torch.cumsum(seg_len.to(torch.int64), 0)[:-1]
    return {
        "k_pre": torch.cat(k_parts), "v": torch.cat(v_parts), "pos": torch.cat(p_parts),
        "seg_off": seg_off.to(device), "seg_len": seg_len.to(device),
        "q_obs": q_obs, "q_pos": q_pos,
        "n_obs": torch.tensor(list(n_obs), dtype=torch.int32, device=device),
        "lengths": list(lengths),
    }


def random_rows(seed: int, shape, dtype: str, device="cpu"):
    """Standard-normal rows of the given shape in the storage dtype (beacon
    buffers and other unstructured inputs of shape sweeps)."""
    g = _g(device, 9_000_011 + seed)
    return torch.randn(*shape, generator=g, device=device).to(_DT[dtype])
