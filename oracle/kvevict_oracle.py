"""Float64 CPU oracle of the eviction step (test infrastructure only).

Every function takes and returns numpy arrays.  Floating point is float64
throughout, including where a value decides an integer (the top-K cut, the
FPS argmax).  Stored tensors (bf16 / fp32) enter as their exact values
widened to float64.

Readings of points the pages leave open are marked READING and collected in
the design notes of the repository.
"""
import math

import numpy as np

__all__ = [
    "round_bf16", "to_storage", "rope", "visible_mask", "segment_probabilities",
    "segment_scores", "layer_scores", "normalized_entropy", "waterfill",
    "largest_remainder", "head_budgets", "layer_wave_budgets", "select_kept",
    "compact_rows", "fps", "fps_acceptable", "epikv_g", "rolling_z", "rolling_mean", "epikv_score",
    "layer_select_compact", "head_weights", "hole_fill", "decode_attention", "sentence_means",
    "pss_later_max", "skipkv_token_scores",
]


# ---------------------------------------------------------------- rounding
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Rounds directly from float64: a float32 intermediate is used only where it
    cannot change the result; when the float32 value sits exactly on a bf16
    midpoint the original float64 value decides."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    r = x.astype(np.float32)
    bits = r.view(np.uint32).astype(np.uint64)
    low = bits & 0xFFFF
    trunc = bits & 0xFFFF0000
    lsb = (bits >> 16) & 1
    rne = (bits + 0x7FFF + lsb) & 0xFFFF0000
    at_mid = low == 0x8000
    mag_x = np.abs(x)
    mag_m = np.abs(r.astype(np.float64))
    away = trunc + 0x10000                        # next bf16 away from zero
    res = np.where(at_mid & (mag_x > mag_m), away, np.where(at_mid & (mag_x < mag_m), trunc, rne))
    return res.astype(np.uint32).view(np.float32).astype(np.float64).reshape(x.shape)


def to_storage(x, dtype):
    """Round float64 values to the storage dtype ("bf16", "f32" or "f64")."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return x
    raise ValueError(dtype)


# ---------------------------------------------------------------- O1: RoPE
def rope(x, pos, theta):
    """Rotary position embedding at integer positions, half-split pairing.

    BeaconKV, section "打分时的 RoPE 对齐" (RoPE alignment at scoring time):
    beacons are stored pre-RoPE and rotated to the current step, recent queries
    keep their own positions.  READING: pairs are (x_i, x_{i+d/2}) with
    frequency theta^(-2i/d); the angle p * freq is formed in float64.
    x: [..., d]; pos: broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    inv = float(theta) ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ------------------------------------------------ O2-O4: observation scores
def visible_mask(key_pos, query_pos, causal=True):
    """[rows, n] boolean: key j visible to query row i iff key_pos[j] <= query_pos[i].

    READING: recent queries attend causally from their own position; beacons
    sit at step t, after every cached key, so they see all keys."""
    key_pos = np.asarray(key_pos)
    query_pos = np.asarray(query_pos)
    if not causal:
        return np.ones((query_pos.shape[0], key_pos.shape[0]), dtype=bool)
    return key_pos[None, :] <= query_pos[:, None]


def segment_probabilities(k, key_pos, q_rot, q_pos, causal=True):
    """Per-row softmax of q.k / sqrt(d) over one KV head's cached keys.

    k: [n, d] cached keys (post-RoPE, exact stored values); q_rot: [rows, d]
    rotated observation queries.  Returns p [rows, n]; masked entries are 0 and
    a row with no visible key is all 0."""
    k = np.asarray(k, dtype=np.float64)
    q_rot = np.asarray(q_rot, dtype=np.float64)
    if k.shape[0] == 0:                          # an empty segment: no key to score
        return np.zeros((q_rot.shape[0], 0))
    d = k.shape[1]
    logits = (q_rot @ k.T) / math.sqrt(d)
    vis = visible_mask(key_pos, q_pos, causal)
    masked = np.where(vis, logits, -np.inf)
    m = masked.max(axis=1, keepdims=True)
    has = np.isfinite(m)
    m = np.where(has, m, 0.0)
    ex = np.where(vis, np.exp(masked - m), 0.0)
    lse = m + np.log(np.where(has, ex.sum(axis=1, keepdims=True), 1.0))
    return np.where(vis & has, np.exp(logits - lse), 0.0)


def segment_scores(k, key_pos, q_rot, q_pos, causal=True, aggregate="max"):
    """Importance of every cached key of one KV head: the maximum, over the
    observation rows of all query heads sharing this KV head, of that row's
    softmax probability.

    BeaconKV, section "打分时的 RoPE 对齐": importance is max-aggregated over
    the observation queries (max, not mean, so a single beacon that rates a key
    highly keeps it).  READING: the maximum also runs over the GQA group.

    aggregate="mean" is the ablation the same page reports in its experiments
    section (max vs mean aggregation): the mean over the same rows.  READING: a
    key that a row cannot see contributes 0 for that row, and every observation
    row counts in the denominator (a row that sees no key at all contributes 0)."""
    p = segment_probabilities(k, key_pos, q_rot, q_pos, causal)
    if p.shape[0] == 0:
        return np.zeros(p.shape[1])
    if aggregate == "mean":
        return p.sum(axis=0) / p.shape[0]
    if aggregate != "max":
        raise ValueError(aggregate)
    return p.max(axis=0)


def layer_scores(k_cache, key_pos, seg_off, seg_len, q_obs, q_pos, n_obs, n_kv_heads,
                 theta, dtype, causal=True, aggregate="max"):
    """Scores for every row of one layer's segmented cache (O1-O4).

    k_cache [rows, d] exact stored values; q_obs [B, Hq, max_obs, d] pre-RoPE
    exact stored values; segment s = b * n_kv_heads + g; query head h belongs
    to KV head h // (Hq / n_kv_heads).  The rotated query is rounded to the
    storage dtype before the contraction (READING: both sides contract
    storage-precision operands).  Returns float64 [rows] (rows outside every
    segment stay 0)."""
    B, Hq, _, d = q_obs.shape
    G = Hq // n_kv_heads
    out = np.zeros(k_cache.shape[0])
    for b in range(B):
        no = int(n_obs[b])
        qp = np.asarray(q_pos[b, :no])
        for g in range(n_kv_heads):
            s = b * n_kv_heads + g
            o, n = int(seg_off[s]), int(seg_len[s])
            rows = []
            for h in range(g * G, (g + 1) * G):
                rows.append(to_storage(rope(q_obs[b, h, :no], qp, theta), dtype))
            qr = np.concatenate(rows, axis=0)
            qpos_rows = np.tile(qp, G)
            out[o:o + n] = segment_scores(k_cache[o:o + n], key_pos[o:o + n], qr, qpos_rows, causal, aggregate)
    return out


# ------------------------------------------------------ O5-O6: budgets
def normalized_entropy(scores):
    """Normalised Shannon entropy of one head's score distribution.

    ReasonAlloc, "Key Concepts" (head utility = normalised attention entropy).
    READING: pi_j = score_j / sum(score); E = -sum pi log pi / log n with
    0 log 0 = 0; n <= 1 or an all-zero head gives 0."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    tot = s.sum()
    if n <= 1 or tot <= 0:
        return 0.0
    pi = s / tot
    nz = pi > 0
    return float(-(pi[nz] * np.log(pi[nz])).sum() / math.log(n))


def waterfill(total, w, lo, hi):
    """Real budgets x_g = clamp(lam * w_g, lo_g, hi_g) with sum x = total.

    Proportional split with per-head floor and cap (ReasonAlloc "Core
    Mechanism": budget moves between heads, the layer total is kept).
    lo_g = min(lo, hi_g).  total >= sum(hi) gives hi; all-zero weights split
    equally.  Raises if total < sum(lo_g).  Solved exactly on the breakpoints
    of the piecewise-linear sum.
    READING (weightless heads, not on the page): a head of weight 0 keeps its
    floor while some lam meets the total; once every weighted head is at its
    cap, the rest of the total is split equally over the weightless heads
    under their caps (the limit of equal tiny weights)."""
    w = np.asarray(w, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    lo_g = np.minimum(np.asarray(lo, dtype=np.float64) * np.ones_like(hi), hi)
    if np.any(w < 0):
        raise ValueError("negative weight")
    if total >= hi.sum():
        return hi.copy()
    if total < lo_g.sum() - 1e-9:
        raise ValueError("layer total below the sum of per-head floors")
    if not np.any(w > 0):
        w = np.ones_like(w)
    pos = w > 0
    if np.any(~pos) and total > hi[pos].sum() + lo_g[~pos].sum():
        # weightless heads cannot grow with lam: weighted heads take their cap
        # and the weightless ones share what is left equally
        x = hi.copy()
        x[~pos] = waterfill(total - hi[pos].sum(), np.ones(int((~pos).sum())), lo_g[~pos], hi[~pos])
        return x

    def f(lam):
        return np.clip(lam * w, lo_g, hi).sum()

    bps = np.unique(np.concatenate([lo_g[pos] / w[pos], hi[pos] / w[pos], [0.0]]))
    vals = np.array([f(b) for b in bps])
    if total <= vals[0]:
        return np.clip(bps[0] * w, lo_g, hi)
    idx = np.searchsorted(vals, total, side="left")
    if idx >= len(bps):
        return hi.copy()
    a, b = bps[idx - 1], bps[idx]
    mid = 0.5 * (a + b)
    free = pos & (mid * w > lo_g) & (mid * w < hi)
    wf = w[free].sum()
    lam = b if wf == 0 else a + (total - vals[idx - 1]) / wf
    return np.clip(lam * w, lo_g, hi)


def largest_remainder(x, total):
    """Integerise real shares x (sum = total) by the largest-remainder rule:
    floor every share, then give +1 to the shares with the largest fractional
    parts, ties to the lower index.  READING (integerisation is not on the pages)."""
    x = np.asarray(x, dtype=np.float64)
    f = np.floor(x)
    frac = x - f
    r = int(round(total - f.sum()))
    if r < 0 or r > len(x):
        raise ValueError("shares do not sum to the total")
    order = sorted(range(len(x)), key=lambda g: (-frac[g], g))
    out = f.astype(np.int64)
    for g in order[:r]:
        out[g] += 1
    return out


def head_weights(entropy, inverse=False):
    """Head weights for the budget split.  The direct reading takes the
    normalised entropy itself; ReasonAlloc, "Key Concepts" (head utility), says
    the focused, low-entropy heads are the useful ones that gain budget, which
    is the inverse reading 1 - E (the two passages of the page disagree; both
    are offered)."""
    E = np.asarray(entropy, dtype=np.float64)
    return 1.0 - E if inverse else E


def head_budgets(weights, seg_len, layer_total, min_per_head):
    """Per-head kept counts of one (request, layer): proportional to the head
    weights (entropy), floor min_per_head, cap seg_len, summing exactly to
    min(layer_total, sum(seg_len))."""
    hi = np.asarray(seg_len, dtype=np.float64)
    x = waterfill(float(layer_total), weights, float(min_per_head), hi)
    tot = min(int(layer_total), int(hi.sum()))
    return largest_remainder(x, tot)


def layer_wave_budgets(n_layers, center, sigma, total, lo):
    """Layer-wise base budgets: a mid-peaked Gaussian over the layer index
    (ReasonAlloc "Core Mechanism": the offline Reasoning Wave), each layer's
    per-head-average budget >= lo, summing to total."""
    l = np.arange(n_layers, dtype=np.float64)
    w = np.exp(-((l - center) ** 2) / (2.0 * sigma * sigma))
    x = waterfill(float(total), w, float(lo), np.full(n_layers, float(total)))
    return largest_remainder(x, total)


# ------------------------------------------------------ O7-O8: select, compact
def select_kept(scores, n, budget, n_prefix, n_recent):
    """Kept slots of one segment, ascending.

    BeaconKV, "打分时的 RoPE 对齐": the prefix and a short recent span are
    always kept, the rest of the budget goes to the highest scores.  Ranking is
    by (score descending, slot ascending)."""
    n = int(n)
    budget = int(budget)
    if budget >= n:
        return np.arange(n)
    if budget < n_prefix + n_recent:
        raise ValueError("budget below the protected prefix + recent window")
    s = np.asarray(scores[:n], dtype=np.float64)
    cand = np.arange(n_prefix, n - n_recent)
    order = np.lexsort((cand, -s[cand]))
    chosen = cand[order[: budget - n_prefix - n_recent]]
    kept = np.concatenate([np.arange(n_prefix), chosen, np.arange(n - n_recent, n)])
    return np.sort(kept)


def compact_rows(rows, kept):
    """Stable gather: out[i] = rows[kept[i]] (BeaconKV "📊 实验": permanent eviction)."""
    return np.asarray(rows)[np.asarray(kept)]


def hole_fill(kept, n):
    """In-place compaction by hole filling.  With K = len(kept) survivors of a
    segment of n rows, survivors already in [0, K) stay where they are and the
    survivors in [K, n), in ascending order, move into the evicted slots of
    [0, K), in ascending order.  Returns src [K]: the slot whose row ends up at
    position i.  At most min(K, n - K) rows move.

    BeaconKV, "📊 实验": eviction is permanent; attention does not depend on the
    order of the cached rows (each row keeps its position, which carries RoPE
    and causality), so the survivors need not stay in slot order.  READING:
    the pairing (holes and movers both ascending) is this library's choice."""
    kept = np.sort(np.asarray(kept, dtype=np.int64))
    K = len(kept)
    keep = np.zeros(int(n), dtype=bool)
    keep[kept] = True
    holes = [j for j in range(K) if not keep[j]]
    movers = [j for j in range(K, int(n)) if keep[j]]
    assert len(holes) == len(movers)
    src = np.arange(K)
    for h, m in zip(holes, movers):
        src[h] = m
    return src


def layer_select_compact(scores, seg_off, seg_len, budgets, n_prefix, n_recent):
    """Kept slots per segment for a whole layer; returns a list of arrays."""
    out = []
    for s in range(len(seg_off)):
        o, n = int(seg_off[s]), int(seg_len[s])
        out.append(select_kept(scores[o:o + n], n, int(budgets[s]), n_prefix, n_recent))
    return out


# ------------------------------------------------------ O9: continual FPS
def _unit_rows(X):
    X = np.asarray(X, dtype=np.float64)
    nrm = np.sqrt((X * X).sum(axis=1))
    return X / np.maximum(nrm, 1e-30)[:, None]


def fps(X, k):
    """Farthest-point sampling of k rows out of the buffer X [m, d] under the
    cosine distance 1 - cos(x_r, x_r').

    BeaconKV, "Continual FPS": when a head's buffer of pre-RoPE queries fills
    to B_Q^max it is shrunk to B_Q^min by FPS in the cosine geometry of
    pre-RoPE queries.  READING: the first pick is row 0 (oldest); each step
    takes the unpicked row farthest from the picked set, ties to the lower
    row.  Returns the picks in selection order."""
    U = _unit_rows(X)
    m = U.shape[0]
    k = min(int(k), m)
    picks = [0]
    dist = 1.0 - U @ U[0]
    taken = np.zeros(m, dtype=bool)
    taken[0] = True
    for _ in range(k - 1):
        cand = np.where(taken, -np.inf, dist)
        j = int(np.argmax(cand))
        picks.append(j)
        taken[j] = True
        dist = np.minimum(dist, 1.0 - U @ U[j])
    return np.array(picks, dtype=np.int64)


def fps_acceptable(X, picks, rtol, atol=1e-6):
    """Validity of a pick sequence: at every step the row taken must be an
    unpicked row whose float64 distance to the picked set lies within
    max(rtol * best, atol) of the farthest one (best), the state being updated
    with the given picks.  Returns (ok, first_bad_step)."""
    U = _unit_rows(X)
    m = U.shape[0]
    picks = [int(p) for p in picks]
    if picks[0] != 0 or len(set(picks)) != len(picks) or any(p < 0 or p >= m for p in picks):
        return False, 0
    dist = 1.0 - U @ U[0]
    taken = np.zeros(m, dtype=bool)
    taken[0] = True
    for step, j in enumerate(picks[1:], start=1):
        best = np.where(taken, -np.inf, dist).max()
        if taken[j] or dist[j] < best - max(rtol * abs(best), atol):
            return False, step
        taken[j] = True
        dist = np.minimum(dist, 1.0 - U @ U[j])
    return True, -1


# ------------------------------------------------------ SkipKV sentence redundancy
def sentence_means(h, starts):
    """Sentence embeddings: the mean of the last-layer hidden states over each
    sentence's tokens, sentence i = tokens [starts[i], starts[i+1]).

    SkipKV page, 核心方法 §4.1 (and observation 2: the mean of last-layer
    hidden states stands in for a sentence embedding)."""
    h = np.asarray(h, dtype=np.float64)
    starts = np.asarray(starts, dtype=np.int64)
    out = np.zeros((max(len(starts) - 1, 0), h.shape[1]))
    for i in range(len(starts) - 1):
        if starts[i + 1] > starts[i]:            # READING: an empty sentence has a zero embedding
            out[i] = h[starts[i]:starts[i + 1]].mean(axis=0)
    return out


def pss_later_max(e):
    """For each sentence i, the largest pairwise sentence similarity (cosine of
    the sentence means) with any LATER sentence j > i; -1 for the last one.

    SkipKV §4.1: of a redundant pair (PSS >= tau) the earlier sentence is the
    one marked evictable, so what matters for sentence i is its most similar
    successor.  READING: a zero-norm mean has cosine 0 with everything."""
    e = np.asarray(e, dtype=np.float64)
    S = e.shape[0]
    nrm = np.sqrt((e * e).sum(axis=1))
    out = np.full(S, -1.0)
    for i in range(S):
        for j in range(i + 1, S):
            den = nrm[i] * nrm[j]
            c = float(e[i] @ e[j]) / den if den > 0 else 0.0
            out[i] = max(out[i], c)
    return out


def skipkv_token_scores(pss_max, starts, T):
    """Per-token eviction score from the sentence redundancy: token t of sentence
    i scores 1 - max(0, pss_max[i]) (a sentence that nearly repeats a later one
    scores near 0 and goes first, whole sentences together); tokens after the
    last complete sentence score 1.  READING: the page's combined score (its
    eq. 6, with token importance and a weight lambda) is not printed; this is
    the sentence term alone.  Pinned to this reading (not to the page's
    unprinted formula) by a hand example through all three steps and by
    invariants."""
    starts = np.asarray(starts, dtype=np.int64)
    sc = np.ones(int(T))
    for i in range(len(starts) - 1):
        sc[starts[i]:starts[i + 1]] = 1.0 - max(0.0, float(pss_max[i]))
    return sc


# ------------------------------------------------------ decode attention
def decode_attention(k, v, q):
    """Attention of the new token's queries over one KV head's cache: for each
    query row, softmax(q . k / sqrt(d)) over every cached row, applied to V.
    Returns (out [rows, d], lse [rows], natural log).

    The step that follows eviction in the decode loop (EPIKV page, part 4:
    the eviction score stays compatible with a fused attention kernel; the
    BeaconKV page's throughput figures are decode throughput over the
    compacted cache).  Every cached row is visible to the new token, and the
    result does not depend on the order of the rows."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    logits = q @ k.T / math.sqrt(k.shape[1])
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, (m + np.log(l))[:, 0]


# ------------------------------------------------------ O10: EPIKV
def epikv_g(h):
    """g(t) = ||h(t) - h(t-1)||_2 for t >= 1; g(0) = 0.

    EPIKV, part 1 (顿悟得分): the step-to-step L2 change of one layer's hidden state."""
    h = np.asarray(h, dtype=np.float64)
    g = np.zeros(h.shape[0])
    if h.shape[0] > 1:
        diff = h[1:] - h[:-1]
        g[1:] = np.sqrt((diff * diff).sum(axis=1))
    return g


def rolling_z(g, window, eps):
    """Causal rolling z-score z(t) = (g(t) - mu(t)) / (sigma(t) + eps).

    EPIKV, part 3 (时间趋势校正).  READING: the window is
    {max(1, t-W+1), ..., t} (g(0) excluded, warm-up windows truncated),
    sigma is the population standard deviation, z(0) = 0."""
    g = np.asarray(g, dtype=np.float64)
    T = g.shape[0]
    z = np.zeros(T)
    for t in range(1, T):
        u = g[max(1, t - window + 1): t + 1]
        mu = u.mean()
        sd = math.sqrt(((u - mu) ** 2).mean())
        z[t] = (g[t] - mu) / (sd + eps)
    return z


def rolling_mean(g, window):
    """Causal rolling mean g_bar(t) over the same window as rolling_z:
    {max(1, t-W+1), ..., t}; g_bar(0) = 0.

    EPIKV, part 2 (双带层解剖结构): the band score is stated on rolling means of g."""
    g = np.asarray(g, dtype=np.float64)
    T = g.shape[0]
    m = np.zeros(T)
    for t in range(1, T):
        m[t] = g[max(1, t - window + 1): t + 1].mean()
    return m


def epikv_score(h_a, h_b, window, eps, form="z"):
    """Eviction score; higher keeps.  h_a, h_b: [T, d_model] hidden states of
    the two layers.  form="z": s(t) = z_a(t) - z_b(t) (EPIKV, part 3:
    z_10 - z_21, the trend-corrected score); form="mean": s(t) = g_bar_a(t) -
    g_bar_b(t) (EPIKV, part 2: the rolling-mean form stated first)."""
    if form == "mean":
        return rolling_mean(epikv_g(h_a), window) - rolling_mean(epikv_g(h_b), window)
    if form != "z":
        raise ValueError(form)
    return rolling_z(epikv_g(h_a), window, eps) - rolling_z(epikv_g(h_b), window, eps)
