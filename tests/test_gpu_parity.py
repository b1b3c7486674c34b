"""GPU library vs CPU oracle, element by element, on seeded inputs.

Sizes are ones the oracle finishes in seconds but that span many 64-key tiles,
several 256-key chunks and ragged tails.  All calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle
from tests.gpu_side import device_layer, score_layer, alloc_out, select_compact
from tests.oracle_side import oracle_cache_keys, oracle_layer_scores, np64
from tests.parity import assert_scores_close, budgets_match, kept_matches
from workloads import get_workload, make_layer, make_traces

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-f32": get_workload("tiny-f32"),
    "qwen3-4b-1l": get_workload("qwen3-4b-1l"),
    "llama-ragged": get_workload("r1-llama-8b").scaled(batch=3, len_lo=700, len_hi=1100, n_layers=1),
    "long-5k": get_workload("long-65k").scaled(batch=1, len_lo=5000, len_hi=5000),
    "qwen-short": get_workload("qwen3-4b-1l").scaled(batch=2, len_lo=333, len_hi=333, budget=300),
}
BUDGET = {"llama-ragged": 640, "long-5k": 1024}


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
        k_orc = oracle_cache_keys(L, w)
        _cache[name] = (w, L, D, k_orc, oracle_layer_scores(L, w, k_orc))
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_rope_keys_bit_exact(name):
    w, L, D, k_orc, _ = _case(name)
    torch.cuda.synchronize()
    got = D["k"].float().cpu().numpy().astype(np.float64)
    mism = int((got != k_orc).sum())
    assert mism == 0, f"{mism} of {got.size} rotated key elements differ"


@pytest.mark.parametrize("impl", ["mfma", "fused", "valu"])
@pytest.mark.parametrize("name", list(CASES))
def test_scores_match_oracle(name, impl, kve_overrides):
    w, L, D, k_orc, s_orc = _case(name)
    if impl != "mfma":
        if w.dtype != "bf16":
            pytest.skip("fp32 caches always use the VALU path")
        kve_overrides(score_impl=impl)
    scores, ent = score_layer(D, w, entropy=True)
    torch.cuda.synchronize()
    g = scores.cpu().numpy()
    worst = assert_scores_close(g, s_orc)
    print(f"{name}/{impl}: worst relative score error {worst:.2e}")
    # head entropy from the same kernel call
    e = ent.cpu().numpy()
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        want = oracle.normalized_entropy(s_orc[o:o + n])
        assert abs(e[s] - want) <= 2e-3 * max(abs(want), 1e-3), (s, e[s], want)


def test_single_read_scoring_long_segments(kve_overrides):
    """The single-read scoring kernel on segments of 32,768 keys: its
    work-groups meet at a per-segment barrier, so each segment is cut into at
    most 12 chunks (with the two-pass chunk it would span 128, enough waiting
    work-groups to fill an XCD while the next work-group in launch order waits
    for a slot there).  Every segment completes (no failure marks) and matches
    the oracle."""
    w = get_workload("long-65k").scaled(batch=1, len_lo=32768, len_hi=32768)
    L = make_layer(w, 0)
    D = device_layer(L, w)
    k_orc = oracle_cache_keys(L, w)
    s_orc = oracle_layer_scores(L, w, k_orc)
    kve_overrides(score_impl="fused")
    scores, _ = score_layer(D, w, entropy=False)
    torch.cuda.synchronize()
    g = scores.cpu().numpy()
    assert np.isfinite(g).all(), f"{int((~np.isfinite(g)).sum())} scores not finite"
    worst = assert_scores_close(g, s_orc)
    print(f"long-32k/fused: worst relative score error {worst:.2e}")


@pytest.mark.parametrize("name", list(CASES))
def test_select_compact_match_oracle(name):
    w, L, D, k_orc, s_orc = _case(name)
    budget = BUDGET.get(name, w.budget)
    scores, _ = score_layer(D, w)
    out = alloc_out(D, w, budget)
    select_compact(D, w, scores, out, uniform=budget)
    torch.cuda.synchronize()
    kept = out["kept"].cpu().numpy()
    seg_len = out["seg_len"].cpu().numpy()
    k_in = D["k"].view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    v_in = D["v"].view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    k_out = out["k"].view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    v_out = out["v"].view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    pos_in, pos_out = D["pos"].cpu().numpy(), out["pos"].cpu().numpy()
    swaps = 0
    for s in range(len(L["seg_len"])):
        o, n = int(L["seg_off"][s]), int(L["seg_len"][s])
        want_len = min(budget, n)
        assert seg_len[s] == want_len
        oo = s * budget
        ks = kept[oo:oo + want_len]
        ok, sw, msg = kept_matches(ks, s_orc[o:o + n], n, budget, w.n_prefix, w.n_recent)
        assert ok, f"segment {s}: {msg}"
        swaps += sw
        # compaction is a byte-exact gather of the GPU's own kept slots
        assert np.array_equal(k_out[oo:oo + want_len], k_in[o + ks])
        assert np.array_equal(v_out[oo:oo + want_len], v_in[o + ks])
        assert np.array_equal(pos_out[oo:oo + want_len], pos_in[o + ks])
        # and equals the oracle's compaction wherever the kept sets agree
        want = oracle.select_kept(s_orc[o:o + n], n, budget, w.n_prefix, w.n_recent)
        if np.array_equal(want, ks):
            ko = oracle.compact_rows(k_orc[o:o + n], want)
            assert np.array_equal(D["k"][o:o + n].float().cpu().numpy()[want], ko)
    print(f"{name}: {swaps} tie-band swaps")


def _select_scores(n_seg, n, scores_np, budget, P=4, R=16, ws=None):
    """Run select/compact on given per-row scores over a synthetic bf16 cache
    (ws None: the workspace the library asks for)."""
    dev = "cuda"
    rows = n_seg * n
    k = torch.arange(rows * 128, dtype=torch.float32, device=dev).view(rows, 128).to(torch.bfloat16)
    v = -k
    pos = torch.arange(rows, dtype=torch.int32, device=dev)
    seg_off = torch.arange(n_seg, dtype=torch.int64, device=dev) * n
    seg_len = torch.full((n_seg,), n, dtype=torch.int32, device=dev)
    cin = kv.make_cache(k, v, pos, seg_off, seg_len, 1, n)
    cap = min(budget, n)
    ok_, ov_ = torch.zeros(n_seg * cap, 128, dtype=torch.bfloat16, device=dev), torch.zeros(n_seg * cap, 128, dtype=torch.bfloat16, device=dev)
    op = torch.zeros(n_seg * cap, dtype=torch.int32, device=dev)
    oo = torch.arange(n_seg, dtype=torch.int64, device=dev) * cap
    ol = torch.zeros(n_seg, dtype=torch.int32, device=dev)
    kept = torch.zeros(n_seg * cap, dtype=torch.int32, device=dev)
    cout = kv.make_cache(ok_, ov_, op, oo, ol, 1, cap)
    sc = torch.from_numpy(np.asarray(scores_np, dtype=np.float32)).to(dev)
    kv.kv_evict_select_compact(cin, sc, None, P, R, cout, kept_idx=kept, uniform_budget=budget, ws=ws)
    torch.cuda.synchronize()
    return kept.cpu().numpy().reshape(n_seg, cap), ol.cpu().numpy(), op.cpu().numpy().reshape(n_seg, cap)


def test_select_ties_signs_and_edges():
    n = 1500
    rng = np.random.default_rng(0)
    cases = [
        np.full(n, 0.5),                                            # all tied: lowest candidates win
        rng.integers(0, 4, n).astype(np.float64),                   # heavy ties on few values
        rng.standard_normal(n),                                     # signed scores
        np.where(rng.random(n) < 0.5, -0.0, 0.0),                   # -0.0 ties with +0.0
        rng.random(n) * 1e-35,                                      # subnormal-range values
    ]
    for budget in (20, 21, 700, 1499, 1500, 4000):
        sc = np.stack(cases)
        kept, lens, pos = _select_scores(len(cases), n, sc.reshape(-1), budget)
        for i, s in enumerate(cases):
            want = oracle.select_kept(s, n, budget, 4, 16)
            assert lens[i] == len(want)
            assert np.array_equal(kept[i][:lens[i]], want), (i, budget)
            assert np.array_equal(pos[i][:lens[i]], i * n + want)


@pytest.mark.parametrize("form", ["split", "one"])
@pytest.mark.parametrize("n", [12289, 40000])
def test_select_long_segments_ties_and_edges(n, form):
    """Segments longer than the selection's LDS key store (12,288) take the
    1024-thread kernels that re-read the scores per radix pass: with the
    workspace the library asks for, few segments are split over several
    work-groups each ("split"); without it, one work-group per segment
    ("one").  The same kept sets as the oracle, ties and signed values
    included."""
    ws = torch.empty(0, dtype=torch.uint8, device="cuda") if form == "one" else None
    rng = np.random.default_rng(n)
    cases = [
        np.full(n, 0.25),
        rng.integers(0, 5, n).astype(np.float64),
        rng.standard_normal(n),
        np.exp(-30 * rng.random(n)),                                # scores over many binades
    ]
    for budget in (20, 21, n // 3, n - 1):
        sc = np.stack(cases)
        kept, lens, pos = _select_scores(len(cases), n, sc.reshape(-1), budget, ws=ws)
        for i, s in enumerate(cases):
            want = oracle.select_kept(s.astype(np.float32).astype(np.float64), n, budget, 4, 16)
            assert lens[i] == len(want)
            assert np.array_equal(kept[i][:lens[i]], want), (i, budget)
            assert np.array_equal(pos[i][:lens[i]], i * n + want)


def _split_case(seed=5):
    """Ragged long and short segments with per-segment budgets (some keeping
    every row, one rejected) over a synthetic bf16 cache."""
    rng = np.random.default_rng(seed)
    lens = np.array([30000, 12289, 500, 20000, 17, 25000, 14000, 9000], dtype=np.int64)
    budgets = np.array([7000, 12289, 600, 19999, 17, 10, 300, 20], dtype=np.int32)   # [5] below P + R: rejected
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = int(lens.sum())
    scores = np.concatenate([
        np.exp(-25 * rng.random(n)) if i % 2 else rng.integers(0, 50, n).astype(np.float64)
        for i, n in enumerate(lens)])
    dev = "cuda"
    k = torch.arange(rows * 128, dtype=torch.float32, device=dev).view(rows, 128).to(torch.bfloat16)
    pos = torch.arange(rows, dtype=torch.int32, device=dev)
    cin = kv.make_cache(k, -k, pos, torch.from_numpy(offs).to(dev), torch.from_numpy(lens.astype(np.int32)).to(dev),
                        1, int(lens.max()))
    cap = int(lens.max())
    n_seg = len(lens)
    out = {"k": torch.zeros(n_seg * cap, 128, dtype=torch.bfloat16, device=dev),
           "v": torch.zeros(n_seg * cap, 128, dtype=torch.bfloat16, device=dev),
           "pos": torch.zeros(n_seg * cap, dtype=torch.int32, device=dev),
           "off": torch.arange(n_seg, dtype=torch.int64, device=dev) * cap,
           "len": torch.full((n_seg,), -9, dtype=torch.int32, device=dev),
           "kept": torch.full((n_seg * cap,), -5, dtype=torch.int32, device=dev)}
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["off"], out["len"], 1, cap)
    sc = torch.from_numpy(scores.astype(np.float32)).to(dev)
    bud = torch.from_numpy(budgets).to(dev)
    return lens, offs, budgets, scores, cin, cout, sc, bud, out, cap


def _check_split(lens, offs, budgets, scores, out, cap, allow_failed):
    got_len = out["len"].cpu().numpy()
    kept = out["kept"].cpu().numpy()
    pos = out["pos"].cpu().numpy()
    for s, (n, o, b) in enumerate(zip(lens, offs, budgets)):
        if b < n and b < 20:                       # below prefix + recent: rejected
            assert got_len[s] == -1, (s, got_len[s])
            continue
        if allow_failed and got_len[s] == -1:
            continue
        want = oracle.select_kept(scores[o:o + n].astype(np.float32).astype(np.float64), int(n), int(b), 4, 16)
        assert got_len[s] == len(want), (s, got_len[s], len(want))
        assert np.array_equal(kept[s * cap:s * cap + len(want)], want), s
        assert np.array_equal(pos[s * cap:s * cap + len(want)], o + want), s


def test_select_split_budgets_and_failed_meetings(kve_overrides):
    """The several-work-groups-per-segment selection with per-segment budgets
    over ragged segments (long and short, budgets keeping everything, a
    rejected one) matches the oracle; with the meeting poll bound forced to
    one poll from the host, segments whose work-groups did not meet report -1
    and every other one is exact; a later call with the default bound is
    whole again."""
    lens, offs, budgets, scores, cin, cout, sc, bud, out, cap = _split_case()
    kv.kv_evict_select_compact(cin, sc, bud, 4, 16, cout, kept_idx=out["kept"])
    torch.cuda.synchronize()
    _check_split(lens, offs, budgets, scores, out, cap, allow_failed=False)
    kve_overrides(spin_limit=1)
    out["len"].fill_(-9)
    kv.kv_evict_select_compact(cin, sc, bud, 4, 16, cout, kept_idx=out["kept"])
    torch.cuda.synchronize()
    _check_split(lens, offs, budgets, scores, out, cap, allow_failed=True)
    kve_overrides(spin_limit=0)
    out["len"].fill_(-9)
    kv.kv_evict_select_compact(cin, sc, bud, 4, 16, cout, kept_idx=out["kept"])
    torch.cuda.synchronize()
    _check_split(lens, offs, budgets, scores, out, cap, allow_failed=False)


def test_select_rejects_budget_below_protected():
    with pytest.raises(kv.KveError) as ei:
        _select_scores(1, 100, np.zeros(100), 19)
    assert ei.value.name == "KVE_EBUDGET"


def test_budgets_match_oracle():
    rng = np.random.default_rng(1)
    B, H = 57, 8
    w = rng.random((B, H)).astype(np.float32)
    w[rng.random((B, H)) < 0.05] = 0.0
    cap = rng.integers(30, 9000, (B, H)).astype(np.int32)
    tot = rng.integers(8 * 64, 8 * 3000, B).astype(np.int32)
    dev = "cuda"
    out = torch.zeros(B * H, dtype=torch.int32, device=dev)
    kv.kv_evict_budgets(torch.from_numpy(w).to(dev), torch.from_numpy(tot).to(dev), torch.from_numpy(cap).to(dev),
                        B, H, 64, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B, H)
    for b in range(B):
        lo = np.minimum(64, cap[b]).sum()
        if tot[b] < lo:
            assert np.all(got[b] == -1)
            continue
        want = oracle.head_budgets(w[b].astype(np.float64), cap[b], int(tot[b]), 64)
        assert np.array_equal(got[b], want), (b, got[b], want)
    wave = torch.zeros(32, dtype=torch.int32, device=dev)
    kv.kv_evict_wave_budgets(32, 16.0, 6.0, 32 * 1024, 64, wave)
    torch.cuda.synchronize()
    assert np.array_equal(wave.cpu().numpy(), oracle.layer_wave_budgets(32, 16.0, 6.0, 32 * 1024, 64))


@pytest.mark.parametrize("name", ["tiny-f32", "qwen3-4b-1l"])
def test_fps_matches_oracle(name):
    w, L, D, _, _ = _case(name)
    buf = D["fps_buf"].clone()
    n_buf, cap, d = buf.shape
    count = D["fps_count"].clone()
    count[::7] = cap - 3                                   # some buffers not full: untouched
    out = torch.zeros_like(buf)
    cnt_out = torch.zeros_like(count)
    picks = torch.zeros(n_buf, w.fps_keep, dtype=torch.int32, device=buf.device)
    kv.beacon_fps_update(buf, out, count, cnt_out, w.fps_keep, picks)
    # in place on a copy must give the same buffer
    inplace = buf.clone()
    cnt_in = count.clone()
    kv.beacon_fps_update(inplace, inplace, cnt_in, cnt_in, w.fps_keep)
    torch.cuda.synchronize()
    X = np64(D["fps_buf"])
    P = picks.cpu().numpy()
    co = cnt_out.cpu().numpy()
    exact = 0
    for p in range(n_buf):
        if p % 7 == 0:
            assert co[p] == cap - 3 and np.all(P[p] == -1)
            assert torch.equal(out[p, :cap - 3], buf[p, :cap - 3])
            continue
        assert co[p] == w.fps_keep
        ok, step = oracle.fps_acceptable(X[p], P[p], 2e-3)
        assert ok, f"buffer {p}: pick {step} not a farthest point ({P[p].tolist()})"
        want = oracle.fps(X[p], w.fps_keep)
        exact += int(np.array_equal(want, P[p]))
        rows = np.sort(P[p])
        assert torch.equal(out[p, :w.fps_keep], buf[p, rows.tolist()])
    assert torch.equal(inplace[:, :w.fps_keep][1::7], out[:, :w.fps_keep][1::7])
    assert torch.equal(cnt_in, cnt_out)
    print(f"{name}: {exact}/{n_buf - len(range(0, n_buf, 7))} pick sequences identical to the oracle's")


@pytest.mark.parametrize("cap,k_keep,d", [(64, 33, 128), (40, 20, 64), (16, 8, 128), (17, 1, 64)])
def test_fps_capacities_and_head_sizes(cap, k_keep, d):
    """Capacities that are not a multiple of the 16-row tiles, the 64-row limit,
    both head sizes, k_keep = 1; some buffers not full (copied through)."""
    g = torch.Generator().manual_seed(cap * 1000 + k_keep)
    n_buf = 37
    buf = (torch.randn(n_buf, cap, d, generator=g) + 0.3 * torch.randn(n_buf, 1, d, generator=g)).to(torch.bfloat16)
    buf = buf.cuda()
    count = torch.full((n_buf,), cap, dtype=torch.int32, device="cuda")
    count[::5] = cap // 2
    out = torch.zeros_like(buf)
    cnt_out = torch.zeros_like(count)
    picks = torch.zeros(n_buf, k_keep, dtype=torch.int32, device="cuda")
    kv.beacon_fps_update(buf, out, count, cnt_out, k_keep, picks)
    torch.cuda.synchronize()
    X = np64(buf)
    P = picks.cpu().numpy()
    for p in range(n_buf):
        if p % 5 == 0:
            assert int(cnt_out[p]) == cap // 2 and np.all(P[p] == -1)
            assert torch.equal(out[p, :cap // 2], buf[p, :cap // 2])
            continue
        assert int(cnt_out[p]) == k_keep
        ok, step = oracle.fps_acceptable(X[p], P[p], 2e-3)
        assert ok, f"buffer {p}: pick {step} not a farthest point"
        assert torch.equal(out[p, :k_keep], buf[p, np.sort(P[p]).tolist()])


@pytest.mark.parametrize("Dm,T", [(512, 1500), (1024, 901), (2048, 777), (4096, 1500), (8192, 333)])
def test_epikv_matches_oracle(Dm, T):
    """Per-wave runs below d_model 2048, row-batched work-group runs from 2048
    on (ragged last batch and run at these T)."""
    w = get_workload("long-65k")
    B, W = 2, 256
    h = make_traces(w, T=T, d_model=Dm, batch=B)
    hd = h.cuda()
    scores = torch.zeros(B, T, dtype=torch.float32, device="cuda")
    g = torch.zeros(2, B, T, dtype=torch.float32, device="cuda")
    kv.epikv_score(hd[0], hd[1], W, w.epikv_eps, scores, g_out=g)
    torch.cuda.synchronize()
    hn = np64(h)
    for b in range(B):
        ga = oracle.epikv_g(hn[0, b])
        gb = oracle.epikv_g(hn[1, b])
        assert_scores_close(g[0, b].cpu().numpy(), ga, rtol=1e-5, floor=1e-6, what="g")
        assert_scores_close(g[1, b].cpu().numpy(), gb, rtol=1e-5, floor=1e-6, what="g")
        want = oracle.epikv_score(hn[0, b], hn[1, b], W, w.epikv_eps)
        got = scores[b].cpu().numpy().astype(np.float64)
        err = np.abs(got - want)
        assert np.all(err <= 2e-3 * np.maximum(1.0, np.abs(want))), float(err.max())


def test_epikv_scores_drive_selection_for_every_head():
    """One per-token score per request, shared by all KV heads via score_off."""
    w = get_workload("long-65k").scaled(batch=2, len_lo=1500, len_hi=1500)
    L = make_layer(w, 0)
    D = device_layer(L, w)
    h = make_traces(w, T=1500, d_model=512, batch=2).cuda()
    scores = torch.zeros(2, 1500, dtype=torch.float32, device="cuda")
    kv.epikv_score(h[0], h[1], 256, w.epikv_eps, scores)
    score_off = (torch.arange(2 * w.n_kv_heads, device="cuda") // w.n_kv_heads * 1500).to(torch.int64)
    budget = 400
    out = alloc_out(D, w, budget)
    select_compact(D, w, scores.view(-1), out, uniform=budget, score_off=score_off)
    torch.cuda.synchronize()
    hn = np64(h.cpu())
    kept = out["kept"].cpu().numpy()
    for b in range(2):
        s_orc = oracle.epikv_score(hn[0, b], hn[1, b], 256, w.epikv_eps)
        for g in range(w.n_kv_heads):
            s = b * w.n_kv_heads + g
            ok, _, msg = kept_matches(kept[s * budget:(s + 1) * budget], s_orc, 1500, budget, 4, 16, rtol=2e-3,
                                      floor=2e-3)
            assert ok, msg


def test_invalid_arguments_raise_before_launch():
    w, L, D, _, _ = _case("qwen-short")
    from tests.gpu_side import cache_of, obs_of
    c, o = cache_of(D, w), obs_of(D, w)
    scores = torch.zeros(D["k"].shape[0], device="cuda")
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score(c, o, D["k"].view(-1)[:10].float(), ws=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "KVE_EWORKSPACE"
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_score(c, o, D["k"].view(torch.float32).view(-1))   # scores aliasing the keys
    assert ei.value.name == "KVE_EALIAS"
    out = alloc_out(D, w, 300)
    from decode_kv_cache_evict_amd import make_cache
    cout = make_cache(D["k"], D["v"], D["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, 300)
    with pytest.raises(kv.KveError) as ei:
        kv.kv_evict_select_compact(c, scores, None, 4, 16, cout, kept_idx=out["kept"], uniform_budget=300)
    assert ei.value.name == "KVE_EALIAS"


def test_entropy_budgets_drive_variable_k_selection():
    """Scores with head entropy -> per-head budgets (layer total from the wave
    table) -> variable-K selection, all on the GPU, against the oracle."""
    w = CASES["llama-ragged"]
    w_, L, D, k_orc, s_orc = _case("llama-ragged")
    n_layers, layer = 32, 9
    table = torch.zeros(n_layers, dtype=torch.int32, device="cuda")
    kv.kv_evict_wave_budgets(n_layers, w.wave_center, w.wave_sigma, 8 * 1024, 64 // 4, table)
    scores, ent = score_layer(D, w, entropy=True)
    torch.cuda.synchronize()
    tab = table.cpu().numpy()
    assert np.array_equal(tab, oracle.layer_wave_budgets(n_layers, w.wave_center, w.wave_sigma, 8 * 1024, 16))
    total = torch.full((w.batch,), int(w.n_kv_heads * tab[layer]), dtype=torch.int32, device="cuda")
    bud = torch.zeros(w.batch * w.n_kv_heads, dtype=torch.int32, device="cuda")
    kv.kv_evict_budgets(ent, total, D["seg_len"], w.batch, w.n_kv_heads, 24, bud)
    out = alloc_out(D, w, int(max(L["lengths"])))
    select_compact(D, w, scores, out, budget=bud)
    torch.cuda.synchronize()
    g_bud, g_ent = bud.cpu().numpy(), ent.cpu().numpy()
    kept = out["kept"].cpu().numpy()
    lens = out["seg_len"].cpu().numpy()
    cap = out["cap"]
    for b in range(w.batch):
        segs = range(b * w.n_kv_heads, (b + 1) * w.n_kv_heads)
        n = [int(L["seg_len"][s]) for s in segs]
        E = np.array([oracle.normalized_entropy(s_orc[int(L["seg_off"][s]):int(L["seg_off"][s]) + n[i]])
                      for i, s in enumerate(segs)])
        got = g_bud[b * w.n_kv_heads:(b + 1) * w.n_kv_heads]
        ok, msg = budgets_match(got, g_ent[list(segs)], E, n, int(w.n_kv_heads * tab[layer]), 24)
        assert ok, f"request {b}: {msg}"
        for i, s in enumerate(segs):
            assert lens[s] == got[i]
            o = int(L["seg_off"][s])
            ok, _, msg = kept_matches(kept[s * cap:s * cap + got[i]], s_orc[o:o + n[i]], n[i], int(got[i]), 4, 16)
            assert ok, msg
