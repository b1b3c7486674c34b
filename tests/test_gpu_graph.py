"""A captured HIP graph of the eviction step replays to the eager result.

The step (FPS on a second stream, per-layer score -> select/compact with the
gather of layer l on the second stream) is captured once and replayed several
times; outputs are cleared eagerly between replays and every replay must
reproduce the eager outputs bit for bit."""
import pytest
import torch

import decode_kv_cache_evict_amd as kv
from tests.gpu_side import device_layer
from workloads import get_workload, make_layer

pytestmark = pytest.mark.gpu


def _step(layers, w, outs, scores, ws, side, fps_out):
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    for li, (D, out, ev) in enumerate(zip(layers, outs, fps_out["ev"])):
        c = kv.make_cache(D["k"], D["v"], D["pos"], D["seg_off"], D["seg_len"], w.n_kv_heads, D["max_len"])
        o = kv.make_obs(D["q_obs"], D["q_pos"], D["n_obs"], w.rope_theta)
        kv.beacon_fps_update(D["fps_buf"], fps_out["buf"][li], D["fps_count"], fps_out["cnt"][li], w.fps_keep,
                             stream=side)
        kv.kv_evict_score(c, o, scores[li], ws=ws, stream=main)
        ev.record(main)
        side.wait_event(ev)
        co = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, w.budget)
        kv.kv_evict_select_compact(c, scores[li], None, w.n_prefix, w.n_recent, co, kept_idx=out["kept"],
                                   uniform_budget=w.budget, stream=side)
    main.wait_stream(side)


def _outputs(outs, scores, fps_out):
    return [t.clone() for o in outs for t in (o["k"], o["v"], o["pos"], o["seg_len"], o["kept"])] + \
           [s.clone() for s in scores] + [b.clone() for b in fps_out["buf"]] + [c.clone() for c in fps_out["cnt"]]


def _clear(outs, scores, fps_out):
    for o in outs:
        for key in ("k", "v", "pos", "seg_len", "kept"):
            o[key].zero_()
    for s in scores:
        s.zero_()
    for b in fps_out["buf"]:
        b.zero_()
    for c in fps_out["cnt"]:
        c.zero_()


def test_captured_step_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = get_workload("qwen3-4b-1l").scaled(batch=3, len_lo=900, len_hi=900, budget=800)
    layers = [device_layer(make_layer(w, l), w) for l in range(3)]
    S = w.batch * w.n_kv_heads
    outs = []
    for _ in layers:
        outs.append({"k": torch.zeros(S * w.budget, w.head_dim, dtype=torch.bfloat16, device="cuda"),
                     "v": torch.zeros(S * w.budget, w.head_dim, dtype=torch.bfloat16, device="cuda"),
                     "pos": torch.zeros(S * w.budget, dtype=torch.int32, device="cuda"),
                     "seg_off": torch.arange(S, dtype=torch.int64, device="cuda") * w.budget,
                     "seg_len": torch.zeros(S, dtype=torch.int32, device="cuda"),
                     "kept": torch.zeros(S * w.budget, dtype=torch.int32, device="cuda")})
    scores = [torch.zeros(D["k"].shape[0], device="cuda") for D in layers]
    fps_out = {"buf": [torch.zeros_like(D["fps_buf"]) for D in layers],
               "cnt": [torch.zeros_like(D["fps_count"]) for D in layers],
               "ev": [torch.cuda.Event() for _ in layers]}
    D0 = layers[0]
    c0 = kv.make_cache(D0["k"], D0["v"], D0["pos"], D0["seg_off"], D0["seg_len"], w.n_kv_heads, D0["max_len"])
    o0 = kv.make_obs(D0["q_obs"], D0["q_pos"], D0["n_obs"], w.rope_theta)
    ws = torch.empty(kv.kv_evict_score_workspace(c0, o0) + 256, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    _step(layers, w, outs, scores, ws, side, fps_out)
    torch.cuda.synchronize()
    want = _outputs(outs, scores, fps_out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(layers, w, outs, scores, ws, side, fps_out)
    for rep in range(4):
        _clear(outs, scores, fps_out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(outs, scores, fps_out)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"
        _step(layers, w, outs, scores, ws, side, fps_out)        # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("form", ["copy", "inplace", "budget"])
def test_captured_one_call_triggers_replay_match_eager(form):
    """The one-kernel triggers (work tickets and meeting counters cleared by a
    kernel inside each call, so a graph holds no memset node) captured once and
    replayed several times, with eager calls between the replays: every replay
    reproduces the eager outputs bit for bit.  The in-place form rewrites the
    cache, which is restored eagerly before every call."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = get_workload("r1-llama-8b").scaled(batch=3, len_lo=900, len_hi=1500, n_layers=1)
    D = device_layer(make_layer(w, 0), w)
    S = w.batch * w.n_kv_heads
    cap = D["max_len"]
    c = kv.make_cache(D["k"], D["v"], D["pos"], D["seg_off"], D["seg_len"], w.n_kv_heads, D["max_len"])
    o = kv.make_obs(D["q_obs"], D["q_pos"], D["n_obs"], w.rope_theta)
    pristine = [D[k].clone() for k in ("k", "v", "pos")]
    scores = torch.zeros(D["k"].shape[0], device="cuda")
    out = {"k": torch.zeros(S * cap, w.head_dim, dtype=torch.bfloat16, device="cuda"),
           "v": torch.zeros(S * cap, w.head_dim, dtype=torch.bfloat16, device="cuda"),
           "pos": torch.zeros(S * cap, dtype=torch.int32, device="cuda"),
           "seg_off": torch.arange(S, dtype=torch.int64, device="cuda") * cap,
           "seg_len": torch.zeros(S, dtype=torch.int32, device="cuda"),
           "kept": torch.zeros(S * cap, dtype=torch.int32, device="cuda")}
    co = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, cap)
    ent = torch.zeros(S, device="cuda")
    bud = torch.zeros(S, dtype=torch.int32, device="cuda")
    new_len = torch.zeros(S, dtype=torch.int32, device="cuda")
    totals = torch.full((w.batch,), 300 * w.n_kv_heads, dtype=torch.int32, device="cuda")
    budget = 700
    if form == "copy":
        ws = torch.empty(kv.kv_evict_score_select_compact_workspace(c, o, co, True) + 256, dtype=torch.uint8,
                         device="cuda")
        call = lambda: kv.kv_evict_score_select_compact(c, o, scores, None, w.n_prefix, w.n_recent, co,  # noqa: E731
                                                        kept_idx=out["kept"], uniform_budget=budget, ws=ws)
        outputs = lambda: [scores, out["k"], out["v"], out["pos"], out["seg_len"], out["kept"]]  # noqa: E731
    elif form == "inplace":
        ws = torch.empty(kv.kv_evict_score_select_compact_inplace_workspace(c, o) + 256, dtype=torch.uint8,
                         device="cuda")
        call = lambda: kv.kv_evict_score_select_compact_inplace(c, o, scores, None, w.n_prefix, w.n_recent,  # noqa: E731
                                                                new_len, uniform_budget=budget, ws=ws)
        outputs = lambda: [scores, D["k"], D["v"], D["pos"], new_len]  # noqa: E731
    else:
        ws = torch.empty(kv.kv_evict_score_budget_select_compact_workspace(c, o, co, True, True) + 256,
                         dtype=torch.uint8, device="cuda")
        call = lambda: kv.kv_evict_score_budget_select_compact(c, o, scores, ent, totals, 24, w.n_prefix,  # noqa: E731
                                                               w.n_recent, co, budget_out=bud, kept_idx=out["kept"],
                                                               ws=ws)
        outputs = lambda: [scores, ent, bud, out["k"], out["v"], out["pos"], out["seg_len"], out["kept"]]  # noqa: E731

    def reset():
        for t, p in zip((D["k"], D["v"], D["pos"]), pristine):
            t.copy_(p)
        for t in (scores, ent, bud, new_len, *out.values()):
            if t is not out["seg_off"]:
                t.zero_()

    reset()
    call()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs()]
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(), want)):
            assert torch.equal(a, b), f"{form} replay {rep}: output {i} differs from the eager call"
        reset()
        call()                                                  # eager work between replays
        torch.cuda.synchronize()
