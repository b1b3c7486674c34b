"""Run the GPU library on generator output (GPU tests, smoke and bench)."""
import torch

import decode_kv_cache_evict_amd as kv


def to_device(L, device="cuda"):
    return {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in L.items()}


def device_layer(L, w, device="cuda"):
    """Lay one generated layer out on the GPU; keys are rotated by kv_rope_apply."""
    D = to_device(L, device)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    k = torch.empty(D["k_pre"].shape, dtype=dt, device=device)
    kv.kv_rope_apply(D["k_pre"].contiguous(), k, D["pos"], w.rope_theta)
    D["k"] = k
    D["max_len"] = int(max(L["lengths"]))
    return D


def cache_of(D, w):
    return kv.make_cache(D["k"], D["v"], D["pos"], D["seg_off"], D["seg_len"], w.n_kv_heads, D["max_len"])


def obs_of(D, w, aggregate=0):
    return kv.make_obs(D["q_obs"], D["q_pos"], D["n_obs"], w.rope_theta, bool(w.causal), aggregate)


def score_layer(D, w, entropy=False, aggregate=0):
    scores = torch.zeros(D["k"].shape[0], dtype=torch.float32, device=D["k"].device)
    ent = torch.zeros(D["seg_off"].numel(), dtype=torch.float32, device=D["k"].device) if entropy else None
    kv.kv_evict_score(cache_of(D, w), obs_of(D, w, aggregate), scores, ent)
    return scores, ent


def alloc_out(D, w, cap):
    n_seg = D["seg_off"].numel()
    dev = D["k"].device
    out = {
        "k": torch.zeros(n_seg * cap, w.head_dim, dtype=D["k"].dtype, device=dev),
        "v": torch.zeros(n_seg * cap, w.head_dim, dtype=D["v"].dtype, device=dev),
        "pos": torch.full((n_seg * cap,), -7, dtype=torch.int32, device=dev),
        "seg_off": torch.arange(n_seg, dtype=torch.int64, device=dev) * cap,
        "seg_len": torch.full((n_seg,), -9, dtype=torch.int32, device=dev),
        "kept": torch.full((n_seg * cap,), -5, dtype=torch.int32, device=dev),
        "cap": cap,
    }
    return out


def select_compact(D, w, scores, out, budget=None, uniform=0, score_off=None):
    cin = cache_of(D, w)
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, out["cap"])
    kv.kv_evict_select_compact(cin, scores, budget, w.n_prefix, w.n_recent, cout, kept_idx=out["kept"],
                               score_off=score_off, uniform_budget=uniform)


def score_select_compact(D, w, out, budget=None, uniform=0, with_kept=True, aggregate=0):
    """One fused trigger (kv_evict_score_select_compact); returns the scores it wrote."""
    scores = torch.zeros(D["k"].shape[0], dtype=torch.float32, device=D["k"].device)
    cout = kv.make_cache(out["k"], out["v"], out["pos"], out["seg_off"], out["seg_len"], w.n_kv_heads, out["cap"])
    kv.kv_evict_score_select_compact(cache_of(D, w), obs_of(D, w, aggregate), scores, budget, w.n_prefix, w.n_recent,
                                     cout,
                                     kept_idx=out["kept"] if with_kept else None, uniform_budget=uniform)
    return scores
