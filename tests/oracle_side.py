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
