"""Writes the oracle's worked example (oracle_worked_example.json) from fixed
inputs built here from integer patterns.  The pages print no worked example
of the step, so these stored values are regression fixtures of the oracle
itself: tests/test_oracle_golden.py recomputes them, and any change of the
oracle's arithmetic shows up there.  Calls nothing but the oracle.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def inputs():
    """One KV head (d = 8) of 12 cached keys at positions 0..11, two query
    heads of the group with one recent row (tau = 11) and one beacon (t = 12)
    each, a six-row pre-RoPE query buffer; every value a small multiple of
    1/4, exact in bf16 and fp32."""
    d, n = 8, 12
    k_pre = np.array([[((7 * j + 3 * i) % 11 - 5) / 4.0 for i in range(d)] for j in range(n)])
    q_pre = np.array([[((5 * r + i * (r + 1)) % 7 - 3) / 2.0 for i in range(d)] for r in range(4)])
    buf = np.array([[((3 * r + 2 * i) % 5 - 2) / 4.0 + (1.0 if i == r % d else 0.0) for i in range(d)]
                    for r in range(6)])
    return {"d": d, "n": n, "theta": 10000.0, "k_pre": k_pre, "key_pos": np.arange(n),
            "q_pre": q_pre, "q_pos": np.array([11, 12, 11, 12]), "budget": 8, "n_prefix": 2, "n_recent": 2,
            "fps_buf": buf, "fps_keep": 3}


def compute(x):
    k = oracle.to_storage(oracle.rope(x["k_pre"], x["key_pos"], x["theta"]), "f32")
    q = oracle.to_storage(oracle.rope(x["q_pre"], x["q_pos"], x["theta"]), "f32")
    scores = oracle.segment_scores(k, x["key_pos"], q, x["q_pos"])
    kept = oracle.select_kept(scores, x["n"], x["budget"], x["n_prefix"], x["n_recent"])
    return {
        "k_cache": k, "q_rot": q, "scores": scores, "kept": kept,
        "compacted_pos": oracle.compact_rows(x["key_pos"], kept),
        "entropy": oracle.normalized_entropy(scores),
        "head_budgets": oracle.head_budgets(np.array([0.9, 0.5, 0.7, 0.1]), np.array([500, 100, 800, 300]),
                                            1000, 64),
        "layer_wave_budgets": oracle.layer_wave_budgets(32, 16.0, 6.0, 32 * 1024, 64),
        "fps_picks": oracle.fps(x["fps_buf"], x["fps_keep"]),
    }


def _plain(v):
    if isinstance(v, np.ndarray):
        return v.tolist()
    if isinstance(v, np.generic):
        return v.item()
    return v


CITES = {
    "k_cache": "BeaconKV, RoPE alignment at scoring: keys stored rotated to their own positions (half-split pairs)",
    "q_rot": "BeaconKV, RoPE alignment at scoring: recent rows at their own positions, beacons at step t",
    "scores": "BeaconKV, observation query set and RoPE alignment: row softmax of q.k/sqrt(d), max over rows",
    "kept": "BeaconKV, RoPE alignment at scoring: prefix and recent span kept, top scores fill the budget",
    "compacted_pos": "BeaconKV, experiments: eviction is permanent, survivors gathered in slot order",
    "entropy": "ReasonAlloc, Key Concepts: normalised attention entropy of a head",
    "head_budgets": "ReasonAlloc, Core Mechanism: head budgets from entropy weights, floor 64, capped at the length",
    "layer_wave_budgets": "ReasonAlloc, Core Mechanism: mid-peaked wave over 32 layers (centre 16, sigma 6), "
                          "32 x 1024 in all, floor 64",
    "fps_picks": "BeaconKV, Continual FPS: cosine farthest-point sampling from the oldest row",
}


def main():
    x = inputs()
    out = compute(x)
    doc = {"about": "oracle worked example; written by tests/golden/make_golden.py from oracle/ only",
           "inputs": {k: _plain(v) for k, v in x.items()},
           "outputs": {k: {"value": _plain(v), "cite": CITES[k]} for k, v in out.items()}}
    with open(os.path.join(HERE, "oracle_worked_example.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
