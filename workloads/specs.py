"""Workload descriptions (shapes, knobs, seeds) for the eviction step, read
from workloads/configs/<name>.json.

Sizes follow the five benchmark cases of the eviction-step build:
  tiny-f32      one fp32 layer, 4 query / 2 KV heads, d=64, 512 keys -> 448
  qwen3-4b-1l   one bf16 Qwen3-4B-shaped layer, batch 14, 2048 -> 1792
  qwen3-4b-36l  36 bf16 layers, batch 16, 4096 -> 3584, 4 triggers, +512 tokens between
  r1-llama-8b   32 bf16 layers, batch 10, ragged lengths U[6144, 8192], per-head budgets
  long-65k      one bf16 layer, batch 4, 65,536 -> 8192, plus hidden-state traces
Value structure (clustered pre-RoPE keys and queries, a few "global" queries
that revisit early clusters) follows the BeaconKV page's observations
(section on thought-revisiting tokens: global queries cluster, Fig. 4).
"""
import json
import os
from dataclasses import dataclass, fields, replace


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # storage dtype of K, V and queries: "bf16" or "f32"
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    len_lo: int                # per-request cache length, drawn uniform in [len_lo, len_hi]
    len_hi: int
    budget: int                # uniform per-head kept count; 0 = entropy-driven per-head budgets
    n_recent_q: int            # recent observation queries (at their own positions)
    n_beacon: int              # beacon queries in the observation set (rotated to step t)
    fps_cap: int               # beacon buffer capacity (B_Q^max); 0 = no FPS in the step
    fps_keep: int              # beacons kept by FPS (B_Q^min)
    n_clusters: int
    early_frac: float          # keys in the first early_frac of positions use the early clusters
    early_clusters: int
    global_frac: float         # fraction of queries aimed at an early cluster
    beacon_mode: str           # "past": near the cluster of a random past key; "c01": near clusters {0,1}
    fps_buf_mode: str          # "beacons": buffer = the beacons; "beacons+recent": beacons then recent
    n_prefix: int = 4          # protected prefix P
    n_recent: int = 16         # protected recent window R
    causal: int = 1
    triggers: int = 1
    append: int = 0
    key_sigma: float = 0.3
    seed_base: int = 0
    # wave budgets (entropy-driven case)
    wave_center: float = 16.0
    wave_sigma: float = 6.0
    wave_total: int = 32 * 1024
    min_per_head: int = 64
    # hidden-state traces (attention-free score)
    trace_layers: tuple = ()
    d_model: int = 0
    epikv_window: int = 256
    epikv_eps: float = 1e-6

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_obs(self):
        return self.n_recent_q + self.n_beacon

    def scaled(self, **kw):
        return replace(self, **kw)


CONFIG_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "configs")


def load_workload(path):
    """A Workload from a JSON file of its fields (every field named; unknown keys are an error)."""
    with open(path) as f:
        d = json.load(f)
    names = {f.name for f in fields(Workload)}
    missing, extra = names - set(d), set(d) - names
    if missing or extra:
        raise ValueError(f"{path}: missing fields {sorted(missing)}, unknown fields {sorted(extra)}")
    d["trace_layers"] = tuple(d["trace_layers"])
    return Workload(**d)


# the five cases, one JSON file each (shapes, seeds and knobs)
WORKLOADS = {w.name: w for w in (load_workload(os.path.join(CONFIG_DIR, f)) for f in sorted(os.listdir(CONFIG_DIR))
                                 if f.endswith(".json"))}


def get_workload(name):
    return WORKLOADS[name]
