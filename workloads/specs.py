"""Workload descriptions (shapes, knobs, seeds) for the eviction step.

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
from dataclasses import dataclass, replace


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


WORKLOADS = {
    "tiny-f32": Workload(
        name="tiny-f32", dtype="f32", n_layers=1, batch=1, n_q_heads=4, n_kv_heads=2,
        head_dim=64, rope_theta=1e4, len_lo=512, len_hi=512, budget=448,
        n_recent_q=8, n_beacon=8, fps_cap=16, fps_keep=8, n_clusters=8,
        early_frac=0.0, early_clusters=0, global_frac=0.0, beacon_mode="c01",
        fps_buf_mode="beacons+recent", seed_base=1000),
    "qwen3-4b-1l": Workload(
        name="qwen3-4b-1l", dtype="bf16", n_layers=1, batch=14, n_q_heads=32, n_kv_heads=8,
        head_dim=128, rope_theta=1e6, len_lo=2048, len_hi=2048, budget=1792,
        n_recent_q=16, n_beacon=32, fps_cap=32, fps_keep=16, n_clusters=16,
        early_frac=0.1, early_clusters=4, global_frac=0.05, beacon_mode="past",
        fps_buf_mode="beacons", seed_base=2000),
    "qwen3-4b-36l": Workload(
        name="qwen3-4b-36l", dtype="bf16", n_layers=36, batch=16, n_q_heads=32, n_kv_heads=8,
        head_dim=128, rope_theta=1e6, len_lo=4096, len_hi=4096, budget=3584,
        n_recent_q=16, n_beacon=32, fps_cap=32, fps_keep=16, n_clusters=16,
        early_frac=0.1, early_clusters=4, global_frac=0.05, beacon_mode="past",
        fps_buf_mode="beacons", triggers=4, append=512, seed_base=3000),
    "r1-llama-8b": Workload(
        name="r1-llama-8b", dtype="bf16", n_layers=32, batch=10, n_q_heads=32, n_kv_heads=8,
        head_dim=128, rope_theta=5e5, len_lo=6144, len_hi=8192, budget=0,
        n_recent_q=16, n_beacon=32, fps_cap=0, fps_keep=0, n_clusters=16,
        early_frac=0.1, early_clusters=4, global_frac=0.05, beacon_mode="past",
        fps_buf_mode="beacons", seed_base=4000),
    "long-65k": Workload(
        name="long-65k", dtype="bf16", n_layers=1, batch=4, n_q_heads=32, n_kv_heads=8,
        head_dim=128, rope_theta=5e5, len_lo=65536, len_hi=65536, budget=8192,
        n_recent_q=16, n_beacon=32, fps_cap=0, fps_keep=0, n_clusters=16,
        early_frac=0.1, early_clusters=4, global_frac=0.05, beacon_mode="past",
        fps_buf_mode="beacons", trace_layers=(10, 21), d_model=4096, seed_base=5000),
}


def get_workload(name):
    return WORKLOADS[name]
