"""Observation-query rotation, bit for bit (BeaconKV, "打分时的 RoPE 对齐":
recent queries are rotated to their own positions and beacons to the current
step, each rounded to the storage dtype before the contraction).

The library keeps the rotated rows at the start of the scoring workspace
(layout [batch, n_q_heads, max_obs, head_dim] of the cache dtype, rows past a
request's n_obs zeroed), where this test reads them after a kv_evict_score
call and compares them with the oracle's float64 rotation rounded to the
storage dtype.  The cases cover both dtypes and head sizes, query-head counts
from 2 to 64 (one to several rotation items per thread), row blocks that end
inside max_obs, requests with no, some or all rows live, and positions up to
70,000 (large angles)."""
import numpy as np
import pytest
import torch

import decode_kv_cache_evict_amd as kv
import oracle

pytestmark = pytest.mark.gpu

# (dtype, head_dim, n_q_heads, n_kv_heads, max_obs, n_obs per request, rope theta)
CASES = {
    "bf16-d128-q32": ("bf16", 128, 32, 8, 48, [48, 17, 0], 1e6),
    "bf16-d64-q8-ragged-blocks": ("bf16", 64, 8, 2, 37, [37, 5], 5e5),
    "bf16-d128-q64": ("bf16", 128, 64, 8, 24, [24, 23], 1e4),
    "f32-d64-q4": ("f32", 64, 4, 2, 16, [13], 1e4),
    "f32-d128-q2": ("f32", 128, 2, 1, 5, [5, 2, 4], 1e6),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.lib()


@pytest.mark.parametrize("name", list(CASES))
def test_rotated_queries_bit_exact(name):
    dt, D, Hq, Hkv, M, n_obs, theta = CASES[name]
    B = len(n_obs)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator().manual_seed(sum(map(ord, name)))
    q = torch.randn(B, Hq, M, D, generator=g).to(tdt)
    q_pos = torch.randint(0, 70_000, (B, M), generator=g, dtype=torch.int32)
    nob = torch.tensor(n_obs, dtype=torch.int32)
    # a small cache: one 64-row segment per (request, KV head)
    n = 64
    S = B * Hkv
    k = torch.randn(S * n, D, generator=g).to(tdt)
    pos = torch.arange(n, dtype=torch.int32).repeat(S)
    seg_off = torch.arange(S, dtype=torch.int64) * n
    seg_len = torch.full((S,), n, dtype=torch.int32)
    dev = "cuda"
    cache = kv.make_cache(k.to(dev), None, pos.to(dev), seg_off.to(dev), seg_len.to(dev), Hkv, n)
    obs = kv.make_obs(q.to(dev), q_pos.to(dev), nob.to(dev), theta, True)
    nbytes = kv.kv_evict_score_workspace(cache, obs)
    ws = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device=dev)
    scores = torch.zeros(S * n, dtype=torch.float32, device=dev)
    kv.kv_evict_score(cache, obs, scores, None, ws=ws)
    torch.cuda.synchronize()
    off = ((ws.data_ptr() + 255) & ~255) - ws.data_ptr()
    esz = 2 if dt == "bf16" else 4
    raw = ws[off:off + B * Hq * M * D * esz].cpu()
    got = raw.view(tdt).view(B, Hq, M, D).to(torch.float64).numpy()
    qn = q.to(torch.float64).numpy()
    pn = q_pos.numpy().astype(np.int64)
    want = oracle.to_storage(oracle.rope(qn, pn[:, None, :], theta), dt)
    live = np.arange(M)[None, :] < nob.numpy()[:, None]                     # [B, M]
    want = np.where(live[:, None, :, None], want, 0.0)
    bad = got != want
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} rotated elements differ; first at "
                           f"{tuple(int(x[0]) for x in np.nonzero(bad))}")
