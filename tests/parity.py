"""Comparison rules between the GPU library and the CPU oracle.

  * scores: |gpu - orc| <= max(rtol * |orc|, floor) with rtol = 2e-3 (bf16
    operands, fp32 accumulation) and floor = 1e-30 (values that far below 1
    may flush to zero in fp32 exponentials);
  * kept sets: identical, except that candidates whose oracle score lies within
    the same tolerance of the oracle's cut score may be swapped (counts equal);
  * FPS picks: each pick must be within rtol of the farthest remaining row
    (oracle distances, state replayed with the given picks); identical to the
    oracle's picks when no step of the oracle has such a near tie.
"""
import numpy as np

import oracle

RTOL = 2e-3
FLOOR = 1e-30


def tol(x, rtol=RTOL, floor=FLOOR):
    return np.maximum(rtol * np.abs(x), floor)


def assert_scores_close(gpu, orc, rtol=RTOL, floor=FLOOR, what="scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    orc = np.asarray(orc, dtype=np.float64)
    err = np.abs(gpu - orc)
    bad = err > tol(orc, rtol, floor)
    if bad.any():
        i = int(np.argmax(err / tol(orc, rtol, floor)))
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} oracle={orc[i]!r}")
    return float((err / np.maximum(np.abs(orc), floor)).max()) if err.size else 0.0


def kept_matches(gpu_kept, orc_scores, n, budget, n_prefix, n_recent, rtol=RTOL, floor=FLOOR):
    """Return (ok, n_swapped, message) for one segment's kept slots."""
    gpu_kept = np.asarray(gpu_kept, dtype=np.int64)
    want = oracle.select_kept(orc_scores, n, budget, n_prefix, n_recent)
    if len(gpu_kept) != len(want):
        return False, 0, f"count {len(gpu_kept)} != {len(want)}"
    if np.any(np.diff(gpu_kept) <= 0):
        return False, 0, "kept slots not strictly ascending"
    if np.array_equal(gpu_kept, want):
        return True, 0, ""
    s32 = np.asarray(orc_scores[:n], dtype=np.float64).astype(np.float32).astype(np.float64)
    cand = np.arange(n_prefix, n - n_recent)
    chosen = np.setdiff1d(want, np.concatenate([np.arange(n_prefix), np.arange(n - n_recent, n)]))
    cut = s32[chosen].min()
    diff = np.setxor1d(gpu_kept, want)
    if not np.all(np.isin(diff, cand)):
        return False, len(diff), "a protected slot differs"
    band = np.abs(s32[diff] - cut) <= max(rtol * abs(cut), floor)
    if not band.all():
        j = diff[~band][0]
        return False, len(diff), f"slot {j} (oracle score {s32[j]!r}) differs outside the band around {cut!r}"
    return True, len(diff) // 2, ""
