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
    s64 = np.asarray(orc_scores[:n], dtype=np.float64)
    cand = np.arange(n_prefix, n - n_recent)
    chosen = np.setdiff1d(want, np.concatenate([np.arange(n_prefix), np.arange(n - n_recent, n)]))
    cut = s64[chosen].min()
    diff = np.setxor1d(gpu_kept, want)
    if not np.all(np.isin(diff, cand)):
        return False, len(diff), "a protected slot differs"
    band = np.abs(s64[diff] - cut) <= max(rtol * abs(cut), floor)
    if not band.all():
        j = diff[~band][0]
        return False, len(diff), f"slot {j} (oracle score {s64[j]!r}) differs outside the band around {cut!r}"
    return True, len(diff) // 2, ""


FRAC_TOL = 1e-3


def _near_cut(x, total, tol):
    """Heads whose largest-remainder rounding of the real shares x can flip:
    those whose fractional part lies within tol of the cut, when the last
    fraction rounded up and the first rounded down are within tol of each
    other (otherwise no head: the rounding is decided)."""
    x = np.asarray(x, dtype=np.float64)
    f = np.floor(x)
    frac = x - f
    r = int(round(total - f.sum()))
    order = sorted(range(len(x)), key=lambda g: (-frac[g], g))
    a = frac[order[r - 1]] if r > 0 else np.inf          # last rounded up
    b = frac[order[r]] if r < len(x) else -np.inf        # first rounded down
    if a - b > tol:
        return np.zeros(len(x), dtype=bool)
    return (frac >= b - tol) & (frac <= a + tol)


def budgets_match(got, e_gpu, e_orc, seg_len, layer_total, floor, inverse=False, tol=FRAC_TOL):
    """Check one request-layer's GPU head budgets (ReasonAlloc, Core Mechanism).

    Invariants: the sum is min(total, sum of lengths), every head between
    min(floor, n) and n.  Against the oracle's budget rule applied to the
    GPU's own entropies: equal, except by one token at heads whose real
    share's fractional part lies within tol of the largest-remainder cut.
    Against the oracle's entropies end to end: the same, with the band widened
    by the largest shift of any real share between the two entropy vectors.
    Returns (ok, message)."""
    got = np.asarray(got, dtype=np.int64)
    n = np.asarray(seg_len, dtype=np.int64)
    tot = min(int(layer_total), int(n.sum()))
    if got.sum() != tot:
        return False, f"sum {got.sum()} != {tot}"
    if np.any(got < np.minimum(floor, n)) or np.any(got > n):
        return False, f"a budget outside [min(floor, n), n]: {got.tolist()} for lengths {n.tolist()}"
    x_g = oracle.waterfill(float(layer_total), oracle.head_weights(e_gpu, inverse), float(floor), n.astype(float))
    x_o = oracle.waterfill(float(layer_total), oracle.head_weights(e_orc, inverse), float(floor), n.astype(float))
    shift = float(np.abs(x_g - x_o).max())
    for x, band, what in ((x_g, tol, "the GPU's entropies"), (x_o, tol + 2 * shift, "the oracle's entropies")):
        want = oracle.largest_remainder(x, tot)
        diff = got != want
        if not diff.any():
            continue
        ok = _near_cut(x, tot, band)
        if np.any(np.abs(got - want) > 1) or np.any(diff & ~ok):
            return False, (f"budgets {got.tolist()} != {want.tolist()} from {what} (real shares {x.tolist()}) "
                           f"outside the remainder band {band:g}")
    return True, ""
