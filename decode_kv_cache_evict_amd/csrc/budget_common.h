// Per-request head budgets of ReasonAlloc ("Core Mechanism"): one wave per
// request, lane g = head g.  Shared by the stand-alone budget kernel and the
// one-kernel trigger with entropy budgets, so both give the same budgets for
// the same entropies.
#pragma once

#include "common.h"

namespace kve {

constexpr int kMaxHeads = 64;

__device__ __forceinline__ double wave_min_f64(double v) {
  return wave_reduce(v, [](double x, double y) { return fmin(x, y); });
}
__device__ __forceinline__ double wave_max_f64(double v) {
  return wave_reduce(v, [](double x, double y) { return fmax(x, y); });
}

// LDS of one wave's solve.
struct HeadBudgetLds {
  double w[kMaxHeads], lo[kMaxHeads], hi[kMaxHeads], fr[kMaxHeads];
  int part[kMaxHeads];
};

// The wave's lanes see each other's LDS writes once they are complete (one
// wave: no work-group barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Every lane of one wave calls this; lane g < H is head g with weight source
// e (the head's normalised entropy; weight e, or 1 - e when form == 1), cap
// cap_g (its cached length) and the request's total tot, floor lo_all.  Real
// shares x_g = clamp(lam * w_g, lo_g, hi_g) with sum x = total, found exactly
// on the breakpoints of the piecewise-linear sum (every sum over heads taken in
// head order by a plain loop, as the serial solver does), then rounded by the
// largest-remainder rule (ties to the lower head).  Returns lane g's budget
// (every lane: -1 when the floors alone exceed the total); lanes >= H return 0.
__device__ __forceinline__ int32_t head_budget_wave(double e, int form, int cap_g, double tot, int lo_all, int H,
                                                    HeadBudgetLds& L) {
  const int g = int(threadIdx.x) & (kWave - 1);
  const bool act = g < H;
  double w = 0.0, hi = 0.0;
  if (act) {
    w = form == 1 ? 1.0 - e : e;              // inverse entropy: focused heads gain budget
    hi = double(cap_g > 0 ? cap_g : 0);
    w = w > 0.0 ? w : 0.0;
  }
  const double lo = act ? fmin(double(lo_all), hi) : 0.0;
  // sums of integers: exact in any order
  const double sum_hi = wave_sum_f64(hi), sum_lo = wave_sum_f64(lo);
  const double total = fmin(tot, sum_hi);
  if (total >= sum_hi) return act ? int32_t(hi) : 0;
  if (total < sum_lo - 1e-9) return act ? -1 : 0;
  if (!__any(act && w > 0.0) && act) w = 1.0;
  const bool pos = act && w > 0.0;
  const double cap_pos = wave_sum_f64(pos ? hi : 0.0), lo_zero = wave_sum_f64(act && !pos ? lo : 0.0);
  const bool any_zero = __any(act && !pos);
  // weightless heads cannot grow with lam: when the weighted heads' caps and the
  // weightless floors cannot absorb the total, the weighted heads sit at their
  // caps and the weightless ones split the rest equally
  const bool zero_split = any_zero && total > cap_pos + lo_zero;
  const bool part = zero_split ? act && !pos : act;
  const double pw = zero_split ? 1.0 : w;
  const double ptot = zero_split ? total - cap_pos : total;
  if (act) {
    L.w[g] = pw;
    L.lo[g] = lo;
    L.hi[g] = hi;
    L.part[g] = part;
  }
  wave_lds_sync();
  auto f = [&](double lam) {                  // sum of the clamped shares, in head order
    double v = 0.0;
    for (int q = 0; q < H; ++q)
      if (L.part[q]) v += fmin(fmax(lam * L.w[q], L.lo[q]), L.hi[q]);
    return v;
  };
  // breakpoints: 0 and, per participating head with weight, lo/w and hi/w
  const bool owns = part && pw > 0.0;
  const double p1 = owns ? lo / pw : 0.0, p2 = owns ? hi / pw : 0.0;
  const double f1 = owns ? f(p1) : 0.0, f2 = owns ? f(p2) : 0.0;
  const double f0 = f(0.0);
  double lam;
  const double kBigD = 1.0e300;
  if (ptot <= f0) {
    lam = 0.0;
  } else {
    double cand = kBigD;                        // smallest breakpoint whose sum reaches the total
    if (owns && f1 >= ptot) cand = fmin(cand, p1);
    if (owns && f2 >= ptot) cand = fmin(cand, p2);
    const double bb = wave_min_f64(cand);
    if (bb == kBigD) {
      lam = wave_max_f64(owns ? fmax(p1, p2) : 0.0);   // the largest breakpoint
    } else {
      double below = 0.0;                       // largest breakpoint below it (0 is one)
      if (owns && p1 < bb) below = fmax(below, p1);
      if (owns && p2 < bb) below = fmax(below, p2);
      const double aa = wave_max_f64(below);
      const double fa = f(aa);
      const double mid = 0.5 * (aa + bb);
      double wf = 0.0;
      for (int q = 0; q < H; ++q) {
        const double v = mid * L.w[q];
        if (L.part[q] && L.w[q] > 0.0 && v > L.lo[q] && v < L.hi[q]) wf += L.w[q];
      }
      lam = wf == 0.0 ? bb : aa + (ptot - fa) / wf;
    }
  }
  const double x = !act ? 0.0 : part ? fmin(fmax(lam * pw, lo), hi) : hi;
  // largest remainder: +1 to the r heads with the largest fractional parts (ties to the lower head)
  const double fl = floor(x);
  const double fr = x - fl;
  const long long r = (long long)(total + 0.5) - (long long)wave_sum_f64(fl);
  if (act) L.fr[g] = fr;
  wave_lds_sync();
  long long rank = 0;
  for (int q = 0; q < H; ++q) rank += (L.fr[q] > fr || (L.fr[q] == fr && q < g)) ? 1 : 0;
  return act ? int32_t(fl) + (rank < r ? 1 : 0) : 0;
}

}  // namespace kve
