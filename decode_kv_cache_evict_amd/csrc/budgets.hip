// Budget allocation (ReasonAlloc, "Core Mechanism" and "Key Concepts"):
//   * head budgets: each request's layer total is split over its heads in
//     proportion to a utility weight (the head's normalised score entropy E, or
//     1 - E when focused heads are to gain budget), with a per-head floor and a
//     cap at the head's cached length;
//   * layer budgets: a mid-peaked Gaussian over the layer index, floored.
// Real shares x_g = clamp(lam * w_g, lo_g, hi_g) with sum x = total are found
// exactly on the breakpoints of the piecewise-linear sum, then rounded by the
// largest-remainder rule (ties to the lower index).  Double precision; the
// layer table is one thread's work, the per-request head budgets one wave's.
#include "budget_common.h"
#include "common.h"
#include "internal.h"

namespace kve {

namespace {

__device__ double clamp_sum(const double* w, const double* lo, const double* hi, int H, double lam) {
  double f = 0.0;
  for (int g = 0; g < H; ++g) f += fmin(fmax(lam * w[g], lo[g]), hi[g]);
  return f;
}

// Real shares for heads with positive weight (others are at their floor), or
// every head when all weights vanish (equal split).
__device__ void solve_shares(const double* w, const double* lo, const double* hi, int H, double total,
                             double* x) {
  double bps[2 * kMaxHeads + 1];
  int nb = 0;
  bps[nb++] = 0.0;
  for (int g = 0; g < H; ++g)
    if (w[g] > 0.0) {
      bps[nb++] = lo[g] / w[g];
      bps[nb++] = hi[g] / w[g];
    }
  for (int i = 1; i < nb; ++i) {            // insertion sort
    const double v = bps[i];
    int j = i - 1;
    while (j >= 0 && bps[j] > v) {
      bps[j + 1] = bps[j];
      --j;
    }
    bps[j + 1] = v;
  }
  double lam = bps[nb - 1];
  double fa = clamp_sum(w, lo, hi, H, bps[0]);
  if (total <= fa) {
    lam = bps[0];
  } else {
    for (int i = 1; i < nb; ++i) {
      const double fb = clamp_sum(w, lo, hi, H, bps[i]);
      if (fb >= total) {
        const double a = bps[i - 1], b = bps[i], mid = 0.5 * (a + b);
        double wf = 0.0;
        for (int g = 0; g < H; ++g) {
          const double v = mid * w[g];
          if (w[g] > 0.0 && v > lo[g] && v < hi[g]) wf += w[g];
        }
        lam = wf == 0.0 ? b : a + (total - fa) / wf;
        break;
      }
      fa = fb;
    }
  }
  for (int g = 0; g < H; ++g) x[g] = fmin(fmax(lam * w[g], lo[g]), hi[g]);
}

// Largest-remainder rounding of x (sum = total) into out.
__device__ void round_shares(const double* x, int H, long long total, int32_t* out) {
  long long fl[kMaxHeads];
  double fr[kMaxHeads];
  long long s = 0;
  for (int g = 0; g < H; ++g) {
    const double f = floor(x[g]);
    fl[g] = (long long)f;
    fr[g] = x[g] - f;
    s += fl[g];
  }
  long long r = total - s;
  bool used[kMaxHeads];
  for (int g = 0; g < H; ++g) used[g] = false;
  for (; r > 0; --r) {
    int best = -1;
    for (int g = 0; g < H; ++g)
      if (!used[g] && (best < 0 || fr[g] > fr[best])) best = g;
    if (best < 0) break;
    used[best] = true;
    fl[best] += 1;
  }
  for (int g = 0; g < H; ++g) out[g] = int32_t(fl[g]);
}

// Proportional split of `total` with floors and caps; writes -1 everywhere
// when the floors alone exceed the total.
__device__ void allocate(const double* w_in, double lo_all, const double* hi, int H, double total, int32_t* out) {
  double w[kMaxHeads], lo[kMaxHeads], x[kMaxHeads];
  double sum_hi = 0.0, sum_lo = 0.0;
  bool any = false;
  for (int g = 0; g < H; ++g) {
    lo[g] = fmin(lo_all, hi[g]);
    sum_hi += hi[g];
    sum_lo += lo[g];
    w[g] = w_in[g] > 0.0 ? w_in[g] : 0.0;
    any = any || w[g] > 0.0;
  }
  if (total >= sum_hi) {
    for (int g = 0; g < H; ++g) out[g] = int32_t(hi[g]);
    return;
  }
  if (total < sum_lo - 1e-9) {
    for (int g = 0; g < H; ++g) out[g] = -1;
    return;
  }
  if (!any)
    for (int g = 0; g < H; ++g) w[g] = 1.0;
  // Weightless heads cannot grow with lam; when the weighted heads' caps and
  // the weightless floors cannot absorb the total, the weighted heads sit at
  // their caps and the weightless ones split the rest equally.
  double cap_pos = 0.0, lo_zero = 0.0;
  int n_zero = 0;
  for (int g = 0; g < H; ++g) {
    if (w[g] > 0.0) cap_pos += hi[g];
    else {
      lo_zero += lo[g];
      ++n_zero;
    }
  }
  if (n_zero > 0 && total > cap_pos + lo_zero) {
    double wz[kMaxHeads], loz[kMaxHeads], hiz[kMaxHeads], xz[kMaxHeads];
    int m = 0;
    for (int g = 0; g < H; ++g)
      if (!(w[g] > 0.0)) {
        wz[m] = 1.0;
        loz[m] = lo[g];
        hiz[m] = hi[g];
        ++m;
      }
    solve_shares(wz, loz, hiz, m, total - cap_pos, xz);
    m = 0;
    for (int g = 0; g < H; ++g) x[g] = w[g] > 0.0 ? hi[g] : xz[m++];
  } else {
    solve_shares(w, lo, hi, H, total, x);
  }
  round_shares(x, H, (long long)(total + 0.5), out);
}

__global__ __launch_bounds__(64) void head_budget_kernel(const float* __restrict__ wts, const int32_t* __restrict__ tot,
                                                         const int32_t* __restrict__ cap, int batch, int H, int lo_all,
                                                         int form, int32_t* __restrict__ out) {
  __shared__ HeadBudgetLds L;
  const int b = blockIdx.x, g = threadIdx.x;
  if (b >= batch) return;
  const bool act = g < H;
  const int32_t v = head_budget_wave(act ? double(wts[b * H + g]) : 0.0, form, act ? cap[b * H + g] : 0,
                                     double(tot[b]), lo_all, H, L);
  if (act) out[b * H + g] = v;
}

__global__ void wave_budget_kernel(int L, double center, double sigma, int total, int lo, int32_t* out) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  double w[kMaxHeads], hi[kMaxHeads];
  for (int l = 0; l < L; ++l) {
    const double d = double(l) - center;
    w[l] = exp(-(d * d) / (2.0 * sigma * sigma));
    hi[l] = double(total);
  }
  allocate(w, double(lo), hi, L, double(total), out);
}

}  // namespace

hipError_t launch_budgets(const float* w, const int32_t* total, const int32_t* cap, int32_t batch,
                          int32_t n_heads, int32_t min_per_head, int32_t* out, hipStream_t st, int weight_form) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(head_budget_kernel, dim3(unsigned(batch)), dim3(64), 0, st, w, total, cap, batch, n_heads,
                     min_per_head, weight_form, out);
  return hipGetLastError();
}

hipError_t launch_wave_budgets(int32_t n_layers, double center, double sigma, int32_t total, int32_t lo,
                               int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(wave_budget_kernel, dim3(1), dim3(64), 0, st, n_layers, center, sigma, total, lo, out);
  return hipGetLastError();
}

}  // namespace kve
