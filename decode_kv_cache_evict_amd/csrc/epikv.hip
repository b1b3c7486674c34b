// Attention-free eviction score (EPIKV page, 方法论 part 1 顿悟得分 and part 3
// 时间趋势校正):
//   g_l(t) = ||h_l(t) - h_l(t-1)||_2 for the two monitored layers,
//   z_l(t) = (g_l(t) - mean) / (std + eps) over a causal window,
//   score(t) = z_a(t) - z_b(t)  (part 3), or, in the rolling-mean form of
//   part 2 (双带层解剖结构), score(t) = mean_a(t) - mean_b(t) over the same window.
// g is a bandwidth-bound stream over the bf16 traces: a wavefront (d_model 512
// or 1024) or a work-group (d_model 2048 and up) walks a run of consecutive
// steps of one (layer, request), keeping the previous row in registers so
// every row is read once.  z works on LDS tiles of g in double, from prefix
// sums.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace kve {

namespace {

constexpr int kRun = 64;          // steps per wavefront in the per-wave g pass
constexpr int kZTile = 256;       // steps per work-group in the z pass

// VPL = 16-byte vectors per lane per row (d_model = 512 * VPL).
template <int VPL>
__global__ __launch_bounds__(256) void epikv_g_kernel(const uint16_t* __restrict__ ha, const uint16_t* __restrict__ hb,
                                                      int batch, int T, float* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int runs = (T + kRun - 1) / kRun;
  const int64_t total = int64_t(2) * batch * runs;
  if (wave >= total) return;
  const int run = int(wave % runs);
  const int lb = int(wave / runs);            // layer * batch + b
  const int layer = lb / batch, b = lb % batch;
  const uint16_t* h = (layer == 0 ? ha : hb) + int64_t(b) * T * (512 * VPL);
  const int t0 = run * kRun, t1 = min(T, t0 + kRun);
  const uint4* base = reinterpret_cast<const uint4*>(h);
  const int64_t row_vec = 64 * VPL;          // uint4 per row

  auto load_row = [&](int t, uint4* dst) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) dst[v] = base[int64_t(t) * row_vec + v * 64 + lane];
  };
  uint4 prev[VPL], cur[VPL];
  if (t0 > 0) load_row(t0 - 1, prev);
  float* gout = g + int64_t(lb) * T;
  for (int t = t0; t < t1; ++t) {
    load_row(t, cur);
    float acc = 0.f;
    if (t > 0) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint16_t* a = reinterpret_cast<const uint16_t*>(&cur[v]);
        const uint16_t* p = reinterpret_cast<const uint16_t*>(&prev[v]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = bf16_to_f32(a[e]) - bf16_to_f32(p[e]);
          acc = fmaf(d, d, acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) gout[t] = t > 0 ? sqrtf(acc) : 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) prev[v] = cur[v];
  }
}

// g for d_model >= 2048: one work-group per run of `run` steps of one
// (layer, request).  Thread j holds the 16-byte chunks j + 256 c (c < CPT) of
// each row.  Rows go in batches of RB = 8 / CPT; the next batch's loads are
// issued before the current batch's differences, so 32 KB per work-group
// stay in flight across the reductions and the barrier.  The previous row
// stays in registers, so every row is read once plus one row per run.  Each
// row's sum of squared differences is reduced over the lanes, then over the
// four waves through LDS (two alternating slots: one barrier per batch).
template <int CPT>
__global__ __launch_bounds__(256) void epikv_g_rows_kernel(const uint16_t* __restrict__ ha,
                                                           const uint16_t* __restrict__ hb, int batch, int T, int run,
                                                           float* __restrict__ g) {
  constexpr int RB = 8 / CPT;
  __shared__ float part[2][4][RB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int runs = (T + run - 1) / run;
  const int lb = int(blockIdx.x) / runs, r = int(blockIdx.x) % runs;   // lb = layer * batch + b
  const int layer = lb / batch, b = lb % batch;
  constexpr int64_t row_vec = 256 * CPT;      // uint4 per row
  const uint4* base = reinterpret_cast<const uint4*>(layer == 0 ? ha : hb) + int64_t(b) * T * row_vec + tid;
  const int t0 = r * run, t1 = min(T, t0 + run);
  float* gout = g + int64_t(lb) * T;
  auto load = [&](int tb, uint4 (&dst)[RB][CPT]) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int t = min(tb + i, t1 - 1);      // past the run's end: the last row again (not written)
#pragma unroll
      for (int c = 0; c < CPT; ++c) dst[i][c] = base[int64_t(t) * row_vec + c * 256];
    }
  };
  uint4 prev[CPT], cur[RB][CPT], nxt[RB][CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) prev[c] = t0 > 0 ? base[int64_t(t0 - 1) * row_vec + c * 256] : make_uint4(0, 0, 0, 0);
  load(t0, cur);
  int slot = 0;
  for (int tb = t0; tb < t1; tb += RB) {
    if (tb + RB < t1) load(tb + RB, nxt);
    float s[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const uint4 pv = i == 0 ? prev[c] : cur[i - 1][c];
        const uint16_t* x = reinterpret_cast<const uint16_t*>(&cur[i][c]);
        const uint16_t* y = reinterpret_cast<const uint16_t*>(&pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = bf16_to_f32(x[e]) - bf16_to_f32(y[e]);
          acc = fmaf(d, d, acc);
        }
      }
      s[i] = wave_sum(acc);
    }
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < RB; ++i) part[slot][w][i] = s[i];
    __syncthreads();
    if (tid < RB && tb + tid < t1) {
      const int t = tb + tid;
      const float v = part[slot][0][tid] + part[slot][1][tid] + part[slot][2][tid] + part[slot][3][tid];
      gout[t] = t > 0 ? sqrtf(v) : 0.f;
    }
    slot ^= 1;
#pragma unroll
    for (int c = 0; c < CPT; ++c) prev[c] = cur[RB - 1][c];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int c = 0; c < CPT; ++c) cur[i][c] = nxt[i][c];
  }
}

// z for both layers and their difference over one tile of steps of one
// request, from prefix sums: each layer's window sums of d and d^2, where d is
// g less the mean c of the tile's span (which keeps the sums near the size of
// the window's spread, so that E[d^2] - E[d]^2 loses little to cancellation),
// are differences of two inclusive prefix sums held in LDS in double.
__global__ __launch_bounds__(kZTile) void epikv_z_kernel(const float* __restrict__ g, int batch, int T, int W,
                                                         float eps, int form, float* __restrict__ out) {
  extern __shared__ double zs[];               // [2][kZTile + W - 1]: prefix sums of d and of d^2
  __shared__ double wtot[2][kZTile / 64];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = blockIdx.x * kZTile;
  const int span = kZTile + W - 1;
  const int first = t0 - (W - 1);              // span entry k is step first + k
  const int per = (span + kZTile - 1) / kZTile; // consecutive span entries per thread
  const int j0 = tid * per, j1 = min(span, j0 + per);
  const int t = t0 + tid;
  double z[2] = {0.0, 0.0};
  for (int l = 0; l < 2; ++l) {
    const float* gl = g + (int64_t(l) * batch + b) * T;
    auto val = [&](int k) {                    // steps before 1 or past T enter no window
      const int tt = first + k;
      return tt >= 1 && tt < T ? double(gl[tt]) : 0.0;
    };
    double loc = 0.0;
    for (int k = j0; k < j1; ++k) loc += val(k);
    loc = wave_sum_f64(loc);
    if (lane == 0) wtot[0][w] = loc;
    __syncthreads();
    const int n_valid = max(1, min(first + span, T) - max(first, 1));
    const double c = (wtot[0][0] + wtot[0][1] + wtot[0][2] + wtot[0][3]) / double(n_valid);
    __syncthreads();
    double s1 = 0.0, s2 = 0.0;
    for (int k = j0; k < j1; ++k) {
      const double d = val(k) - c;
      s1 += d;
      s2 += d * d;
      zs[k] = s1;
      zs[span + k] = s2;
    }
    const double i1 = wave_inclusive_sum(s1), i2 = wave_inclusive_sum(s2);
    if (lane == 63) {
      wtot[0][w] = i1;
      wtot[1][w] = i2;
    }
    __syncthreads();
    double o1 = i1 - s1, o2 = i2 - s2;         // the entries before this thread's
    for (int q = 0; q < w; ++q) {
      o1 += wtot[0][q];
      o2 += wtot[1][q];
    }
    for (int k = j0; k < j1; ++k) {
      zs[k] += o1;
      zs[span + k] += o2;
    }
    __syncthreads();
    if (t >= 1 && t < T) {
      const int lo = max(1, t - W + 1), cnt = t - lo + 1;
      const int kh = t - first, kl = lo - first;
      const double S1 = zs[kh] - (kl > 0 ? zs[kl - 1] : 0.0);
      const double S2 = zs[span + kh] - (kl > 0 ? zs[span + kl - 1] : 0.0);
      const double md = S1 / cnt;              // window mean of d
      if (form == 1) {                         // rolling-mean form: g_bar(t)
        z[l] = c + md;
      } else {
        const double sd = sqrt(fmax(S2 / cnt - md * md, 0.0));
        z[l] = (double(gl[t]) - c - md) / (sd + double(eps));
      }
    }
    __syncthreads();                           // zs and wtot are rewritten for the other layer
  }
  if (t < T) out[int64_t(b) * T + t] = t == 0 ? 0.f : float(z[0] - z[1]);
}

}  // namespace

size_t epikv_ws_bytes(int32_t batch, int32_t T) { return size_t(2) * batch * T * sizeof(float); }

hipError_t launch_epikv(const void* h_a, const void* h_b, int32_t batch, int32_t T, int32_t d_model, int32_t window,
                        float eps, int32_t form, float* g_out, float* scores, void* ws, hipStream_t st) {
  if (batch == 0 || T == 0) return hipSuccess;
  float* g = g_out ? g_out : static_cast<float*>(ws);
  const uint16_t* a = static_cast<const uint16_t*>(h_a);
  const uint16_t* b = static_cast<const uint16_t*>(h_b);
  if (d_model >= 2048) {
    // runs sized so that the launch is about one round of resident
    // work-groups (five per CU at this kernel's register use), in whole batches
    constexpr int64_t kResident = 5 * 256;
    const int64_t pairs = int64_t(2) * batch;
    const int64_t per_pair = std::max<int64_t>(1, kResident / pairs);
    const int rb = 8 / (d_model / 2048);
    const int run = int(std::max<int64_t>(rb, (T + per_pair - 1) / per_pair + rb - 1) / rb * rb);
    const dim3 grid(unsigned(pairs * ((T + run - 1) / run)));
    switch (d_model / 2048) {
      case 1: hipLaunchKernelGGL(epikv_g_rows_kernel<1>, grid, dim3(256), 0, st, a, b, batch, T, run, g); break;
      case 2: hipLaunchKernelGGL(epikv_g_rows_kernel<2>, grid, dim3(256), 0, st, a, b, batch, T, run, g); break;
      case 4: hipLaunchKernelGGL(epikv_g_rows_kernel<4>, grid, dim3(256), 0, st, a, b, batch, T, run, g); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const int runs = (T + kRun - 1) / kRun;
    const int64_t waves = int64_t(2) * batch * runs;
    const dim3 grid(unsigned((waves + 3) / 4));
    switch (d_model / 512) {
      case 1: hipLaunchKernelGGL(epikv_g_kernel<1>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
      case 2: hipLaunchKernelGGL(epikv_g_kernel<2>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t sh = size_t(2) * (kZTile + window - 1) * sizeof(double);
  hipLaunchKernelGGL(epikv_z_kernel, dim3(unsigned((T + kZTile - 1) / kZTile), unsigned(batch)), dim3(kZTile), sh, st,
                     g, batch, T, window, eps, form, scores);
  return hipGetLastError();
}

}  // namespace kve
