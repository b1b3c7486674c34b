// Attention-free eviction score (EPIKV page, 方法论 part 1 顿悟得分 and part 3
// 时间趋势校正):
//   g_l(t) = ||h_l(t) - h_l(t-1)||_2 for the two monitored layers,
//   z_l(t) = (g_l(t) - mean) / (std + eps) over a causal window,
//   score(t) = z_a(t) - z_b(t)  (part 3), or, in the rolling-mean form of
//   part 2 (双带层解剖结构), score(t) = mean_a(t) - mean_b(t) over the same window.
// g is a bandwidth-bound stream over the bf16 traces: one wavefront walks a run
// of consecutive steps of one (layer, request), keeping the previous row in
// registers so every row is read once.  z works on LDS tiles of g in double.
#include "common.h"
#include "internal.h"

namespace kve {

namespace {

constexpr int kRun = 64;          // steps per wavefront in the g pass
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

// z for both layers and their difference over one tile of steps of one request.
__global__ __launch_bounds__(kZTile) void epikv_z_kernel(const float* __restrict__ g, int batch, int T, int W,
                                                         float eps, int form, float* __restrict__ out) {
  extern __shared__ double zs[];               // [2][kZTile + W - 1]
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kZTile;
  const int span = kZTile + W - 1;
  const int first = t0 - (W - 1);
  for (int i = threadIdx.x; i < 2 * span; i += kZTile) {
    const int l = i / span, k = i % span;
    const int t = first + k;
    zs[i] = (t >= 1 && t < T) ? double(g[(int64_t(l) * batch + b) * T + t]) : 0.0;
  }
  __syncthreads();
  const int t = t0 + threadIdx.x;
  if (t >= T) return;
  if (t == 0) {
    out[int64_t(b) * T] = 0.f;
    return;
  }
  const int lo = max(1, t - W + 1);
  const int cnt = t - lo + 1;
  double z[2];
  for (int l = 0; l < 2; ++l) {
    const double* u = zs + l * span + (lo - first);
    double s = 0.0;
    for (int k = 0; k < cnt; ++k) s += u[k];
    const double mu = s / cnt;
    if (form == 1) {                           // rolling-mean form: g_bar(t)
      z[l] = mu;
      continue;
    }
    double v = 0.0;
    for (int k = 0; k < cnt; ++k) {
      const double d = u[k] - mu;
      v += d * d;
    }
    const double sd = sqrt(v / cnt);
    z[l] = (u[cnt - 1] - mu) / (sd + double(eps));
  }
  out[int64_t(b) * T + t] = float(z[0] - z[1]);
}

}  // namespace

size_t epikv_ws_bytes(int32_t batch, int32_t T) { return size_t(2) * batch * T * sizeof(float); }

hipError_t launch_epikv(const void* h_a, const void* h_b, int32_t batch, int32_t T, int32_t d_model, int32_t window,
                        float eps, int32_t form, float* g_out, float* scores, void* ws, hipStream_t st) {
  if (batch == 0 || T == 0) return hipSuccess;
  float* g = g_out ? g_out : static_cast<float*>(ws);
  const int runs = (T + kRun - 1) / kRun;
  const int64_t waves = int64_t(2) * batch * runs;
  const dim3 grid(unsigned((waves + 3) / 4));
  const uint16_t* a = static_cast<const uint16_t*>(h_a);
  const uint16_t* b = static_cast<const uint16_t*>(h_b);
  switch (d_model / 512) {
    case 1: hipLaunchKernelGGL(epikv_g_kernel<1>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
    case 2: hipLaunchKernelGGL(epikv_g_kernel<2>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
    case 4: hipLaunchKernelGGL(epikv_g_kernel<4>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
    case 8: hipLaunchKernelGGL(epikv_g_kernel<8>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
    case 16: hipLaunchKernelGGL(epikv_g_kernel<16>, grid, dim3(256), 0, st, a, b, batch, T, g); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t sh = size_t(2) * (kZTile + window - 1) * sizeof(double);
  hipLaunchKernelGGL(epikv_z_kernel, dim3(unsigned((T + kZTile - 1) / kZTile), unsigned(batch)), dim3(kZTile), sh, st,
                     g, batch, T, window, eps, form, scores);
  return hipGetLastError();
}

}  // namespace kve
