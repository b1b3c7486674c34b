// Continual farthest-point sampling of the beacon buffers (BeaconKV, "Continual
// FPS"): a head's bounded buffer of pre-RoPE queries that has filled to its
// capacity is shrunk to k_keep rows by FPS in the cosine geometry.
//
// One wavefront per buffer (up to 64 rows): lane r holds row r in registers and
// its inverse norm; the row just picked is broadcast from LDS; the distance to
// the picked set is kept per lane and the next pick is a wave argmax (largest
// distance, lowest row on ties).  Picked rows are written back oldest first.
#include "common.h"
#include "internal.h"

namespace kve {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void fps_kernel(const T* __restrict__ q_in, T* q_out,
                                                   const int32_t* count_in, int32_t* count_out, int n_buf, int cap,
                                                   int k_keep, int32_t* __restrict__ picks) {
  constexpr int VPR = D * int(sizeof(T)) / 16;      // 16-byte vectors per row
  constexpr int EPV = 16 / int(sizeof(T));          // elements per vector
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = blockIdx.x * 4 + w;
  const bool active = p < n_buf;
  uint4* rows = reinterpret_cast<uint4*>(smem) + size_t(w) * cap * VPR;   // this wave's buffer copy
  const int cnt = active ? count_in[p] : 0;
  const bool full = active && cnt == cap;

  const uint4* src = reinterpret_cast<const uint4*>(q_in + size_t(active ? p : 0) * cap * D);
  uint4* dst = reinterpret_cast<uint4*>(q_out + size_t(active ? p : 0) * cap * D);
  uint4 mine[VPR];
  const bool has_row = full && lane < cap;
#pragma unroll
  for (int v = 0; v < VPR; ++v) {
    mine[v] = has_row ? src[lane * VPR + v] : make_uint4(0, 0, 0, 0);
    if (has_row) rows[lane * VPR + v] = mine[v];
  }
  // Not full: copy through unchanged (a no-op in place).
  if (active && !full) {
    const int rows_n = cnt < 0 ? 0 : (cnt > cap ? cap : cnt);
    if (static_cast<const void*>(q_in) != static_cast<void*>(q_out))
      for (int e = lane; e < rows_n * VPR; e += kWave) dst[e] = src[e];
    if (lane == 0) count_out[p] = cnt;
    if (picks)
      for (int i = lane; i < k_keep; i += kWave) picks[size_t(p) * k_keep + i] = -1;
  }
  __syncthreads();
  if (!full) return;

  auto dot_with = [&](const uint4* other) {
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < VPR; ++v) {
      const uint4 a = mine[v];
      const uint4 b = other[v];
      const T* ea = reinterpret_cast<const T*>(&a);
      const T* eb = reinterpret_cast<const T*>(&b);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc = fmaf(Elem<T>::widen(ea[e]), Elem<T>::widen(eb[e]), acc);
    }
    return acc;
  };
  const float nrm = sqrtf(dot_with(mine));
  const float inv = 1.f / fmaxf(nrm, 1e-30f);
  const float inv0 = __shfl(inv, 0, kWave);
  float dist = has_row ? 1.f - dot_with(rows) * inv * inv0 : -__builtin_huge_valf();
  bool taken = lane == 0;
  int my_pick = lane == 0 ? 0 : -1;                // lane i records the i-th pick
  for (int step = 1; step < k_keep; ++step) {
    float v = (has_row && !taken) ? dist : -__builtin_huge_valf();
    int idx = lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, kWave);
      const int oi = __shfl_xor(idx, o, kWave);
      if (ov > v || (ov == v && oi < idx)) {
        v = ov;
        idx = oi;
      }
    }
    const int j = idx < cap ? idx : cap - 1;        // uniform across the wave
    if (lane == j) taken = true;
    if (lane == step) my_pick = j;
    const float invj = __shfl(inv, j, kWave);
    const float dj = 1.f - dot_with(rows + j * VPR) * inv * invj;
    dist = fminf(dist, dj);
  }
  const uint64_t tm = __ballot(taken && has_row);
  if (taken && has_row) {
    const int rank = __popcll(tm & ((uint64_t(1) << lane) - 1));
#pragma unroll
    for (int v = 0; v < VPR; ++v) dst[rank * VPR + v] = mine[v];
  }
  if (picks && lane < k_keep) picks[size_t(p) * k_keep + lane] = my_pick;
  if (lane == 0) count_out[p] = k_keep;
}

template <typename T, int D>
hipError_t launch_fps_t(const void* q_in, void* q_out, const int32_t* ci, int32_t* co, int n_buf, int cap, int k,
                        int32_t* picks, hipStream_t st) {
  const size_t sh = size_t(4) * cap * D * sizeof(T);
  hipLaunchKernelGGL((fps_kernel<T, D>), dim3(unsigned((n_buf + 3) / 4)), dim3(256), sh, st,
                     static_cast<const T*>(q_in), static_cast<T*>(q_out), ci, co, n_buf, cap, k, picks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fps(const void* q_in, void* q_out, const int32_t* count_in, int32_t* count_out, int32_t n_buf,
                      int32_t cap, int32_t k_keep, int32_t head_dim, int32_t dtype, int32_t* picks, hipStream_t st) {
  if (n_buf == 0) return hipSuccess;
  if (dtype == 0)
    return head_dim == 128 ? launch_fps_t<uint16_t, 128>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st)
                           : launch_fps_t<uint16_t, 64>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st);
  return head_dim == 128 ? launch_fps_t<float, 128>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st)
                         : launch_fps_t<float, 64>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st);
}

}  // namespace kve
