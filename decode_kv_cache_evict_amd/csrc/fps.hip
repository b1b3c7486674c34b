// Continual farthest-point sampling of the beacon buffers (BeaconKV, "Continual
// FPS"): a head's bounded buffer of pre-RoPE queries that has filled to its
// capacity is shrunk to k_keep rows by FPS in the cosine geometry.
//
// One wavefront per buffer (up to 64 rows): lane r owns row r's distance to the
// picked set; the next pick is a wave argmax (largest distance, lowest row on
// ties).  Picked rows are written back oldest first.  fp32 buffers take the dot
// products on the vector ALUs (lane r holds row r, the pick is broadcast from
// LDS); bf16 buffers read them from the Gram matrix (below).
#include "common.h"
#include "internal.h"

namespace kve {

namespace {

// The lane holding the largest v, the lowest lane among equal values (-0.0
// equals +0.0), the same in every lane: one 64-bit max reduction over
// (order key of v, inverted lane index), moved between lanes with DPP and the
// row swaps.
__device__ __forceinline__ int wave_argmax_low(float v, int idx) {
  const uint64_t key = (uint64_t(float_order_key(v)) << 32) | uint64_t(~uint32_t(idx));
  const uint64_t m = wave_reduce(key, [](uint64_t x, uint64_t y) { return x > y ? x : y; });
  return __builtin_amdgcn_readfirstlane(int(~uint32_t(m)));
}
__device__ __forceinline__ float lane_value(float v, int lane) {   // lane: wave-uniform
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

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
  const float inv0 = lane_value(inv, 0);
  float dist = has_row ? 1.f - dot_with(rows) * inv * inv0 : -__builtin_huge_valf();
  bool taken = lane == 0;
  int my_pick = lane == 0 ? 0 : -1;                // lane i records the i-th pick
  for (int step = 1; step < k_keep; ++step) {
    const int idx = wave_argmax_low((has_row && !taken) ? dist : -__builtin_huge_valf(), lane);
    const int j = idx < cap ? idx : cap - 1;        // uniform across the wave
    if (lane == j) taken = true;
    if (lane == step) my_pick = j;
    const float invj = lane_value(inv, j);
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

// bf16 buffers: the cosine geometry comes from the buffer's Gram matrix,
// formed once on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 sums) and
// kept in LDS; each FPS step then reads one row of it.  One wavefront per
// buffer.  The rows are held in registers as MFMA fragments: lane l holds
// rows 16*t + l%16 (tile t), 16-byte slice 8*(l/16) + 32*ks of each 32-wide
// k-step; since the second operand of X X^T is X itself, the same fragments
// serve both.  Picked rows are written back, oldest first, from the fragments.
template <int D, int NT>
__global__ __launch_bounds__(256) void fps_gram_kernel(const uint16_t* __restrict__ q_in, uint16_t* q_out,
                                                        const int32_t* count_in, int32_t* count_out, int n_buf,
                                                        int cap, int k_keep, int32_t* __restrict__ picks) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int KS = D / 32;                        // k-steps
  constexpr int CAP = 16 * NT;                      // padded rows
  __shared__ float gram[4][CAP * CAP];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = blockIdx.x * 4 + w;
  if (p >= n_buf) return;                           // wave-uniform: no block barrier below
  const int cnt = count_in[p];
  const uint4* src = reinterpret_cast<const uint4*>(q_in + size_t(p) * cap * D);
  uint4* dst = reinterpret_cast<uint4*>(q_out + size_t(p) * cap * D);
  constexpr int VPR = D / 8;                        // 16-byte vectors per row
  if (cnt != cap) {                                 // not full: copy through unchanged (a no-op in place)
    const int rows_n = cnt < 0 ? 0 : (cnt > cap ? cap : cnt);
    if (static_cast<const void*>(q_in) != static_cast<void*>(q_out))
      for (int e = lane; e < rows_n * VPR; e += kWave) dst[e] = src[e];
    if (lane == 0) count_out[p] = cnt;
    if (picks)
      for (int i = lane; i < k_keep; i += kWave) picks[size_t(p) * k_keep + i] = -1;
    return;
  }
  const int col = lane & 15, quad = lane >> 4;
  uint4 frag[NT][KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * t + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      frag[t][ks] = r < cap ? src[r * VPR + ks * 4 + quad] : make_uint4(0, 0, 0, 0);
  }
  float* G = gram[w];
#pragma unroll
  for (int ti = 0; ti < NT; ++ti)
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, frag[ti][ks]),
                                                      __builtin_bit_cast(bf16x8, frag[tj][ks]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) G[(16 * ti + 4 * quad + i) * CAP + 16 * tj + col] = acc[i];
    }
  __builtin_amdgcn_s_waitcnt(0);                    // this wave's LDS writes before its reads
  __builtin_amdgcn_wave_barrier();
  const bool has_row = lane < cap;
  const float nrm = has_row ? sqrtf(fmaxf(G[lane * CAP + lane], 0.f)) : 0.f;
  const float inv = 1.f / fmaxf(nrm, 1e-30f);
  const float inv0 = lane_value(inv, 0);
  float dist = has_row ? 1.f - G[lane] * inv * inv0 : -__builtin_huge_valf();   // row 0 of G = column 0
  bool taken = lane == 0;
  int my_pick = lane == 0 ? 0 : -1;                 // lane i records the i-th pick
  for (int step = 1; step < k_keep; ++step) {
    const int idx = wave_argmax_low((has_row && !taken) ? dist : -__builtin_huge_valf(), lane);
    const int j = idx < cap ? idx : cap - 1;         // uniform across the wave
    if (lane == j) taken = true;
    if (lane == step) my_pick = j;
    const float invj = lane_value(inv, j);
    if (has_row) dist = fminf(dist, 1.f - G[j * CAP + lane] * inv * invj);
  }
  const uint64_t tm = __ballot(taken && has_row);
  const int rank = __popcll(tm & ((uint64_t(1) << lane) - 1));   // output slot of row `lane` if taken
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 16 * t + col;
    const int rr = __shfl(rank, r < 64 ? r : 0, kWave);
    const bool keep = r < cap && ((tm >> r) & 1);
    if (keep)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[rr * VPR + ks * 4 + quad] = frag[t][ks];
  }
  if (picks && lane < k_keep) picks[size_t(p) * k_keep + lane] = my_pick;
  if (lane == 0) count_out[p] = k_keep;
}

template <int D>
hipError_t launch_fps_gram(const void* q_in, void* q_out, const int32_t* ci, int32_t* co, int n_buf, int cap, int k,
                           int32_t* picks, hipStream_t st) {
  const dim3 grid(unsigned((n_buf + 3) / 4));
  const uint16_t* in = static_cast<const uint16_t*>(q_in);
  uint16_t* out = static_cast<uint16_t*>(q_out);
  switch ((cap + 15) / 16) {
    case 1: hipLaunchKernelGGL((fps_gram_kernel<D, 1>), grid, dim3(256), 0, st, in, out, ci, co, n_buf, cap, k, picks); break;
    case 2: hipLaunchKernelGGL((fps_gram_kernel<D, 2>), grid, dim3(256), 0, st, in, out, ci, co, n_buf, cap, k, picks); break;
    case 3: hipLaunchKernelGGL((fps_gram_kernel<D, 3>), grid, dim3(256), 0, st, in, out, ci, co, n_buf, cap, k, picks); break;
    default: hipLaunchKernelGGL((fps_gram_kernel<D, 4>), grid, dim3(256), 0, st, in, out, ci, co, n_buf, cap, k, picks); break;
  }
  return hipGetLastError();
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
    return head_dim == 128 ? launch_fps_gram<128>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st)
                           : launch_fps_gram<64>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st);
  return head_dim == 128 ? launch_fps_t<float, 128>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st)
                         : launch_fps_t<float, 64>(q_in, q_out, count_in, count_out, n_buf, cap, k_keep, picks, st);
}

}  // namespace kve
