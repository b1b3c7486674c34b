// Decode attention over the (compacted) cache: for every request b and query
// head h of the new token, softmax(q . k / sqrt(d)) over all cached rows of
// KV head h / G, applied to V.  This is the step that follows eviction in the
// decode loop (the EPIKV page's part 4 keeps the eviction score compatible
// with a fused attention kernel; the BeaconKV page's throughput figures are
// decode throughput over the compacted cache).  The rows may be in any order
// (the in-place compaction does not keep slot order).
//
// Split over keys: one work-group per (segment, 1024-row chunk) keeps, for
// each of the G query rows of the segment, a running maximum, sum and output
// over its chunk in 64-row tiles staged through LDS (one row per lane for the
// logits; 8 output elements per lane for the weighted V sum), and writes
// them to the workspace; a second kernel merges each segment's chunks.  The
// logits are taken in log2 units (scaled by log2(e)/sqrt(d)) and exponentiated
// with exp2.  fp32 accumulation.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace kve {

namespace {

constexpr int kAttnChunk = 1024;   // rows per work-group
constexpr int kAttnTile = 64;      // rows per LDS tile

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  constexpr int RB = D * int(sizeof(T));           // bytes per row
  constexpr int RS = RB + 16;                      // padded LDS row stride
  constexpr int CPR = RB / 16;                     // 16-byte chunks per row
  constexpr int LPT = kAttnTile * CPR / 256;       // chunks per thread per tile (each of K and V)
  constexpr int EPC = 16 / int(sizeof(T));         // elements per chunk
  constexpr int NSL = D / 8;                       // 8-element output slices per query
  constexpr int KS = 64 / NSL;                     // key subsets per (query, slice)
  __shared__ __attribute__((aligned(16))) unsigned char kt[kAttnTile * RS];
  __shared__ __attribute__((aligned(16))) unsigned char vt[kAttnTile * RS];
  __shared__ float qs[G][D];
  __shared__ float pr[G][kAttnTile];               // logits, then probabilities
  __shared__ float alpha[G];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const int64_t off = a.seg_off[s];
  const int n = a.seg_len[s];
  if (!(n >= 0 && n <= a.max_seg_len && off >= 0 && off + n <= a.n_rows)) return;
  const int k0 = ch * kAttnChunk;
  if (k0 >= n) return;
  const int k1 = min(n, k0 + kAttnChunk);
  const int b = s / a.n_kv, g = s % a.n_kv;
  const float c = kLog2e / sqrtf(float(D));
  const T* q = static_cast<const T*>(a.q) + (int64_t(b) * a.n_q + g * G) * D;
  for (int e = tid; e < G * D; e += 256) qs[e / D][e % D] = Elem<T>::widen(q[e]);

  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* kg = static_cast<const u32x4*>(a.k);
  const u32x4* vg = static_cast<const u32x4*>(a.v);
  u32x4 pk[LPT], pv[LPT];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = u * 256 + tid, r = idx / CPR, part = idx % CPR;
      const bool ok = kb + r < k1;
      const int64_t row = off + (ok ? kb + r : k0);
      pk[u] = ok ? kg[row * CPR + part] : u32x4{0u, 0u, 0u, 0u};
      pv[u] = ok ? __builtin_nontemporal_load(&vg[row * CPR + part]) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int idx = u * 256 + tid, r = idx / CPR, part = idx % CPR;
      *reinterpret_cast<u32x4*>(kt + r * RS + part * 16) = pk[u];
      *reinterpret_cast<u32x4*>(vt + r * RS + part * 16) = pv[u];
    }
  };
  // running statistics of query rows w, w+4 (held by wave w); output accumulators
  float m_run[(G + 3) / 4], l_run[(G + 3) / 4];
#pragma unroll
  for (int i = 0; i < (G + 3) / 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  const int sl = lane / KS, ks = lane % KS;        // output slice and key subset of this lane
  float acc[(G + 3) / 4][8];
#pragma unroll
  for (int i = 0; i < (G + 3) / 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

  load_tile(k0);
  for (int kb = k0; kb < k1; kb += kAttnTile) {
    __syncthreads();                               // previous tile's readers are done
    store_tile();
    if (kb + kAttnTile < k1) load_tile(kb + kAttnTile);
    __syncthreads();
    // logits: lane = row of the tile; waves take query rows w, w+4
    const bool live = kb + lane < k1;
#pragma unroll
    for (int i = 0; i < (G + 3) / 4; ++i) {
      const int qi = w + 4 * i;
      if (qi < G) {
        float x = 0.f;
#pragma unroll
        for (int cpart = 0; cpart < CPR; ++cpart) {
          const uint4 raw = *reinterpret_cast<const uint4*>(kt + lane * RS + cpart * 16);
          const T* ev = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int e = 0; e < EPC; ++e) x = fmaf(Elem<T>::widen(ev[e]), qs[qi][cpart * EPC + e], x);
        }
        // online softmax of this tile for query qi (the whole wave holds it)
        const float y = live ? x * c : -INFINITY;
        const float m_new = fmaxf(m_run[i], wave_max(y));
        const float sc = exp2f(m_run[i] - m_new);   // 0 on the first tile
        const float p = live ? exp2f(y - m_new) : 0.f;
        l_run[i] = l_run[i] * sc + wave_sum(p);
        m_run[i] = m_new;
        pr[qi][lane] = p;
        if (lane == 0) alpha[qi] = sc;
      }
    }
    __syncthreads();
    // weighted V: lane -> (slice sl, key subset ks); waves take query rows w, w+4
#pragma unroll
    for (int i = 0; i < (G + 3) / 4; ++i) {
      const int qi = w + 4 * i;
      if (qi < G) {
        const float sc = alpha[qi];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] *= sc;
#pragma unroll 4
        for (int r = ks; r < kAttnTile; r += KS) {
          const float p = pr[qi][r];
          const unsigned char* vrow = vt + r * RS + sl * 8 * int(sizeof(T));
          if (sizeof(T) == 2) {
            const uint4 raw = *reinterpret_cast<const uint4*>(vrow);
            const T* ev = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(p, Elem<T>::widen(ev[e]), acc[i][e]);
          } else {
            const uint4 r0 = *reinterpret_cast<const uint4*>(vrow);
            const uint4 r1 = *reinterpret_cast<const uint4*>(vrow + 16);
            const T* e0 = reinterpret_cast<const T*>(&r0);
            const T* e1 = reinterpret_cast<const T*>(&r1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[i][e] = fmaf(p, Elem<T>::widen(e0[e]), acc[i][e]);
              acc[i][4 + e] = fmaf(p, Elem<T>::widen(e1[e]), acc[i][4 + e]);
            }
          }
        }
      }
    }
  }
  // merge the key subsets (consecutive lanes) and write this chunk's partials
  float* part = a.part + (int64_t(s) * a.n_chunks + ch) * G * (D + 2);
#pragma unroll
  for (int i = 0; i < (G + 3) / 4; ++i) {
    const int qi = w + 4 * i;
    if (qi < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int o = 1; o < KS; o <<= 1) acc[i][e] += __shfl_xor(acc[i][e], o, kWave);
      float* pq = part + qi * (D + 2);
      if (ks == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) pq[sl * 8 + e] = acc[i][e];
      if (lane == 0) {
        pq[D] = m_run[i];
        pq[D + 1] = l_run[i];
      }
    }
  }
}

// Merge each segment's chunk partials: out = sum_c o_c 2^(m_c - M) / L, L =
// sum_c l_c 2^(m_c - M); lse in natural log.  One work-group per segment.
template <int D, int G>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int s = blockIdx.x;
  const int64_t off = a.seg_off[s];
  const int n = a.seg_len[s];
  const bool ok = n >= 0 && n <= a.max_seg_len && off >= 0 && off + n <= a.n_rows;
  const int nch = ok ? (n + kAttnChunk - 1) / kAttnChunk : 0;
  const int b = s / a.n_kv, g = s % a.n_kv;
  const float* part = a.part + int64_t(s) * a.n_chunks * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int qi = e / D, d = e % D;
    float M = -INFINITY;
    for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, part[(cc * G + qi) * (D + 2) + D]);
    float L = 0.f, o = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
      const float* pq = part + (cc * G + qi) * (D + 2);
      const float f = exp2f(pq[D] - M);
      L += pq[D + 1] * f;
      o += pq[d] * f;
    }
    const int64_t row = int64_t(b) * a.n_q + g * G + qi;
    a.out[row * D + d] = L > 0.f ? o / L : 0.f;     // an empty or rejected segment gives zeros
    if (d == 0 && a.lse) a.lse[row] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
  }
}

template <typename T, int D, int G>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_partial_kernel<T, D, G>), dim3(unsigned(int64_t(a.n_seg) * a.n_chunks)), dim3(256), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3(unsigned(a.n_seg)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_g(const AttnArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_attn_t<T, D, 1>(a, st);
    case 2: return launch_attn_t<T, D, 2>(a, st);
    case 4: return launch_attn_t<T, D, 4>(a, st);
    case 8: return launch_attn_t<T, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t attn_workspace_bytes(int32_t n_seg, int32_t max_seg_len, int32_t group, int32_t head_dim) {
  const size_t nch = (size_t(max_seg_len) + kAttnChunk - 1) / kAttnChunk;
  return size_t(n_seg) * (nch ? nch : 1) * group * (head_dim + 2) * sizeof(float);
}

hipError_t launch_decode_attention(AttnArgs& a, hipStream_t st) {
  a.n_chunks = (a.max_seg_len + kAttnChunk - 1) / kAttnChunk;
  if (a.n_seg == 0) return hipSuccess;
  if (a.n_chunks == 0) a.n_chunks = 1;              // every segment is empty: the combine writes zeros
  if (a.dtype == 0)
    return a.head_dim == 128 ? launch_attn_g<uint16_t, 128>(a, st) : launch_attn_g<uint16_t, 64>(a, st);
  return a.head_dim == 128 ? launch_attn_g<float, 128>(a, st) : launch_attn_g<float, 64>(a, st);
}

}  // namespace kve
