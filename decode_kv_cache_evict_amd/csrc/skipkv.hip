// Sentence-level redundancy score (SkipKV page, 核心方法 §4.1): a sentence's
// embedding is the mean of its tokens' last-layer hidden states; the pairwise
// sentence similarity (PSS) is the cosine of two embeddings, and of a pair
// with PSS >= tau the earlier sentence is the evictable one.  Per sentence the
// library returns its largest PSS with any later sentence (and the tau mark);
// per token it returns 1 - max(0, that PSS) of its sentence (1 after the last
// complete sentence), a score the protected top-K selection can consume.
//
//   sent_mean_kernel: one work-group per (sentence, request): fp32 sums of the
//     bf16 rows, 16-byte loads, then the mean scaled to unit length;
//   pss_kernel: 32x32 tiles of sentence pairs (upper triangle only), the dot
//     products of the unit means on the fp32 matrix cores (four waves, a
//     quarter of the dimensions each, summed in LDS); each row's best later
//     partner goes to a global order-preserving atomic maximum;
//   skipkv_finish_kernel: PSS, marks and per-token scores.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace kve {

namespace {

constexpr int kPssTile = 32;

__device__ __forceinline__ float order_key_to_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Sentence i of request b covers [lo, hi); an out-of-range or reversed span is empty.
__device__ __forceinline__ void sentence_span(const SkipArgs& a, int b, int i, int& lo, int& hi) {
  const int ns = min(max(a.n_sent[b], 0), a.max_sent);
  lo = hi = 0;
  if (i >= ns) return;
  const int32_t* st = a.starts + int64_t(b) * (a.max_sent + 1);
  lo = st[i];
  hi = st[i + 1];
  if (lo < 0 || hi > a.T || hi < lo) lo = hi = 0;
}

__global__ __launch_bounds__(256) void sent_mean_kernel(SkipArgs a) {
  __shared__ float red[4];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int lo, hi;
  sentence_span(a, b, i, lo, hi);
  const int nc = a.d_model / 8;                       // 16-byte chunks per row
  const uint4* h = static_cast<const uint4*>(a.h) + int64_t(b) * a.T * nc;
  float* e = a.emb + (int64_t(b) * a.max_sent + i) * a.d_model;
  float ss = 0.f;
  const float inv_n = hi > lo ? 1.f / float(hi - lo) : 0.f;
  for (int cchunk = tid; cchunk < nc; cchunk += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int t = lo;
    for (; t + 4 <= hi; t += 4) {                    // four rows' loads in flight, summed in token order
      uint4 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[u] = h[int64_t(t + u) * nc + cchunk];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t* v = reinterpret_cast<const uint16_t*>(&raw[u]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += bf16_to_f32(v[k]);
      }
    }
    for (; t < hi; ++t) {
      const uint4 raw = h[int64_t(t) * nc + cchunk];
      const uint16_t* v = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += bf16_to_f32(v[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[k] *= inv_n;
      ss = fmaf(acc[k], acc[k], ss);
      e[cchunk * 8 + k] = acc[k];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float nrm = sqrtf(red[0] + red[1] + red[2] + red[3]);
  const float inv = nrm > 0.f ? 1.f / nrm : 0.f;      // a zero mean stays zero: cosine 0 with everything
  for (int cchunk = tid; cchunk < nc; cchunk += 256)  // each thread rescales what it wrote
#pragma unroll
    for (int k = 0; k < 8; ++k) e[cchunk * 8 + k] *= inv;
}

__global__ __launch_bounds__(256) void pss_init_kernel(uint32_t* key, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) key[i] = float_order_key(-1.f);
}

// One work-group per 32x32 tile of sentence pairs (upper triangle of tiles).
// The tile's dot products run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: lane l holds A row l%16 and B column l%16 at
// k-slot l/16, and result rows 4*(l/16)+i of column l%16); the four waves split
// the dimensions into quarters and their partial tiles are summed in LDS.  A
// dot product does not depend on the order of its terms, so lane group q takes
// dimensions k + 4q .. k + 4q + 3 of each 16-dimension step with one 16-byte
// load and feeds them to four successive products.
__global__ __launch_bounds__(256) void pss_kernel(SkipArgs a) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ float part[4][kPssTile][kPssTile + 1];
  __shared__ uint32_t best[kPssTile];
  const int b = blockIdx.z, ti = blockIdx.y, tj = blockIdx.x;
  if (tj < ti) return;                                // upper triangle of tiles only
  const int ns = min(max(a.n_sent[b], 0), a.max_sent);
  const int i0 = ti * kPssTile, j0 = tj * kPssTile;
  if (i0 >= ns || j0 >= ns) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const float* E = a.emb + int64_t(b) * a.max_sent * a.d_model;
  const int last = a.max_sent - 1;                    // rows past the tile's end repeat a valid row (masked below)
  const float4* pa0 = reinterpret_cast<const float4*>(E + int64_t(min(i0 + r16, last)) * a.d_model);
  const float4* pa1 = reinterpret_cast<const float4*>(E + int64_t(min(i0 + 16 + r16, last)) * a.d_model);
  const float4* pb0 = reinterpret_cast<const float4*>(E + int64_t(min(j0 + r16, last)) * a.d_model);
  const float4* pb1 = reinterpret_cast<const float4*>(E + int64_t(min(j0 + 16 + r16, last)) * a.d_model);
  const int kq = a.d_model / 4;                       // dimensions per wave (a multiple of 16)
  const int kb = w * kq;
  f32x4 c00 = {0.f, 0.f, 0.f, 0.f}, c01 = c00, c10 = c00, c11 = c00;
  for (int k = kb; k < kb + kq; k += 16) {
    const int v = (k >> 2) + q;
    const float4 xa0 = pa0[v], xa1 = pa1[v], xb0 = pb0[v], xb1 = pb1[v];
    const float ea0[4] = {xa0.x, xa0.y, xa0.z, xa0.w}, ea1[4] = {xa1.x, xa1.y, xa1.z, xa1.w};
    const float eb0[4] = {xb0.x, xb0.y, xb0.z, xb0.w}, eb1[4] = {xb1.x, xb1.y, xb1.z, xb1.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c00 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea0[u], eb0[u], c00, 0, 0, 0);
      c01 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea0[u], eb1[u], c01, 0, 0, 0);
      c10 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea1[u], eb0[u], c10, 0, 0, 0);
      c11 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea1[u], eb1[u], c11, 0, 0, 0);
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    part[w][4 * q + x][r16] = c00[x];
    part[w][4 * q + x][16 + r16] = c01[x];
    part[w][16 + 4 * q + x][r16] = c10[x];
    part[w][16 + 4 * q + x][16 + r16] = c11[x];
  }
  if (tid < kPssTile) best[tid] = float_order_key(-1.f);
  __syncthreads();
  for (int e = tid; e < kPssTile * kPssTile; e += 256) {
    const int r = e / kPssTile, c = e % kPssTile;
    const int i = i0 + r, j = j0 + c;
    if (j > i && i < ns && j < ns) {
      const float dot = (part[0][r][c] + part[1][r][c]) + (part[2][r][c] + part[3][r][c]);
      atomicMax(&best[r], float_order_key(dot));
    }
  }
  __syncthreads();
  if (tid < kPssTile && i0 + tid < ns) atomicMax(&a.pss_key[int64_t(b) * a.max_sent + i0 + tid], best[tid]);
}

__global__ __launch_bounds__(256) void skipkv_finish_kernel(SkipArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n_tok = int64_t(a.batch) * a.T;
  if (idx < int64_t(a.batch) * a.max_sent) {          // per sentence: PSS and mark
    const float p = order_key_to_float(a.pss_key[idx]);
    a.pss_max[idx] = p;
    if (a.marks) a.marks[idx] = p >= a.tau ? 1 : 0;
  }
  if (idx >= n_tok) return;
  const int b = int(idx / a.T), t = int(idx % a.T);  // per token: its sentence's score
  const int ns = min(max(a.n_sent[b], 0), a.max_sent);
  const int32_t* st = a.starts + int64_t(b) * (a.max_sent + 1);
  float sc = 1.f;
  int lo = 0, hi = ns - 1;                            // last sentence i with start <= t
  int found = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (st[mid] <= t) {
      found = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  if (found >= 0) {
    int s0, s1;
    sentence_span(a, b, found, s0, s1);
    if (t >= s0 && t < s1) sc = 1.f - fmaxf(0.f, order_key_to_float(a.pss_key[int64_t(b) * a.max_sent + found]));
  }
  a.token_scores[idx] = sc;
}

}  // namespace

size_t skipkv_ws_bytes(int32_t batch, int32_t max_sent, int32_t d_model) {
  const size_t emb = (size_t(batch) * max_sent * d_model * sizeof(float) + 255) & ~size_t(255);
  return emb + size_t(batch) * max_sent * sizeof(uint32_t);
}

hipError_t launch_skipkv(SkipArgs& a, void* ws, hipStream_t st) {
  a.emb = static_cast<float*>(ws);
  a.pss_key = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) +
                                          ((size_t(a.batch) * a.max_sent * a.d_model * sizeof(float) + 255) &
                                           ~size_t(255)));
  const int n_sent_all = a.batch * a.max_sent;
  if (n_sent_all > 0) {
    hipLaunchKernelGGL(pss_init_kernel, dim3(unsigned((n_sent_all + 255) / 256)), dim3(256), 0, st, a.pss_key,
                       n_sent_all);
    hipLaunchKernelGGL(sent_mean_kernel, dim3(unsigned(a.max_sent), unsigned(a.batch)), dim3(256), 0, st, a);
    const unsigned nt = unsigned((a.max_sent + kPssTile - 1) / kPssTile);
    hipLaunchKernelGGL(pss_kernel, dim3(nt, nt, unsigned(a.batch)), dim3(256), 0, st, a);
  }
  const int64_t n = std::max(int64_t(a.batch) * a.T, int64_t(n_sent_all));
  if (n > 0)
    hipLaunchKernelGGL(skipkv_finish_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kve
