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
//   pss_kernel: 32x32 tiles of sentence pairs (upper triangle only), the unit
//     means staged through LDS 64 dimensions at a time, 2x2 dot products per
//     thread in fp32; each row's best later partner goes to a global
//     order-preserving atomic maximum;
//   skipkv_finish_kernel: PSS, marks and per-token scores.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace kve {

namespace {

constexpr int kPssTile = 32;
constexpr int kPssK = 64;

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
    for (int t = lo; t < hi; ++t) {
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

__global__ __launch_bounds__(256) void pss_kernel(SkipArgs a) {
  __shared__ float A[kPssTile][kPssK + 1], Bt[kPssTile][kPssK + 1];
  __shared__ uint32_t best[kPssTile];
  const int b = blockIdx.z, ti = blockIdx.y, tj = blockIdx.x;
  if (tj < ti) return;                                // upper triangle of tiles only
  const int ns = min(max(a.n_sent[b], 0), a.max_sent);
  const int i0 = ti * kPssTile, j0 = tj * kPssTile;
  if (i0 >= ns || j0 >= ns) return;
  const int tid = threadIdx.x;
  const int ri = (tid / 16) * 2, cj = (tid % 16) * 2;   // this thread's 2x2 block
  const float* E = a.emb + int64_t(b) * a.max_sent * a.d_model;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  if (tid < kPssTile) best[tid] = float_order_key(-1.f);
  for (int k0 = 0; k0 < a.d_model; k0 += kPssK) {
    __syncthreads();
    for (int x = tid; x < kPssTile * kPssK; x += 256) {
      const int r = x / kPssK, k = x % kPssK;
      A[r][k] = i0 + r < ns ? E[int64_t(i0 + r) * a.d_model + k0 + k] : 0.f;
      Bt[r][k] = j0 + r < ns ? E[int64_t(j0 + r) * a.d_model + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kPssK; ++k) {
      const float a0 = A[ri][k], a1 = A[ri + 1][k], b0 = Bt[cj][k], b1 = Bt[cj + 1][k];
      acc[0][0] = fmaf(a0, b0, acc[0][0]);
      acc[0][1] = fmaf(a0, b1, acc[0][1]);
      acc[1][0] = fmaf(a1, b0, acc[1][0]);
      acc[1][1] = fmaf(a1, b1, acc[1][1]);
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int i = i0 + ri + x, j = j0 + cj + y;
      if (j > i && i < ns && j < ns) atomicMax(&best[ri + x], float_order_key(acc[x][y]));
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
