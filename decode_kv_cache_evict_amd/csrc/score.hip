// Observation-set attention scores (BeaconKV, "打分时的 RoPE 对齐"):
//   scores[j] = max over the group's observation rows r of softmax_r(q_r . k_j / sqrt(d))
// computed in two passes over each segment's keys:
//   pass 1: per (segment, 256-key chunk) work-group, partial row statistics
//           (running max m, sum of exp2 below it) of the logits;
//   pass 2: merge the chunk statistics into each row's log-sum-exp, recompute
//           the logits of the chunk and take the per-key maximum of exp2(x - lse).
// The bf16 path contracts on the matrix cores (v_mfma_f32_16x16x32_bf16) with
// key tiles staged through LDS by coalesced 16-byte loads; a plain VALU path
// serves fp32 caches.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "budget_common.h"
#include "common.h"
#include "internal.h"
#include "select_common.h"

namespace kve {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kInf = __builtin_huge_valf();

// Position a key is compared against by observation row r of segment s;
// -1 marks an absent row (never sees a key).
__device__ __forceinline__ int row_position(const ScoreArgs& a, int b, int r) {
  if (r >= a.rows) return -1;
  const int i = r % a.max_obs;
  const int no = a.n_obs ? a.n_obs[b] : a.max_obs;
  if (i >= no) return -1;
  return a.causal ? a.q_pos[b * a.max_obs + i] : INT_MAX - 1;
}

__device__ __forceinline__ int64_t row_qr_index(const ScoreArgs& a, int b, int g, int r) {
  const int h = g * a.group + r / a.max_obs;
  const int i = r % a.max_obs;
  return (int64_t(b) * a.n_q + h) * a.max_obs + i;
}

// 1 / (number of observation rows that exist for request b): the denominator of
// the mean aggregation (every existing row counts, including a row that sees
// no key yet).
__device__ __forceinline__ float live_row_inverse(const ScoreArgs& a, int b) {
  const int no = a.n_obs ? min(a.n_obs[b], a.max_obs) : a.max_obs;
  return no > 0 ? 1.f / float(a.group * no) : 0.f;
}

__device__ __forceinline__ bool segment_ok(const ScoreArgs& a, int s, int64_t& off, int& n) {
  off = a.seg_off[s];
  n = a.seg_len[s];
  return n >= 0 && n <= a.max_seg_len && off >= 0 && off + n <= a.n_rows;
}

// ------------------------------------------------------------ query rotation
// Rotate every observation row to its q_pos (double-precision angle and
// rotation) and round to the storage dtype; rows past n_obs are zeroed.  One
// work-group per block of R consecutive observation rows of one request (R
// chosen on the host so a block holds about 256 rotation items): its threads
// first form the R * D/2 sines and cosines, one each, into LDS (the angles
// are shared by every query head), then each thread rotates its items, one
// item being V frequencies of one row of one head (both halves, 16-byte loads
// and stores), all of its loads issued before the first rotation.  Items run
// fastest over the frequencies and then the rows, which are contiguous in
// memory for one head.  Work-groups past the row blocks only clear the
// n_zero control ints of the scoring kernel that follows (queue tickets and
// arrival counters): one launch fewer, and no memset node when the call is
// captured in a graph.
constexpr int kRotMaxAngles = 512;                // sines and cosines per work-group (LDS)
constexpr int kRotItems = 4;                      // items per thread in flight

template <typename T>
__global__ __launch_bounds__(256) void rotate_obs_kernel(const T* __restrict__ q, const int32_t* __restrict__ q_pos,
                                                         const int32_t* __restrict__ n_obs, T* __restrict__ qr,
                                                         int n_blocks, int rblk, int n_q, int max_obs, int D,
                                                         InvFreq inv, int* __restrict__ zero, int n_zero) {
  constexpr int V = 16 / int(sizeof(T));          // frequencies per item
  __shared__ double2 cs_s[kRotMaxAngles];         // (cos, sin) of row r, frequency i at r * half + i
  const int tid = threadIdx.x;
  for (int64_t z = int64_t(blockIdx.x) * blockDim.x + tid; z < n_zero; z += int64_t(gridDim.x) * blockDim.x)
    zero[z] = 0;
  if (int(blockIdx.x) >= n_blocks) return;
  const int half = D / 2, runs = half / V;
  const int obl = (max_obs + rblk - 1) / rblk;    // row blocks per request
  const int b = int(blockIdx.x) / obl, o0 = int(blockIdx.x) % obl * rblk;
  const int nr = min(rblk, max_obs - o0);
  const int no = n_obs ? n_obs[b] : max_obs;
  for (int e = tid; e < nr * half; e += blockDim.x) {
    const int r = e / half, i = e % half;
    double sn = 0.0, cs = 1.0;
    if (o0 + r < no) {
      const double ang = double(q_pos[int64_t(b) * max_obs + o0 + r]) * inv.v[i];
      sincos(ang, &sn, &cs);
    }
    cs_s[e] = make_double2(cs, sn);
  }
  __syncthreads();
  const int n_items = nr * n_q * runs;
  for (int it0 = 0; it0 < n_items; it0 += kRotItems * int(blockDim.x)) {
    uint4 x[kRotItems], y[kRotItems];
    int64_t at[kRotItems];
    bool live[kRotItems];
#pragma unroll
    for (int u = 0; u < kRotItems; ++u) {
      if (it0 + u * int(blockDim.x) >= n_items) break;                  // the same for every thread
      const int it = min(it0 + u * int(blockDim.x) + tid, n_items - 1);   // past the end: repeat the last item
      const int run = it % runs, r = it / runs % nr, h = it / runs / nr;
      at[u] = ((int64_t(b) * n_q + h) * max_obs + o0 + r) * D + run * V;
      live[u] = o0 + r < no;
      x[u] = live[u] ? *reinterpret_cast<const uint4*>(q + at[u]) : make_uint4(0, 0, 0, 0);
      y[u] = live[u] ? *reinterpret_cast<const uint4*>(q + at[u] + half) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRotItems; ++u) {
      const int it = it0 + u * int(blockDim.x) + tid;
      if (it >= n_items) break;
      const int run = it % runs, r = it / runs % nr;
      uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
      if (live[u]) {
        const T* xe = reinterpret_cast<const T*>(&x[u]);
        const T* ye = reinterpret_cast<const T*>(&y[u]);
        T* le = reinterpret_cast<T*>(&lo);
        T* he = reinterpret_cast<T*>(&hi);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const double2 c = cs_s[r * half + run * V + v];
          const RotPair p = rotate_pair(double(Elem<T>::widen(xe[v])), double(Elem<T>::widen(ye[v])), c.x, c.y);
          le[v] = Elem<T>::from_f64(p.a);
          he[v] = Elem<T>::from_f64(p.b);
        }
      }
      *reinterpret_cast<uint4*>(qr + at[u]) = lo;
      *reinterpret_cast<uint4*>(qr + at[u] + half) = hi;
    }
  }
}

// Merge each row's chunk statistics into its log-sum-exp (log2 units); +inf
// when the row saw no key.  One thread per (segment, row).
__global__ __launch_bounds__(256) void merge_lse_kernel(ScoreArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(a.n_seg) * a.rows) return;
  const int s = int(idx / a.rows), r = int(idx % a.rows);
  const int n = a.seg_len[s];
  const int nch = (n >= 0 && n <= a.max_seg_len) ? (n + a.chunk - 1) / a.chunk : 0;
  const float2* st = a.stats + int64_t(s) * a.n_chunks * a.rows + r;
  float M = kNegBig, L = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 8) {        // eight independent loads in flight, merged online
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + u < nch ? st[int64_t(c0 + u) * a.rows] : make_float2(kNegBig, 0.f);
    float M2 = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) M2 = fmaxf(M2, v[u].x);
    L *= exp2f(M - M2);
#pragma unroll
    for (int u = 0; u < 8; ++u) L += v[u].y * exp2f(v[u].x - M2);
    M = M2;
  }
  a.lse[idx] = L > 0.f ? M + log2f(L) : kInf;
}

// ------------------------------------------------------------ VALU path
// One thread per key; query rows broadcast from LDS.  Used for fp32 caches.
template <typename T, int D, bool PASS2>
__global__ __launch_bounds__(256) void score_valu_kernel(ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* qs = reinterpret_cast<T*>(smem);                                   // [rows, D]
  float2* wst = reinterpret_cast<float2*>(smem + size_t(a.rows) * D * sizeof(T));  // [4, rows]
  float* lse_s = reinterpret_cast<float*>(wst + 4 * a.rows);            // [rows]
  int* rp_s = reinterpret_cast<int*>(lse_s + a.rows);                   // [rows]

  const int s = blockIdx.y, ch = blockIdx.x;
  int64_t off;
  int n;
  if (!segment_ok(a, s, off, n)) return;
  const int k0 = ch * a.chunk;
  if (k0 >= n) return;
  const int b = s / a.n_kv, g = s % a.n_kv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float c = kLog2e / sqrtf(float(D));
  const T* qr = static_cast<const T*>(a.qr);

  for (int e = tid; e < a.rows * D; e += blockDim.x) {
    const int r = e / D, d = e % D;
    qs[e] = qr[row_qr_index(a, b, g, r) * D + d];
  }
  for (int r = tid; r < a.rows; r += blockDim.x) {
    rp_s[r] = row_position(a, b, r);
    if (PASS2) lse_s[r] = a.lse[int64_t(s) * a.rows + r];
  }
  __syncthreads();

  const int j = k0 + tid;
  const bool valid = j < n;
  float kv[D];
  int kpos = INT_MAX;
  const T* kp = static_cast<const T*>(a.k) + (off + (valid ? j : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) kv[d] = valid ? Elem<T>::widen(kp[d]) : 0.f;
  if (valid) kpos = a.pos[off + j];

  float best = -kInf, sum = 0.f;
  for (int r = 0; r < a.rows; ++r) {
    const T* qrow = qs + r * D;
    float x = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) x = fmaf(Elem<T>::widen(qrow[d]), kv[d], x);
    const bool vis = valid && kpos <= rp_s[r];
    if (PASS2) {
      const float y = vis ? fmaf(x, c, -lse_s[r]) : -kInf;
      best = fmaxf(best, y);
      if (a.aggregate) sum += vis ? exp2f(y) : 0.f;
    } else {
      const float xv = vis ? x : -kInf;
      const float m = wave_max(fmaxf(xv, kNegBig));
      const float l = wave_sum(vis ? exp2f(fmaf(x, c, -m * c)) : 0.f);
      if (lane == 0) wst[w * a.rows + r] = make_float2(m, l);
    }
  }
  if (PASS2) {
    if (valid) a.scores[off + j] = a.aggregate ? sum * live_row_inverse(a, b) : exp2f(best);
    return;
  }
  __syncthreads();
  for (int r = tid; r < a.rows; r += blockDim.x) {
    float M = kNegBig;
    for (int q = 0; q < 4; ++q) M = fmaxf(M, wst[q * a.rows + r].x);
    float L = 0.f;
    for (int q = 0; q < 4; ++q) {
      const float2 v = wst[q * a.rows + r];
      L += v.y * exp2f((v.x - M) * c);
    }
    a.stats[(int64_t(s) * a.n_chunks + ch) * a.rows + r] = make_float2(M * c, L);
  }
}

// ------------------------------------------------------------ MFMA path (bf16)
// Two launches over (segment, 1024-key chunk) work-groups of 4 waves: pass 1
// publishes per-chunk row statistics, merge_lse_kernel folds them into each
// row's log-sum-exp, pass 2 recomputes the logits and keeps the per-key max.
//
// Wave w owns row tiles w*RT .. w*RT+RT-1 (16 rows each) and keeps their
// rotated queries in registers as MFMA A operands; keys stream through a
// double-buffered LDS tile of 64 keys (one barrier per tile) that every wave
// reads as B operands.  For v_mfma_f32_16x16x32_bf16 lane l holds A row l%16 /
// B column l%16 with k-slice 8*(l/16)..+7 of each 32-wide step, and result rows
// 4*(l/16)+i of column l%16.  The epilogue works on two 16-key tiles at a time.
//
// Pass 1 keeps, per lane and row, a reference value m and l = sum of
// exp2(c*x - c*m) over the keys it has seen.  m is only moved when a sum leaves
// [0, 2^64] (a term overflowed or grew far above the reference): the tiles are
// then redone with m raised to the running maximum.  The first tiles always take
// that path (m starts at -1e30), later ones almost never, so the common case
// costs one fma, one exp and one add per logit.  The causal mask is applied only
// to tiles holding a key newer than the wave's earliest query position.
constexpr float kBig = 18446744073709551616.0f;   // 2^64

// ---------------------------------------------------------------- phase stamps
// Built with -DKVE_STAMPS (libkvevict_stamps.so), the one-call trigger kernels
// record the memory-clock time (s_memrealtime) at each phase boundary of every
// work-group item (ticket) below kStampItems; kve_debug_stamps() copies them
// out.  Phases: 0 item taken, 1 pass 1 done and its row statistics stored,
// 2 first segment barrier passed, 3 log-sum-exp merged, 4 pass 2 done,
// 5 second meeting passed (scores, and with entropy budgets the head budgets,
// known), 6 threshold found, 7 output places ranked, 8 rows gathered.  In the
// regular build the stamps compile to nothing.
#ifdef KVE_STAMPS
constexpr int kStampItems = 1 << 16;
__device__ unsigned long long kve_stamps[kStampItems][kStampPhases];
#define KVE_STAMP(item, ph)                                                                      \
  do {                                                                                             \
    if (threadIdx.x == 0 && (item) >= 0 && (item) < kStampItems)                                   \
      kve_stamps[(item)][(ph)] = __builtin_amdgcn_s_memrealtime();                                 \
  } while (0)
#else
#define KVE_STAMP(item, ph) \
  do {                      \
  } while (0)
#endif
constexpr int kBK = 64;                           // keys per LDS batch

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Block -> (segment, chunk) so that the chunks of one segment land on the same
// XCD (work-groups are handed to the 8 XCDs round-robin by linear block id):
// they then share that XCD's L2 for the segment's rotated queries.
__device__ __forceinline__ void xcd_item(const ScoreArgs& a, int& s, int& ch) {
  const int L = blockIdx.x;
  const int full = (a.n_seg / 8) * 8;                // segments covered by the XCD-striped part
  if (L < full * a.n_chunks) {
    const int x = L % 8, slot = L / 8;
    s = (slot / a.n_chunks) * 8 + x;
    ch = slot % a.n_chunks;
  } else {
    const int r = L - full * a.n_chunks;
    s = full + r / a.n_chunks;
    ch = r % a.n_chunks;
  }
}

template <int D, int RT>
struct WaveRows {
  static constexpr int KS = D / 32;
  bf16x8 qa[RT][KS];
  int minpos;

  // rpos/qoff: per-row position and row index into the rotated queries (-1: absent), in LDS.
  __device__ __forceinline__ void load(const uint16_t* qr, const int* rpos, const int* qoff, int w, int col,
                                       int quad) {
    minpos = INT_MAX;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int t = w * RT + rt;
      const int qo = qoff[16 * t + col];
      const uint16_t* src = qr + int64_t(qo >= 0 ? qo : 0) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = qo >= 0 ? *reinterpret_cast<const uint4*>(src + ks * 32 + quad * 8) : make_uint4(0, 0, 0, 0);
        qa[rt][ks] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rp = rpos[16 * t + 4 * quad + i];
        if (rp >= 0) minpos = min(minpos, rp);
      }
    }
    minpos = wave_reduce(minpos, [](int x, int y) { return min(x, y); });
  }

  // Logits of key tiles q0, q0+1 of one LDS batch (row stride LS): acc[j][rt] holds
  // rows 16*(w*RT+rt) + 4*quad + i against key (q0+j)*16 + col.  SHIFT: the
  // accumulation starts from shift[rt] (one value per row) instead of 0.
  template <int LS, bool SHIFT>
  __device__ __forceinline__ void logits2(f32x4 (&acc)[2][RT], const uint16_t* kb, int q0, int col, int quad,
                                          const f32x4 (&shift)[RT]) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 bfr[KS];
      const uint16_t* krow = kb + ((q0 + j) * 16 + col) * LS + quad * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bfr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + ks * 32));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 x = SHIFT ? shift[rt] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][ks], bfr[ks], x, 0, 0, 0);
        acc[j][rt] = x;
      }
    }
  }

  // Causal mask for the rare tiles holding keys newer than some row (row positions from LDS).
  __device__ __forceinline__ void mask2(f32x4 (&acc)[2][RT], const int (&kpos)[2], const int* rpos, int w,
                                        int quad) const {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rp = rpos[16 * (w * RT + rt) + 4 * quad + i];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (kpos[j] > rp) acc[j][rt][i] = -kInf;
      }
  }
};

// Pass-1 update of (m, l) with two key tiles of logits; m is kept scaled by c
// (the exp2 argument's units), so the common case needs no multiply.
template <int RT>
__device__ __forceinline__ void stats_update(float (&mc)[RT][4], float (&l)[RT][4], const f32x4 (&acc)[2][RT],
                                             float c) {
  float lsum[RT][4];
  float big = 0.f;                           // the largest sum (one compare instead of one per sum)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = l[rt][i] + fast_exp2(fmaf(acc[0][rt][i], c, -mc[rt][i])) +
                      fast_exp2(fmaf(acc[1][rt][i], c, -mc[rt][i]));
      lsum[rt][i] = v;
      big = __builtin_fmaxf(big, v);
    }
  if (__any(!(big <= kBig))) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // scaling by c > 0 is monotone, so max(m, x0, x1) * c = max(m * c, max(x0, x1) * c)
        const float mn = fmaxf(mc[rt][i], fmaxf(acc[0][rt][i], acc[1][rt][i]) * c);
        lsum[rt][i] = l[rt][i] * fast_exp2(mc[rt][i] - mn) + fast_exp2(fmaf(acc[0][rt][i], c, -mn)) +
                      fast_exp2(fmaf(acc[1][rt][i], c, -mn));
        mc[rt][i] = mn;
      }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) l[rt][i] = lsum[rt][i];
}

// Pass-2: per key of tiles q0, q0+1, the max over this wave's rows of
// c*x - lse (MEAN: the sum of exp2(c*x - lse)), combined over the 4 lane
// groups; written to redw[key].  The logits arrive shifted, acc = x - lse/c
// (the MFMA accumulation starts from -lse/c), so c*x - lse = c*acc, and since
// c > 0 the max over the rows needs one multiply per key instead of one
// multiply-add per row.
template <int RT, bool MEAN>
__device__ __forceinline__ void key_max2(const f32x4 (&acc)[2][RT], float c, float* redw, int q0, int col, int quad) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float best = MEAN ? 0.f : -kInf;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) best = MEAN ? best + fast_exp2(acc[j][rt][i] * c) : fmaxf(best, acc[j][rt][i]);
    best = MEAN ? lanes16_sum(best) : lanes16_max(best);
    best = MEAN ? lanes32_sum(best) : lanes32_max(best);
    if (quad == 0) redw[(q0 + j) * 16 + col] = MEAN ? best : best * c;
  }
}

// Single-read variant (MODE 2): the chunk's two passes run in one work-group.
// Between them the work-groups of a segment exchange their row statistics
// through coherent (agent-scope) atomic stores and loads and meet at a
// per-segment arrival counter; pass 2 then re-reads the chunk it has just read,
// which the memory-side cache still holds, so K crosses HBM once.
//
// Work assignment in that mode: eight ticket queues, queue q holding the chunks
// of the segments s = q (mod 8).  A work-group takes a ticket from the queue of
// the XCD it runs on (a segment's chunks then share one L2) and steals from the
// other queues when its own is empty.  A ticket is only taken by a running
// work-group and each queue hands its tickets out in order, so only the newest
// segment of each queue can miss chunks: at most 8 (nch - 1) work-groups wait
// on work-groups not yet started.  Work-groups start in launch order, spread
// round-robin over the XCDs, and a later one waits while the XCD of the next
// has no free slot; with at most 12 chunks per segment the waiting
// work-groups (at most 88) cannot fill the 96 slots of an XCD (32 CUs, three
// work-groups each), so a full XCD always holds a work-group that will finish,
// and the launches keep to that (or to one round of resident work-groups).
// The wait is bounded all the same (ScoreArgs::spin_limit polls).
constexpr int kMaxWaitChunks = 12;
constexpr int kQueues = 8;
constexpr int kModePass1 = 0, kModePass2 = 1, kModeFused = 2, kModeStep = 3, kModeFill = 4, kModeBudget = 5;

__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & (kQueues - 1);
}

__device__ __forceinline__ void store_stat(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __builtin_bit_cast(unsigned long long, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_stat(const float2* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Segment barrier of the single-read kernels, thread 0 only: count this
// work-group in and poll until all nch work-groups of the segment are in, for
// at most `limit` polls.  Returns false on a timeout (the scheduling above
// rules it out; it would take a device stalled for that long) after pushing
// the counter far below zero, so that no work-group of the segment passes this
// barrier afterwards and each of them reports the segment as failed.
__device__ __forceinline__ bool segment_barrier(int* arrive, int nch, int limit) {
  atomicAdd(arrive, 1);
  int spins = 0;
  while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nch && ++spins < limit)
    __builtin_amdgcn_s_sleep(1);
  if (spins < limit) return true;
  atomicAdd(arrive, -(1 << 24));
  return false;
}

// Ticket from the XCD-local queue, else from any other; -1 when all are empty.
__device__ __forceinline__ int take_ticket(const ScoreArgs& a, int* ctl) {
  const unsigned x = xcc_id();
  for (int k = 0; k < kQueues; ++k) {
    const int q = int((x + k) & (kQueues - 1));
    const int nq = (q < a.n_seg ? (a.n_seg - q + kQueues - 1) / kQueues : 0) * a.n_chunks;
    if (nq == 0) continue;
    // the XCD's own queue is taken from at once (one round trip; a count past
    // nq is harmless); the others are looked at first so that an empty one is
    // not counted up by every work-group that steals
    if (k > 0 && __hip_atomic_load(&ctl[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= nq) continue;
    const int t = atomicAdd(&ctl[q], 1);
    if (t < nq) return (t / a.n_chunks * kQueues + q) * a.n_chunks + t % a.n_chunks;
  }
  return -1;
}

// One-kernel trigger (kv_evict_score_select_compact and its in-place form):
// each work-group scores its chunk with the single-read scheme above, stores
// the chunk's scores with coherent stores and counts itself in at a second
// per-segment arrival counter.  The copying form gathers most of the segment,
// so every work-group waits there, finds the protected top-K threshold over the
// segment's scores (copied to LDS) and gathers its own chunk's kept rows.  The
// in-place form moves at most min(K, n - K) rows, so the last work-group to
// arrive selects and moves them all and the others are done, which frees
// their slots for new chunks.  keys: LDS scratch of step_max_seg(D) words.

// The segment's scores into LDS as order keys (eight loads in flight per
// thread, clamped addresses so that no load waits on a branch) and the
// candidates' smallest and largest key.  With ENT, also the segment's
// normalised score entropy (ReasonAlloc, "Key Concepts"), with the arithmetic
// of entropy_kernel: per score, fp32 s * log2(s) for s > 1e-30, double sums.
// hist: 256 words of LDS.
struct SegKeys {
  uint32_t kmin, kmax;
  float entropy;
};
template <bool ENT>
__device__ __forceinline__ SegKeys segment_keys(const ScoreArgs& a, int64_t off, int n, uint32_t* keys,
                                                uint32_t* hist, int tid) {
  __shared__ double esum[2][4];
  const int P = a.n_prefix, R = a.n_recent;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  double S = 0.0, Q2 = 0.0;
  for (int j0 = 0; j0 < n; j0 += 8 * 256) {
    float raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      raw[u] = __hip_atomic_load(&a.scores[off + min(j0 + u * 256 + tid, n - 1)], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * 256 + tid;
      if (j < n) {
        const uint32_t key = float_order_key(raw[u]);
        keys[j] = key;
        if (j >= P && j < n - R) {
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
        if (ENT) {
          S += double(raw[u]);
          if (raw[u] > 1e-30f) Q2 += double(raw[u] * __builtin_amdgcn_logf(raw[u]));
        }
      }
    }
  }
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (ENT) {
    S = wave_sum_f64(S);
    Q2 = wave_sum_f64(Q2 * 0.69314718055994530942);   // log2 -> ln
  }
  if ((tid & 63) == 0) {
    hist[tid >> 6] = kmin;
    hist[4 + (tid >> 6)] = kmax;
    if (ENT) {
      esum[0][tid >> 6] = S;
      esum[1][tid >> 6] = Q2;
    }
  }
  __syncthreads();
  SegKeys r;
  r.kmin = min(min(hist[0], hist[1]), min(hist[2], hist[3]));
  r.kmax = max(max(hist[4], hist[5]), max(hist[6], hist[7]));
  r.entropy = 0.f;
  if (ENT) {
    const double St = esum[0][0] + esum[0][1] + esum[0][2] + esum[0][3];
    const double Qt = esum[1][0] + esum[1][1] + esum[1][2] + esum[1][3];
    if (n > 1 && St > 0.0) r.entropy = float((log(St) - Qt / St) / log(double(n)));
  }
  __syncthreads();
  return r;
}

// T, the kc-th largest candidate key among the keys in LDS, and kk, the number
// of candidates equal to T that are kept.  hist: 256 words of LDS; sh: 2 words.
__device__ __forceinline__ void segment_radix(const ScoreArgs& a, int n, int kc, const uint32_t* keys,
                                              const SegKeys& sk, uint32_t* hist, uint32_t* sh, int tid,
                                              uint32_t& T, uint32_t& kk) {
  const int P = a.n_prefix, R = a.n_recent;
  // every candidate shares the leading bits of its min and max: the radix digits start below them
  const int known = sk.kmin == sk.kmax ? 32 : __clz(int(sk.kmin ^ sk.kmax));
  radix_threshold_v<256>(
      [&](const auto& f) {
        for (int j = P + tid; j < n - R; j += 256) f(keys[j]);
      },
      kc, hist, sh, T, kk, sk.kmin, known);
}

__device__ __forceinline__ void segment_threshold(const ScoreArgs& a, int64_t off, int n, int kc, uint32_t* keys,
                                                  uint32_t* hist, uint32_t* sh, int tid, uint32_t& T, uint32_t& kk) {
  const SegKeys sk = segment_keys<false>(a, off, n, keys, hist, tid);
  segment_radix(a, n, kc, keys, sk, hist, sh, tid, T, kk);
}

// Copying form: every work-group of the segment finds the threshold for
// budget K and gathers its own chunk's kept rows to their places in the output
// segment, in ascending slot order (the kept slots and threshold ties before
// the chunk give its first output row).  `loaded`: the segment's keys are
// already in LDS (else they are loaded here).  Returns keep_n (-1 for a
// rejected segment).
template <int D>
__device__ __forceinline__ int step_select_compact(const ScoreArgs& a, int s, int64_t off, int n, int k0, int k1,
                                                   int K, uint32_t* keys, const SegKeys* loaded, int tid, int item) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot[4];
  __shared__ int mine[kMfmaChunk];           // kept slots of the piece being gathered, ascending
  const int64_t oo = a.out_off[s];
  const int P = a.n_prefix, R = a.n_recent;
  const bool out_ok = oo >= 0 && oo + a.out_cap <= a.out_rows;
  const bool bud_ok = K >= n || (K >= P + R && K >= 0);
  const int keep_n = K >= n ? n : K;
  if (!out_ok || !bud_ok || keep_n > a.out_cap || n > step_max_seg(D))
    return -1;                               // the segment keeps the failure mark stored after the first barrier
  // The chunk's kept slots are listed in `mine` (256 slots ranked per round)
  // and gathered whenever the next round could overflow it, so every gather
  // but the last moves at least kMfmaChunk - 255 rows however sparse the kept
  // slots are (whole segments of up to step_max_seg keys with small per-head
  // budgets in the entropy-budget kernel), which keeps its loads in flight.
  int base = 0;                              // output row of the next kept slot
  bool first = true;
  auto gather_piece = [&](int cnt) {         // mine[0, cnt) -> output rows base .. base + cnt - 1
    __syncthreads();
    if (first) KVE_STAMP(item, 7);
    first = false;
    const int64_t dst0 = oo + base;
    gather_rows<CPR>([&](int r) { return mine[r]; }, [&](int r) { return dst0 + r; }, cnt, a.k, a.v, a.pos, off,
                     a.k_out, a.v_out, a.pos_out, a.kept, tid, n, oo, oo + a.out_cap);
    base += cnt;
    __syncthreads();                         // the next piece rewrites mine
  };
  if (K >= n) {
    base = k0;
    for (int p0 = k0; p0 < k1; p0 += kMfmaChunk) {
      const int p1 = min(k1, p0 + kMfmaChunk);
      for (int j = p0 + tid; j < p1; j += 256) mine[j - p0] = j;
      gather_piece(p1 - p0);
    }
  } else {
    uint32_t T, kk;
    if (loaded) segment_radix(a, n, K - P - R, keys, *loaded, hist, sh, tid, T, kk);
    else segment_threshold(a, off, n, K - P - R, keys, hist, sh, tid, T, kk);
    KVE_STAMP(item, 6);
    // kept slots and threshold ties before this chunk
    int eq_b = 0, gt_b = 0;
    for (int j = P + tid; j < min(k0, n - R); j += 256) {
      eq_b += keys[j] == T;
      gt_b += keys[j] > T;
    }
    eq_b = kk != 0u ? block_sum<256>(eq_b, wtot) : 0;   // kk == 0: no threshold tie is kept
    gt_b = block_sum<256>(gt_b, wtot);
    const int prot_b = min(k0, P) + max(0, k0 - (n - R));
    base = prot_b + gt_b + min(eq_b, int(kk));
    int eq_seen = eq_b;
    int cnt = 0;                             // kept slots listed in `mine` and not yet gathered
    for (int j0 = k0; j0 < k1; j0 += 256) {
      if (cnt > kMfmaChunk - 256) {          // a round lists at most 256 more: gather the list first
        gather_piece(cnt);
        cnt = 0;
      }
      const int j = j0 + tid;
      const bool in = j < k1;
      const bool cand = in && j >= P && j < n - R;
      const uint32_t key = cand ? keys[j] : 0u;
      const bool eq = cand && key == T;
      int eq_tot = 0, eq_rank = 0;
      if (kk != 0u) eq_rank = eq_seen + block_flag_scan<256>(eq, wtot, eq_tot);
      const bool keep = in && (!cand || key > T || (eq && uint32_t(eq_rank) < kk));
      int keep_tot;
      const int at = cnt + block_flag_scan<256>(keep, wtot, keep_tot);
      if (keep && KVE_CHECK(at < kMfmaChunk, 7)) mine[at] = j;
      cnt += keep_tot;
      eq_seen += eq_tot;
    }
    gather_piece(cnt);
  }
  return keep_n;
}

// In-place form (kv_evict_score_select_compact_inplace): the same threshold,
// then hole filling within the cache: the survivors in [K, n), in ascending
// slot order, move into the evicted slots of [0, K), in ascending slot order.
// One pass over the slots (8 consecutive per thread and round, two block
// scans) replaces each key in LDS by (kept << 31) | (kept slots before it); a
// mover's rank is then its kept-before count minus that of slot K, and a
// hole's rank its slot minus its kept-before count, so each piece of at most
// 1024 slots of [K, n) finds the holes that pair with its movers by a plain
// sweep.  Sources lie in [K, n) and destinations in [0, K), so no row is
// overwritten before it is read.  Returns the segment's new length (-1 for a
// rejected segment).
template <int D>
__device__ __forceinline__ int step_select_fill(const ScoreArgs& a, int s, int64_t off, int n, uint32_t* keys,
                                                int tid) {
  constexpr int CPR = D / 8;
  constexpr int kPiece = 1024;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  __shared__ int wtot[4];
  __shared__ uint16_t hole_at[kPiece], mover_at[kPiece];   // slots < step_max_seg fit in 16 bits
  const int K = a.budget ? a.budget[s] : a.uniform_budget;
  const int P = a.n_prefix, R = a.n_recent;
  if (K >= n) return n;                      // every row stays where it is
  if (K < P + R || K < 0 || n > step_max_seg(D)) return -1;
  uint32_t T, kk;
  segment_threshold(a, off, n, K - P - R, keys, hist, sh, tid, T, kk);
  // keys -> (kept << 31) | kept slots before
  int kept_seen = 0, eq_seen = 0;
  for (int j0 = 0; j0 < n; j0 += 8 * 256) {
    const int jt = j0 + 8 * tid;
    uint32_t kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = jt + u < n ? keys[jt + u] : 0u;
    int n_eq = 0, n_sure = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= P && j < n - R;
      n_eq += cand && kv[u] == T;
      n_sure += j < n && (!cand || kv[u] > T);
    }
    int eq_tot;
    const int eq_before = eq_seen + block_scan<256>(n_eq, wtot, eq_tot);
    const int n_keep = n_sure + min(n_eq, max(0, int(kk) - eq_before));
    int keep_tot;
    int before = kept_seen + block_scan<256>(n_keep, wtot, keep_tot);
    int eq_rank = eq_before;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jt + u;
      const bool cand = j >= P && j < n - R;
      const bool eq = cand && kv[u] == T;
      const bool keep = j < n && (!cand || kv[u] > T || (eq && eq_rank < int(kk)));
      eq_rank += eq;
      if (j < n) keys[j] = (keep ? 0x80000000u : 0u) | uint32_t(before);
      before += keep;
    }
    kept_seen += keep_tot;
    eq_seen += eq_tot;
    __syncthreads();
  }
  const int base_k = int(keys[K] & 0x7fffffffu);           // kept slots before K (K < n)
  for (int p0 = K; p0 < n; p0 += kPiece) {
    const int p1 = min(n, p0 + kPiece);
    const int r_lo = int(keys[p0] & 0x7fffffffu) - base_k;  // ranks of this piece's movers among all movers
    const int r_hi = (p1 < n ? int(keys[p1] & 0x7fffffffu) : K) - base_k;
    const int cnt = r_hi - r_lo;
    if (cnt <= 0) continue;                                // the same decision in every thread
    for (int j = p0 + tid; j < p1; j += 256) {
      const uint32_t e = keys[j];
      if (e >> 31) {
        const int m = int(e & 0x7fffffffu) - base_k - r_lo;
        if (KVE_CHECK(m >= 0 && m < cnt, 6)) mover_at[m] = uint16_t(j);
      }
    }
    for (int h = tid; h < K; h += 256) {                   // holes: evicted slots below K
      const uint32_t e = keys[h];
      const int rank = h - int(e & 0x7fffffffu);
      if (!(e >> 31) && rank >= r_lo && rank < r_hi && KVE_CHECK(rank - r_lo < kPiece, 6))
        hole_at[rank - r_lo] = uint16_t(h);
    }
    __syncthreads();
    gather_rows<CPR>([&](int r) { return int(mover_at[r]); }, [&](int r) { return off + hole_at[r]; }, cnt, a.k,
                     a.v, a.pos, off, a.k_out, a.v_out, a.pos_out, nullptr, tid, n, off, off + K);
    __syncthreads();                         // the next piece rebuilds the lists
  }
  return K;
}

// One-kernel trigger with ReasonAlloc's entropy budgets
// (kv_evict_score_budget_select_compact).  Every (segment, chunk) is two
// tickets of one queue: a scoring ticket (both passes; chunk 0 then publishes
// the segment's score entropy and counts its head in at the request-layer's
// arrival counter) and a selection ticket (wait until the request-layer's
// n_kv heads are in, solve the head budgets with the budget kernel's wave
// solver, select with the own head's budget, gather the chunk's kept rows).
// A request-layer's selection tickets come kSelectLag tickets after its
// scoring tickets (four rounds of resident work-groups), so by the time one
// is taken its heads have been scored: no work-group sits idle waiting for the
// slowest head of its request-layer while it holds a slot.  (A lag of one
// round left selections waiting; the 32-layer, 2560-head launch gains little
// beyond two.)
// Progress: a scoring work-group waits only at its segment barrier, for chunks
// of its own segment (consecutive tickets: only the newest segment can miss
// one, a segment takes one or two chunks); a selection ticket is only handed
// out after every scoring ticket of its request-layer, all taken by running
// work-groups that wait on nothing else.  The waits are bounded all the same.
constexpr int kNoBudget = INT_MIN;
constexpr int kSelectLag = 4 * 3 * 256;

// Ticket t of the entropy-budget trigger -> (segment * n_chunks + chunk) and
// whether it is a selection ticket.  With U = n_kv * n_chunks tickets per
// request-layer and D request-layers of lag: scoring tickets of request-layers
// 0..D-1; then pairs (scoring of request-layer D + p, selection of p); then the
// selection tickets of the last D request-layers.
__device__ __forceinline__ int budget_ticket(const ScoreArgs& a, int t, bool& select) {
  const int U = a.n_kv * a.n_chunks, G = a.n_seg / a.n_kv;
  const int D = min(G, (kSelectLag + U - 1) / U);
  select = false;
  if (t < D * U) return t;
  const int u = t - D * U;
  if (u < 2 * (G - D) * U) {
    const int p = u / (2 * U), r = u % (2 * U);
    select = r >= U;
    return select ? p * U + (r - U) : (D + p) * U + r;
  }
  select = true;
  return (G - D) * U + (u - 2 * (G - D) * U);
}

// Thread 0 of chunk 0's work-group: publish the segment's entropy and count
// the head in.
__device__ __forceinline__ void group_arrive(const ScoreArgs& a, int* ctl, int s, float e) {
  __hip_atomic_store(&a.entropy[s], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  atomicAdd(ctl + kQueues + 3 * a.n_seg + s / a.n_kv, 1);
}

// Every thread of a selection work-group of segment s: the head's budget, or
// kNoBudget when the heads did not all arrive within the poll bound or the
// floors exceed the request-layer's total (the segment then keeps -1).
__device__ __forceinline__ int group_budget(const ScoreArgs& a, int* ctl, int s, int ch, int tid) {
  __shared__ HeadBudgetLds L;
  __shared__ int met, kb;                      // two words: kb is written while others may still read met
  const int H = a.n_kv, grp = s / H;
  int* cnt = ctl + kQueues + 3 * a.n_seg + grp;
  if (tid == 0) {
    int spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < H && ++spins < a.spin_limit)
      __builtin_amdgcn_s_sleep(1);
    met = spins < a.spin_limit;
    if (!met) atomicAdd(cnt, -(1 << 24));
  }
  __syncthreads();
  if (!met) return kNoBudget;
  if (tid < kWave) {
    const bool act = tid < H;
    const int hs = grp * H + tid;
    const float eh = act ? __hip_atomic_load(&a.entropy[hs], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
    int cap = 0;
    if (act) {
      const int nl = a.seg_len[hs];
      cap = nl >= 0 && nl <= a.max_seg_len ? nl : 0;
    }
    const int32_t b = head_budget_wave(double(eh), a.ent_form, cap, double(a.layer_total[grp]), a.min_per_head, H, L);
    if (tid == s - grp * H) {
      if (ch == 0 && a.budget_out) a.budget_out[s] = b;   // -1: the floors exceed the total
      kb = b < 0 ? kNoBudget : b;
    }
  }
  __syncthreads();
  return kb;
}

// The work-group item (ticket) of segment s, chunk ch, for the phase stamps
// (recomputed where it is stamped, so no register holds it in between).
__device__ __forceinline__ int stamp_item(const ScoreArgs& a, int s, int ch) { return s * a.n_chunks + ch; }

// Selection ticket of the entropy-budget trigger for (segment s, chunk ch):
// wait for the request-layer's heads, solve the head budgets (chunk 0 writes
// the head's), then select over the segment's stored scores and gather the
// chunk's kept rows; the last chunk to finish publishes the length.  A segment
// with nothing to gather (rejected or empty) only has its budget written; its
// length was written by its scoring ticket.  keys: step_max_seg(D) words of LDS.
template <int D>
__device__ __forceinline__ void budget_select(const ScoreArgs& a, int* ctl, int s, int ch, uint32_t* keys, int tid) {
  int64_t off;
  int n;
  const bool ok = segment_ok(a, s, off, n);
  const int k0 = ch * a.chunk;
  const bool gather = ok && k0 < n;
  if (!gather && ch != 0) return;
  const int K = group_budget(a, ctl, s, ch, tid);
  if (!gather || K == kNoBudget) return;
  KVE_STAMP(stamp_item(a, s, ch), 5);
  const int k1 = min(n, k0 + a.chunk), nch = (n + a.chunk - 1) / a.chunk;
  const int keep_n = step_select_compact<D>(a, s, off, n, k0, k1, K, keys, nullptr, tid, stamp_item(a, s, ch));
  if (keep_n < 0) return;
  KVE_STAMP(stamp_item(a, s, ch), 8);
  // the last work-group to count itself out publishes the segment's length
  // (no wait for the gather's stores: the length is read only after the
  // kernel, and a work-group that gets here has passed every meeting)
  if (tid == 0 && atomicAdd(ctl + kQueues + 2 * a.n_seg + s, 1) == nch - 1)
    __hip_atomic_store(&a.out_len[s], keep_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int RT, int MODE>
__device__ __forceinline__ void score_mfma_body(const ScoreArgs& a, int* ctl) {
  // Padded LDS row (bf16 elements).  A 16-byte fragment read of the MFMA B
  // operand has lane (col, quad) read row col at byte 16 * quad; with rows of
  // D + 16 elements (288 bytes at D = 128) the reads of a wave hit distinct
  // banks, while D + 8 (272 bytes) costs four conflict cycles per read on gfx950.
  constexpr int LS = D + 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int KPU = 256 / CPR;             // keys covered by one 16-byte load per thread
  constexpr int CPT = kBK / KPU;             // loads per thread per batch
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kBK * LS];
  static_assert(sizeof(kt) == 4 * step_max_seg(D), "selection keys reuse the key tiles");
  __shared__ int kps[2][kBK];
  __shared__ float red[2][4][kBK];
  __shared__ float lse_s[kMaxObsRows];
  __shared__ int rpos_s[kMaxObsRows];
  __shared__ int qoff_s[kMaxObsRows];
  __shared__ int sh_item;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  int s, ch;
  int item = -1;                             // the ticket (one-call kernels), for the phase stamps
  if (MODE >= kModeFused) {
    if (tid == 0) {
      if (MODE == kModeBudget) {               // one queue: scoring and (lagging) selection tickets
        const int t = atomicAdd(&ctl[0], 1);
        sh_item = t < 2 * a.n_seg * a.n_chunks ? t : -1;
      } else {
        sh_item = take_ticket(a, ctl);
      }
    }
    __syncthreads();
    item = sh_item;
    if (item < 0) return;
    if (MODE == kModeBudget) {
      bool select;
      item = budget_ticket(a, item, select);
      if (select) {
        budget_select<D>(a, ctl, item / a.n_chunks, item % a.n_chunks, reinterpret_cast<uint32_t*>(&kt[0][0]), tid);
        return;
      }
    }
    s = item / a.n_chunks;
    ch = item % a.n_chunks;
    KVE_STAMP(stamp_item(a, s, ch), 0);
  } else {
    xcd_item(a, s, ch);
  }
  int64_t off;
  int n;
  // a segment with nothing to score still takes part in its request-layer's
  // budgets (entropy 0, its cap is its length) and gets its budget written
  if (!segment_ok(a, s, off, n)) {
    if (MODE >= kModeStep && ch == 0 && tid == 0) a.out_len[s] = -1;
    if (MODE == kModeBudget && ch == 0 && tid == 0) group_arrive(a, ctl, s, 0.f);
    return;
  }
  const int k0 = ch * a.chunk;
  if (k0 >= n) {
    if (MODE >= kModeStep && ch == 0 && tid == 0) a.out_len[s] = 0;   // empty segment
    if (MODE == kModeBudget && ch == 0 && tid == 0) group_arrive(a, ctl, s, 0.f);
    return;
  }
  const int k1 = min(n, k0 + a.chunk);
  const int nch = (n + a.chunk - 1) / a.chunk;
  const int b = s / a.n_kv, g = s % a.n_kv;
  const float c = kLog2e / sqrtf(float(D));
  const bool mean = a.aggregate != 0;
  const float inv_live = live_row_inverse(a, b);

  // per-row metadata, once per work-group
  for (int r = tid; r < 16 * 4 * RT; r += 256) {
    const int rp = row_position(a, b, r);
    rpos_s[r] = rp;
    qoff_s[r] = rp >= 0 ? int(row_qr_index(a, b, g, r)) : -1;
    if (MODE == kModePass2) lse_s[r] = rp >= 0 ? a.lse[int64_t(s) * a.rows + r] : kInf;
  }
  __syncthreads();
  WaveRows<D, RT> rows;
  rows.load(static_cast<const uint16_t*>(a.qr), rpos_s, qoff_s, w, col, quad);
  float st0[RT][4], st1[RT][4];   // pass 1: (m * c, l); pass 2: st0 = lse (log2 units)
  f32x4 shift[RT];                // pass 2: -lse / c, where the rows' MFMA accumulation starts
  auto set_shift = [&]() {
    const float ninv = -1.f / c;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) shift[rt][i] = st0[rt][i] * ninv;
  };
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st0[rt][i] = MODE == kModePass2 ? lse_s[16 * (w * RT + rt) + 4 * quad + i] : kNegBig;
      st1[rt][i] = 0.f;
    }

  const int span = k1 - k0;

  // One sweep over the chunk: pass 1 updates (st0, st1); pass 2 writes scores.
  auto sweep = [&](auto pass2_tag) {
    constexpr bool P2 = decltype(pass2_tag)::value;
    // Pass 2 forms its per-thread addresses from an opaque copy of the thread
    // index: the compiler then computes them after pass 1 instead of keeping
    // pass 1's copies in registers (spilled) across pass 1's loop.
    int t = tid;
    if constexpr (P2) asm volatile("" : "+v"(t));
    // thread's share of a batch: keys key0 + u*KPU (u < CPT), 16-byte chunk `part`
    const int key0 = t / CPR, part = t % CPR;
    const uint16_t* gk = static_cast<const uint16_t*>(a.k) + (off + k0 + key0) * D + part * 8;
    uint4 pre[CPT];
    int prepos = INT_MAX;
    // the batch's loads go out at the top wave priority, so that a wave
    // issuing them is not held behind the exp2 and MFMA streams of the other
    // work-groups on its SIMD (36-layer step about 1.5 % shorter)
    auto load_batch = [&](int kb) {        // kb: batch start relative to k0
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const bool ok = k0 + kb + key0 + u * KPU < k1;
        pre[u] = ok ? *reinterpret_cast<const uint4*>(gk + int64_t(kb + u * KPU) * D) : make_uint4(0, 0, 0, 0);
      }
      if (t < kBK) prepos = (k0 + kb + t < k1) ? a.pos[off + k0 + kb + t] : INT_MAX;
      __builtin_amdgcn_s_setprio(0);
    };
    auto store_batch = [&](int buf) {
#pragma unroll
      for (int u = 0; u < CPT; ++u) *reinterpret_cast<uint4*>(&kt[buf][(key0 + u * KPU) * LS + part * 8]) = pre[u];
      if (t < kBK) kps[buf][t] = prepos;
    };
    auto finish_keys = [&](int bi, int kb) {  // per-key max (sum) over the 4 waves -> score
      const int j = k0 + kb + t;
      if (t < kBK && j < k1) {
        const float sc =
            mean ? (red[bi][0][t] + red[bi][1][t] + red[bi][2][t] + red[bi][3][t]) * inv_live
                 : fast_exp2(fmaxf(fmaxf(red[bi][0][t], red[bi][1][t]), fmaxf(red[bi][2][t], red[bi][3][t])));
        if (MODE >= kModeStep)   // read back by the segment's other work-groups: coherent store
          __hip_atomic_store(&a.scores[off + j], sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          a.scores[off + j] = sc;
      }
    };
    // pass 2 walks the chunk backwards: its first batches are the ones pass 1
    // read last (the likeliest still in L2), and it ends where the gather of the
    // kept rows begins
    const int ntl = (span + kBK - 1) / kBK;
    auto kb_at = [&](int it) { return P2 ? (ntl - 1 - it) * kBK : it * kBK; };
    load_batch(kb_at(0));
    store_batch(0);
    if (ntl > 1) load_batch(kb_at(1));
    __syncthreads();
    int cur = 0;
    for (int it = 0; it < ntl; ++it) {
      int kpos[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) kpos[q4] = kps[cur][q4 * 16 + col];
      const bool late = kpos[0] > rows.minpos || kpos[1] > rows.minpos || kpos[2] > rows.minpos ||
                        kpos[3] > rows.minpos;
      const bool any_late = __any(late);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc[2][RT];
        rows.template logits2<LS, P2>(acc, kt[cur], 2 * h, col, quad, shift);
        if (any_late) {
          const int kp2[2] = {kpos[2 * h], kpos[2 * h + 1]};
          rows.mask2(acc, kp2, rpos_s, w, quad);
        }
        if (!P2) stats_update<RT>(st0, st1, acc, c);
        else if (mean) key_max2<RT, true>(acc, c, red[cur][w], 2 * h, col, quad);
        else key_max2<RT, false>(acc, c, red[cur][w], 2 * h, col, quad);
      }
      if (it + 1 < ntl) store_batch(cur ^ 1);
      if (it + 2 < ntl) load_batch(kb_at(it + 2));
      if (P2 && it > 0) finish_keys(cur ^ 1, kb_at(it - 1));
      __syncthreads();
      cur ^= 1;
    }
    if (P2) finish_keys(cur ^ 1, kb_at(ntl - 1));
  };

  if (MODE == kModePass2) {
    set_shift();
    sweep(std::integral_constant<bool, true>{});
    return;
  }
  sweep(std::integral_constant<bool, false>{});
  // combine the 16 key columns held by each lane group, then publish
  float2* stats_seg = a.stats + int64_t(s) * a.n_chunks * a.rows;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (m, l) pairs merged over the row's 16 lanes; the pair travels as one
      // 64-bit lane value
      const float2 ml = row16_reduce(make_float2(st0[rt][i], st1[rt][i]), [](float2 x, float2 y) {
        const float M = fmaxf(x.x, y.x);
        return make_float2(M, x.y * fast_exp2(x.x - M) + y.y * fast_exp2(y.x - M));
      });
      const float mm = ml.x, ll = ml.y;
      const int r = 16 * (w * RT + rt) + 4 * quad + i;
      if (col == 0 && r < a.rows) {
        if (MODE >= kModeFused) store_stat(&stats_seg[int64_t(ch) * a.rows + r], make_float2(mm, ll));
        else stats_seg[int64_t(ch) * a.rows + r] = make_float2(mm, ll);
      }
    }
  if (MODE < kModeFused) return;

  // segment barrier: the stores above are acknowledged before the arrival count
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  KVE_STAMP(stamp_item(a, s, ch), 1);
  if (tid == 0) sh_item = segment_barrier(ctl + kQueues + s, nch, a.spin_limit) ? 0 : -1;
  __syncthreads();
  KVE_STAMP(stamp_item(a, s, ch), 2);
  // Every work-group of the segment has read the segment's length by now (the
  // output length may be the input length array): the segment counts as failed
  // until its last work-group has moved its rows.  Both this store and the
  // final one are device-coherent: the segment's work-groups may run on
  // different XCDs, whose L2 caches would otherwise write their copies of the
  // line back in any order at the end of the kernel.
  if (MODE >= kModeStep && ch == 0 && tid == 0)
    __hip_atomic_store(&a.out_len[s], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (sh_item < 0) {                       // the segment's work-groups did not meet: it stays failed
    if (MODE < kModeStep)
      for (int j = k0 + tid; j < k1; j += 256) a.scores[off + j] = __builtin_nanf("");
    return;
  }
  for (int r = tid; r < 16 * 4 * RT; r += 256) {
    float lse = kInf;
    if (r < a.rows && rpos_s[r] >= 0) {
      float M = kNegBig, L = 0.f;
      for (int q0 = 0; q0 < nch; q0 += 8) {          // 8 independent loads in flight per pass
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = q0 + u < nch ? load_stat(&stats_seg[int64_t(q0 + u) * a.rows + r]) : make_float2(kNegBig, 0.f);
        float Mn = M;
#pragma unroll
        for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, v[u].x);
        L *= fast_exp2(M - Mn);
#pragma unroll
        for (int u = 0; u < 8; ++u) L += v[u].y * fast_exp2(v[u].x - Mn);
        M = Mn;
      }
      lse = L > 0.f ? M + log2f(L) : kInf;
    }
    lse_s[r] = lse;
  }
  __syncthreads();
  KVE_STAMP(stamp_item(a, s, ch), 3);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) st0[rt][i] = lse_s[16 * (w * RT + rt) + 4 * quad + i];
  set_shift();
  sweep(std::integral_constant<bool, true>{});
  KVE_STAMP(stamp_item(a, s, ch), 4);
  if (MODE < kModeStep) return;

  // Every chunk's scores are stored (acknowledged before the arrival count).
  // A work-group that gave up at the first barrier never arrives, so a failed
  // segment is never selected and keeps -1.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* keys = reinterpret_cast<uint32_t*>(&kt[0][0]);
  int keep_n;
  if constexpr (MODE == kModeFill) {
    // in place: the last work-group to arrive selects and moves the segment's
    // few survivors past K; the others are done
    if (tid == 0) sh_item = atomicAdd(ctl + kQueues + a.n_seg + s, 1) == nch - 1 ? 0 : -1;
    __syncthreads();
    if (sh_item < 0) return;
    keep_n = step_select_fill<D>(a, s, off, n, keys, tid);
    if (keep_n < 0) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&a.out_len[s], keep_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // copying: the kept rows are most of the segment, so every work-group
    // waits for the others, selects and gathers its own chunk's kept rows
    if (tid == 0) sh_item = segment_barrier(ctl + kQueues + a.n_seg + s, nch, a.spin_limit) ? 0 : -1;
    __syncthreads();
    if (sh_item < 0) return;
    if constexpr (MODE == kModeBudget) {
      // every chunk's scores are stored: chunk 0 publishes the segment's
      // entropy and counts the head in; the selection has a ticket of its own
      if (ch == 0) {
        const SegKeys sk = segment_keys<true>(a, off, n, keys, reinterpret_cast<uint32_t*>(&red[0][0][0]), tid);
        if (tid == 0) group_arrive(a, ctl, s, sk.entropy);
      }
      return;
    }
    const int K = a.budget ? a.budget[s] : a.uniform_budget;
    KVE_STAMP(stamp_item(a, s, ch), 5);
    keep_n = step_select_compact<D>(a, s, off, n, k0, k1, K, keys, nullptr, tid, stamp_item(a, s, ch));
    if (keep_n < 0) return;
    KVE_STAMP(stamp_item(a, s, ch), 8);
    // the last work-group to count itself out publishes the segment's length
    // (no wait for the gather's stores: the length is read only after the
    // kernel, and a work-group that gets here has passed both barriers)
    if (tid == 0 && atomicAdd(ctl + kQueues + 2 * a.n_seg + s, 1) == nch - 1)
      __hip_atomic_store(&a.out_len[s], keep_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Pass 1 and the single-read kernel carry the row statistics in registers.
// Up to 192 observation rows (three 16-row tiles per wave) every form fits
// 3 waves per SIMD without spilling; four tiles per wave (up to 256 rows) need
// more registers and run at 2 waves per SIMD.
template <int RT>
constexpr int kScoreWaves = RT <= 3 ? 3 : 2;
template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_pass1_kernel(ScoreArgs a) {
  score_mfma_body<D, RT, kModePass1>(a, nullptr);
}
template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_pass2_kernel(ScoreArgs a) {
  score_mfma_body<D, RT, kModePass2>(a, nullptr);
}
template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_fused_kernel(ScoreArgs a,
                                                                                                    int* ctl) {
  score_mfma_body<D, RT, kModeFused>(a, ctl);
}

template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_step_kernel(ScoreArgs a,
                                                                                                   int* ctl) {
  score_mfma_body<D, RT, kModeStep>(a, ctl);
}
template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_budget_kernel(ScoreArgs a,
                                                                                                     int* ctl) {
  score_mfma_body<D, RT, kModeBudget>(a, ctl);
}
template <int D, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kScoreWaves<RT>, 8))) void score_fill_kernel(ScoreArgs a,
                                                                                                   int* ctl) {
  score_mfma_body<D, RT, kModeFill>(a, ctl);
}

// ------------------------------------------------------------ entropy
// E = (ln S - sum(s ln s) / S) / ln n over one segment's scores: each term
// s log2 s in fp32 (the hardware log2, about one ulp; scores under 1e-30 are
// left out), the sums in double, four loads in flight per thread.
__global__ __launch_bounds__(256) void entropy_kernel(ScoreArgs a) {
  __shared__ double part[2][4];
  const int s = blockIdx.x;
  int64_t off;
  int n;
  if (!segment_ok(a, s, off, n)) return;
  double S = 0.0, Q2 = 0.0;
  const float* sc = a.scores + off;
  for (int j0 = 0; j0 < n; j0 += 4 * 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = sc[min(j0 + u * 256 + int(threadIdx.x), n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + u * 256 + int(threadIdx.x) < n) {
        S += double(v[u]);
        // terms below 1e-30 (and the denormals the hardware log2 does not take) add under 1e-28 each
        if (v[u] > 1e-30f) Q2 += double(v[u] * __builtin_amdgcn_logf(v[u]));
      }
  }
  double Q = Q2 * 0.69314718055994530942;    // log2 -> ln
  S = wave_sum_f64(S);
  Q = wave_sum_f64(Q);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    part[0][w] = S;
    part[1][w] = Q;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    S = part[0][0] + part[0][1] + part[0][2] + part[0][3];
    Q = part[1][0] + part[1][1] + part[1][2] + part[1][3];
    double E = 0.0;
    if (n > 1 && S > 0.0) E = (log(S) - Q / S) / log(double(n));
    a.entropy[s] = float(E);
  }
}

void launch_merge(const ScoreArgs& a, hipStream_t st) {
  const int64_t n = int64_t(a.n_seg) * a.rows;
  hipLaunchKernelGGL(merge_lse_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a);
}

template <int D, int RT>
hipError_t launch_mfma(const ScoreArgs& a, dim3, hipStream_t st) {
  const dim3 grid1(unsigned(int64_t(a.n_seg) * a.n_chunks));
  hipLaunchKernelGGL((score_pass1_kernel<D, RT>), grid1, dim3(256), 0, st, a);
  launch_merge(a, st);
  hipLaunchKernelGGL((score_pass2_kernel<D, RT>), grid1, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma_rt(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  const int tiles = (a.rows + 15) / 16;
  const int rt = (tiles + 3) / 4;
  switch (rt) {
    case 1: return launch_mfma<D, 1>(a, grid, st);
    case 2: return launch_mfma<D, 2>(a, grid, st);
    case 3: return launch_mfma<D, 3>(a, grid, st);
    default: return launch_mfma<D, 4>(a, grid, st);
  }
}

// The control ints (tickets, arrival counters) were cleared by the query rotation.
template <int D, int RT>
hipError_t launch_fused_t(const ScoreArgs& a, int* ctl, hipStream_t st) {
  const unsigned items = unsigned(int64_t(a.n_seg) * a.n_chunks);
  hipLaunchKernelGGL((score_fused_kernel<D, RT>), dim3(items), dim3(256), 0, st, a, ctl);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fused(const ScoreArgs& a, int* ctl, hipStream_t st) {
  const int rt = ((a.rows + 15) / 16 + 3) / 4;
  switch (rt) {
    case 1: return launch_fused_t<D, 1>(a, ctl, st);
    case 2: return launch_fused_t<D, 2>(a, ctl, st);
    case 3: return launch_fused_t<D, 3>(a, ctl, st);
    default: return launch_fused_t<D, 4>(a, ctl, st);
  }
}

template <int D, int RT>
hipError_t launch_step_t(const ScoreArgs& a, int* ctl, hipStream_t st) {
  const unsigned items = unsigned(int64_t(a.n_seg) * a.n_chunks);
  if (a.layer_total)   // a scoring and a selection ticket per item
    hipLaunchKernelGGL((score_budget_kernel<D, RT>), dim3(2 * items), dim3(256), 0, st, a, ctl);
  else if (a.inplace)
    hipLaunchKernelGGL((score_fill_kernel<D, RT>), dim3(items), dim3(256), 0, st, a, ctl);
  else
    hipLaunchKernelGGL((score_step_kernel<D, RT>), dim3(items), dim3(256), 0, st, a, ctl);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  const size_t sh = size_t(a.rows) * D * sizeof(T) + size_t(a.rows) * (4 * sizeof(float2) + sizeof(float) + sizeof(int));
  hipLaunchKernelGGL((score_valu_kernel<T, D, false>), grid, dim3(256), sh, st, a);
  launch_merge(a, st);
  hipLaunchKernelGGL((score_valu_kernel<T, D, true>), grid, dim3(256), sh, st, a);
  return hipGetLastError();
}

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Keys per MFMA work-group of the two scoring passes: the multiple of 64 in
// [256, 8192] with the shortest expected launch, counted as rounds of
// resident work-groups (three per CU) times the keys a work-group scores plus
// a fixed cost of about 96 keys' worth (query load, statistics); ties go to
// the length nearest 1024.  This keeps the last round of a launch from
// running mostly empty (65,536-key segments, 32 of them: 2752 keys, one full
// round, instead of 1024 keys, 2.7 rounds).
int mfma_chunk(int n_seg, int max_seg_len) {
  constexpr int64_t kResident = 3 * 256, kOverhead = 96;
  int best = kMfmaChunk;
  int64_t best_cost = INT64_MAX;
  for (int c = 256; c <= 8192; c += 64) {
    const int64_t wgs = int64_t(n_seg) * ((max_seg_len + c - 1) / c);
    const int64_t cost = (wgs + kResident - 1) / kResident * (c + kOverhead);
    if (cost < best_cost || (cost == best_cost && std::abs(c - kMfmaChunk) < std::abs(best - kMfmaChunk))) {
      best = c;
      best_cost = cost;
    }
  }
  return best;
}

// The single-read scoring kernel: the two-pass chunk, lengthened (in 64-key
// steps) where a segment would otherwise span more than kMaxWaitChunks chunks.
int fused_chunk(int n_seg, int max_seg_len) {
  const int c = mfma_chunk(n_seg, max_seg_len);
  const int lo = (max_seg_len + kMaxWaitChunks - 1) / kMaxWaitChunks;
  return c >= lo ? c : (lo + kBK - 1) / kBK * kBK;
}

// The one-kernel trigger: every work-group of a segment also selects over the
// whole segment and waits at two barriers, so more, shorter work-groups only
// pay off while they still fit in one round of resident work-groups (three
// per CU): 1024 keys, halved (down to 256) while the halved launch still fits.
int step_chunk(int n_seg, int max_seg_len) {
  static_assert((step_max_seg(128) + kMfmaChunk - 1) / kMfmaChunk <= kMaxWaitChunks, "segment spans too many chunks");
  constexpr int64_t kResident = 3 * 256;
  int c = kMfmaChunk;
  while (c > 256 && int64_t(n_seg) * ((max_seg_len + c / 2 - 1) / (c / 2)) <= kResident) c >>= 1;
  return c;
}

// The in-place trigger: only the segment's last work-group selects, so a
// whole segment per work-group (no barrier waits, no exchange of row
// statistics) is best while the launch still fills the chip: the smallest
// power of two covering the longest segment (at most 8192), halved (down to
// 256) while the halved launch still fits in one round of resident
// work-groups.
int fill_chunk(int n_seg, int max_seg_len) {
  constexpr int64_t kResident = 3 * 256;
  int c = 256;
  while (c < 8192 && c < max_seg_len) c <<= 1;
  while (c > 256 && int64_t(n_seg) * ((max_seg_len + c / 2 - 1) / (c / 2)) <= kResident) c >>= 1;
  return c;
}

}  // namespace

size_t score_workspace_bytes(int32_t batch, int32_t n_q, int32_t max_obs, int32_t head_dim, int32_t dtype,
                             int32_t n_seg, int32_t max_seg_len, int32_t rows) {
  const size_t elem = dtype == 0 ? 2 : 4;
  const size_t qr = align_up(size_t(batch) * n_q * max_obs * head_dim * elem);
  const size_t nch = (size_t(max_seg_len) + kScoreChunk - 1) / kScoreChunk;
  const size_t st = align_up(size_t(n_seg) * (nch ? nch : 1) * rows * sizeof(float2));
  const size_t ls = align_up(size_t(n_seg) * rows * sizeof(float));
  const size_t ct = align_up(size_t(4 * n_seg + kQueues) * sizeof(int));
  return qr + st + ls + ct;
}

size_t valu_lds_bytes(int rows, int D, int dtype) {
  return size_t(rows) * D * (dtype == 0 ? 2 : 4) + size_t(rows) * (4 * sizeof(float2) + sizeof(float) + sizeof(int));
}

namespace {

// Carve the workspace and rotate the observation queries; returns the control
// counters' address.
int* prepare(ScoreArgs& a, void* ws, hipStream_t st, hipError_t& e, int n_zero) {
  const int batch = a.n_seg / a.n_kv;
  const size_t elem = a.dtype == 0 ? 2 : 4;
  const size_t nch256 = (size_t(a.max_seg_len) + kScoreChunk - 1) / kScoreChunk;
  a.n_chunks = (a.max_seg_len + a.chunk - 1) / a.chunk;
  char* w = static_cast<char*>(ws);
  a.qr = w;
  w += align_up(size_t(batch) * a.n_q * a.max_obs * a.head_dim * elem);
  a.stats = reinterpret_cast<float2*>(w);
  w += align_up(size_t(a.n_seg) * (nch256 ? nch256 : 1) * a.rows * sizeof(float2));
  a.lse = reinterpret_cast<float*>(w);
  w += align_up(size_t(a.n_seg) * a.rows * sizeof(float));
  int* ctl = reinterpret_cast<int*>(w);
  // rows per work-group: about 256 items (V frequencies of one head's row) per block, at most
  // kRotMaxAngles sines and cosines, at most every row of a request
  const int items_per_row = a.n_q * (a.head_dim / 2) / (16 / int(elem));
  int rblk = std::max(1, 256 / std::max(1, items_per_row));
  rblk = std::min({rblk, kRotMaxAngles / (a.head_dim / 2), std::max(1, a.max_obs)});
  const int64_t n_blocks = a.max_obs > 0 ? int64_t(batch) * ((a.max_obs + rblk - 1) / rblk) : 0;
  const int64_t zero_blocks = (int64_t(n_zero) + 255) / 256;
  const InvFreq inv = inv_freq(a.theta, a.head_dim);
  if (n_blocks > 0 || n_zero > 0) {
    const dim3 rg(unsigned(std::max(n_blocks, zero_blocks)));
    if (a.dtype == 0)
      hipLaunchKernelGGL(rotate_obs_kernel<uint16_t>, rg, dim3(256), 0, st, static_cast<const uint16_t*>(a.q),
                         a.q_pos, a.n_obs, static_cast<uint16_t*>(a.qr), int(n_blocks), rblk, a.n_q, a.max_obs,
                         a.head_dim, inv, ctl, n_zero);
    else
      hipLaunchKernelGGL(rotate_obs_kernel<float>, rg, dim3(256), 0, st, static_cast<const float*>(a.q), a.q_pos,
                         a.n_obs, static_cast<float*>(a.qr), int(n_blocks), rblk, a.n_q, a.max_obs, a.head_dim, inv,
                         ctl, n_zero);
  }
  e = hipGetLastError();
  return ctl;
}

template <int D>
hipError_t launch_step(const ScoreArgs& a, int* ctl, hipStream_t st) {
  const int rt = ((a.rows + 15) / 16 + 3) / 4;
  switch (rt) {
    case 1: return launch_step_t<D, 1>(a, ctl, st);
    case 2: return launch_step_t<D, 2>(a, ctl, st);
    case 3: return launch_step_t<D, 3>(a, ctl, st);
    default: return launch_step_t<D, 4>(a, ctl, st);
  }
}

}  // namespace

hipError_t launch_score(ScoreArgs& a, void* ws, hipStream_t st) {
  const bool mfma = a.dtype == 0 && a.impl == 0;
  const bool fused = a.dtype == 0 && a.impl == 2;
  a.chunk = fused ? fused_chunk(a.n_seg, a.max_seg_len) : mfma ? mfma_chunk(a.n_seg, a.max_seg_len) : kScoreChunk;
  hipError_t e;
  int* ctl = prepare(a, ws, st, e, fused ? kQueues + a.n_seg : 0);   // tickets and an arrival counter per segment
  if (e != hipSuccess) return e;
  if (a.n_chunks == 0 || a.n_seg == 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_chunks), unsigned(a.n_seg));
  if (fused) {
    e = a.head_dim == 128 ? launch_fused<128>(a, ctl, st) : launch_fused<64>(a, ctl, st);
  } else if (mfma) {
    e = a.head_dim == 128 ? launch_mfma_rt<128>(a, grid, st) : launch_mfma_rt<64>(a, grid, st);
  } else if (a.dtype == 0) {
    e = a.head_dim == 128 ? launch_valu<uint16_t, 128>(a, grid, st) : launch_valu<uint16_t, 64>(a, grid, st);
  } else {
    e = a.head_dim == 128 ? launch_valu<float, 128>(a, grid, st) : launch_valu<float, 64>(a, grid, st);
  }
  if (e != hipSuccess) return e;
  if (a.entropy) {
    hipLaunchKernelGGL(entropy_kernel, dim3(unsigned(a.n_seg)), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

// The entropy-budget trigger keeps far fewer rows than it scores, so, as for
// the in-place form, a whole segment per work-group serves it best (one
// selection per segment, no segment barrier waits; 32-layer per-head-budget
// workload: 3.0 ms, against 3.9 ms with 1024-key chunks and 3.2 ms for the
// three calls).
bool budget_step_fits(int32_t n_seg, int32_t n_kv, int32_t max_seg_len, int32_t head_dim) {
  if (n_kv < 1 || n_kv > kMaxHeads || n_seg % n_kv != 0 || max_seg_len > step_max_seg(head_dim)) return false;
  const int c = fill_chunk(n_seg, max_seg_len);
  const int64_t items = int64_t(n_seg) * ((max_seg_len + c - 1) / c);
  return items <= 3 * 256 || int64_t(n_kv) * ((max_seg_len + c - 1) / c) <= 96;
}

hipError_t launch_score_budget_select_compact(ScoreArgs& a, void* ws, hipStream_t st) {
  a.chunk = fill_chunk(a.n_seg, a.max_seg_len);
  hipError_t e;
  // one ticket queue, three counters per segment, one per request-layer
  int* ctl = prepare(a, ws, st, e, kQueues + 3 * a.n_seg + a.n_seg / a.n_kv);
  if (e != hipSuccess) return e;
  if (a.n_chunks == 0 || a.n_seg == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_step<128>(a, ctl, st) : launch_step<64>(a, ctl, st);
}

// Scratch of the entry point that allocates nothing: a file-scope device
// array (each device holds its own copy from the code object's load until the
// process ends).  Host code must not use the array's name as an address: its
// device address is taken once per device, with that device current, and
// kept here.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

int64_t debug_take_stamps(unsigned long long* host, int64_t n_items) {
#ifdef KVE_STAMPS
  const int64_t n = n_items < kStampItems ? n_items : kStampItems;
  const size_t bytes = size_t(n) * kStampPhases * sizeof(unsigned long long);
  if (n <= 0) return 0;
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(kve_stamps), bytes) != hipSuccess) return -1;
  void* dev = nullptr;
  if (hipGetSymbolAddress(&dev, HIP_SYMBOL(kve_stamps)) != hipSuccess) return -1;
  if (hipMemset(dev, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return -1;
  return n;
#else
  (void)host;
  (void)n_items;
  return 0;
#endif
}

unsigned int debug_take_score() {
#ifdef KVE_DEBUG
  unsigned int v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kve_debug_word), sizeof(v)) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(kve_debug_word), &z, sizeof(z)) != hipSuccess) return ~0u;
  return v;
#else
  return 0;
#endif
}

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}

hipError_t launch_score_select_compact(ScoreArgs& a, void* ws, hipStream_t st) {
  a.chunk = a.inplace ? fill_chunk(a.n_seg, a.max_seg_len) : step_chunk(a.n_seg, a.max_seg_len);
  hipError_t e;
  // tickets, two arrival counters and a finish counter per segment
  int* ctl = prepare(a, ws, st, e, kQueues + 3 * a.n_seg);
  if (e != hipSuccess) return e;
  if (a.n_chunks == 0 || a.n_seg == 0) return hipSuccess;
  return a.head_dim == 128 ? launch_step<128>(a, ctl, st) : launch_step<64>(a, ctl, st);
}

}  // namespace kve
