// Key rotation at cache-write time: rows of fp32 pre-RoPE keys rotated to their
// positions (half-split pairs, double-precision angle and rotation) and
// rounded once to the storage dtype.  The same rotation rotates observation
// queries inside the scoring call (BeaconKV, "打分时的 RoPE 对齐").
#include "common.h"
#include "internal.h"

namespace kve {

namespace {

template <typename T>
__global__ void rope_rows_kernel(const float* __restrict__ src, T* __restrict__ dst, const int32_t* __restrict__ pos,
                                 int64_t n_pairs, int D, InvFreq inv) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_pairs) return;
  const int half = D / 2;
  const int64_t row = idx / half;
  const int i = int(idx % half);
  const float* x = src + row * D;
  RotPair r = rope_pair(double(x[i]), double(x[i + half]), inv.v[i], pos[row]);
  dst[row * D + i] = Elem<T>::from_f64(r.a);
  dst[row * D + i + half] = Elem<T>::from_f64(r.b);
}

}  // namespace

hipError_t launch_rope_rows(const float* src, void* dst, const int32_t* pos, int64_t n_rows, int32_t head_dim,
                            double theta, int32_t dtype, hipStream_t st) {
  const int64_t n_pairs = n_rows * (head_dim / 2);
  if (n_pairs == 0) return hipSuccess;
  const dim3 grid(unsigned((n_pairs + 255) / 256));
  const InvFreq inv = inv_freq(theta, head_dim);
  if (dtype == 0)
    hipLaunchKernelGGL(rope_rows_kernel<uint16_t>, grid, dim3(256), 0, st, src, static_cast<uint16_t*>(dst), pos,
                       n_pairs, head_dim, inv);
  else
    hipLaunchKernelGGL(rope_rows_kernel<float>, grid, dim3(256), 0, st, src, static_cast<float*>(dst), pos, n_pairs,
                       head_dim, inv);
  return hipGetLastError();
}

}  // namespace kve
