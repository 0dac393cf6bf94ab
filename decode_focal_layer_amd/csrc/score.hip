// Group-sum and average-pool post-pass over fp64 partial scores.
//
// FastKV section 2A: the saliency is averaged over a window of queries; the
// average pool of width 7 smooths it along the sequence.  Partial rows (one
// per kv head) are summed in a fixed order, pooled in fp64 and rounded to
// fp32 once.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x, o = blockIdx.y, b = blockIdx.z;
  const int n = clampi(a.seq_len[b], 0, a.cap_rows);
  const int s0 = clampi(a.seg_begin[b], 0, n);
  const int s1 = clampi(a.seg_end[b], s0, n);
  const int seg = (int)min(min((int64_t)(s1 - s0), a.ld64), a.ld);
  if (i >= seg) return;
  const int per = a.n_in / a.n_out;
  const int h = a.width / 2;
  const int j0 = i - h < 0 ? 0 : i - h;
  const int j1 = i + h >= seg ? seg - 1 : i + h;
  double s = 0.0;
  for (int p = 0; p < per; ++p) {
    const double *x = a.part + ((size_t)b * a.n_in + o * per + p) * a.ld64;
    for (int j = j0; j <= j1; ++j) s += x[j];
  }
  a.scores[((size_t)b * a.n_out + o) * a.ld + i] = (float)(s / (double)a.width);
}

}  // namespace

hipError_t launch_pool(const PoolArgs &a, int batch, int max_seg_len, hipStream_t s) {
  const int bx = (max_seg_len + 255) / 256;
  hipLaunchKernelGGL(pool_kernel, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
