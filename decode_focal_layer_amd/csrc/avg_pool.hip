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

// The same pool for widths up to 2 kPoolMaxHalo + 1: each work-group first
// sums the partial rows (in order) of its 256 positions and the window's halo
// into LDS, one position per thread with all its loads issued together, then
// each output adds its window from LDS (positions outside the segment are 0).
constexpr int kPoolMaxHalo = 255;

__global__ __launch_bounds__(256) void pool_lds_kernel(PoolArgs a) {
  __shared__ double s_h[256 + 2 * kPoolMaxHalo];
  const int i0 = blockIdx.x * 256, o = blockIdx.y, b = blockIdx.z;
  const int n = clampi(a.seq_len[b], 0, a.cap_rows);
  const int s0 = clampi(a.seg_begin[b], 0, n);
  const int s1 = clampi(a.seg_end[b], s0, n);
  const int seg = (int)min(min((int64_t)(s1 - s0), a.ld64), a.ld);
  if (i0 >= seg) return;   // the whole work-group
  const int per = a.n_in / a.n_out;
  const int h = a.width / 2;
  const double *x0 = a.part + ((size_t)b * a.n_in + o * per) * a.ld64;
  for (int q = threadIdx.x; q < 256 + 2 * h; q += 256) {
    const int j = i0 - h + q;
    double v = 0.0;
    if (j >= 0 && j < seg) {
#pragma unroll 8
      for (int p = 0; p < per; ++p) v += x0[(size_t)p * a.ld64 + j];
    }
    s_h[q] = v;
  }
  __syncthreads();
  const int i = i0 + (int)threadIdx.x;
  if (i >= seg) return;
  double sum = 0.0;
  for (int d = 0; d < a.width; ++d) sum += s_h[threadIdx.x + d];   // positions i - h .. i + h
  a.scores[((size_t)b * a.n_out + o) * a.ld + i] = (float)(sum / (double)a.width);
}

}  // namespace

hipError_t launch_pool(const PoolArgs &a, int batch, int max_seg_len, hipStream_t s) {
  const int bx = (max_seg_len + 255) / 256;
  if (a.width / 2 <= kPoolMaxHalo)
    hipLaunchKernelGGL(pool_lds_kernel, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pool_kernel, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
