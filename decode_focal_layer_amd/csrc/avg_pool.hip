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
// sums the partial rows (in order) of its PER * 256 positions and the
// window's halo into LDS, PER positions per thread with all their loads
// issued together (read at clamped positions, unbranched, and masked after),
// then each output adds its window from LDS (positions outside the segment
// are 0).  Same sums in the same order as pool_kernel.  PER > 1 turns many
// small work-groups (whose launch and first load dominate) into fewer with
// more loads in flight, where the launch has plenty of them.
constexpr int kPoolMaxHalo = 255;

template <int kPoolPer>
__global__ __launch_bounds__(256) void pool_lds_kernel(PoolArgs a) {
  constexpr int P = 256 * kPoolPer;   // positions per work-group
  __shared__ double s_h[P + 2 * kPoolMaxHalo];
  const int i0 = blockIdx.x * P, o = blockIdx.y, b = blockIdx.z;
  const int n = clampi(a.seq_len[b], 0, a.cap_rows);
  const int s0 = clampi(a.seg_begin[b], 0, n);
  const int s1 = clampi(a.seg_end[b], s0, n);
  const int seg = (int)min(min((int64_t)(s1 - s0), a.ld64), a.ld);
  if (i0 >= seg) return;   // the whole work-group (seg >= 1 below)
  const int per = a.n_in / a.n_out;
  const int h = a.width / 2;
  const int span = P + 2 * h;   // halo included
  const double *x0 = a.part + ((size_t)b * a.n_in + o * per) * a.ld64;
  for (int q0 = threadIdx.x; q0 < span; q0 += 256 * kPoolPer) {
    double v[kPoolPer];
    int jc[kPoolPer];
    bool in[kPoolPer];
#pragma unroll
    for (int r = 0; r < kPoolPer; ++r) {
      const int j = i0 - h + q0 + 256 * r;
      in[r] = q0 + 256 * r < span && j >= 0 && j < seg;
      jc[r] = min(max(j, 0), seg - 1);
      v[r] = 0.0;
    }
#pragma unroll 8
    for (int p = 0; p < per; ++p) {   // unrolled: the rows' loads go out together
      const double *xp = x0 + (size_t)p * a.ld64;
      double t[kPoolPer];
#pragma unroll
      for (int r = 0; r < kPoolPer; ++r) t[r] = xp[jc[r]];
#pragma unroll
      for (int r = 0; r < kPoolPer; ++r) v[r] += in[r] ? t[r] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < kPoolPer; ++r)
      if (q0 + 256 * r < span) s_h[q0 + 256 * r] = v[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPoolPer; ++r) {
    const int q = (int)threadIdx.x + 256 * r, i = i0 + q;
    if (i >= seg) break;
    double sum = 0.0;
    for (int d = 0; d < a.width; ++d) sum += s_h[q + d];   // positions i - h .. i + h
    a.scores[((size_t)b * a.n_out + o) * a.ld + i] = (float)(sum / (double)a.width);
  }
}

}  // namespace

// work-groups below which fewer positions per thread are taken (4 per CU)
constexpr int64_t kPoolMinGroups = 1024;

hipError_t launch_pool(const PoolArgs &a, int batch, int max_seg_len, hipStream_t s) {
  if (a.width / 2 <= kPoolMaxHalo) {
    auto groups = [&](int per) { return (int64_t)((max_seg_len + 256 * per - 1) / (256 * per)) * a.n_out * batch; };
    auto go = [&](auto kern, int per) {
      const int bx = (max_seg_len + 256 * per - 1) / (256 * per);
      hipLaunchKernelGGL(kern, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
    };
    if (groups(8) >= kPoolMinGroups)
      go(pool_lds_kernel<8>, 8);
    else if (groups(4) >= kPoolMinGroups)
      go(pool_lds_kernel<4>, 4);
    else if (groups(2) >= kPoolMinGroups)
      go(pool_lds_kernel<2>, 2);
    else
      go(pool_lds_kernel<1>, 1);
  } else {
    const int bx = (max_seg_len + 255) / 256;
    hipLaunchKernelGGL(pool_kernel, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvsel
