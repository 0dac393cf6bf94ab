// Focal score arithmetic shared by the fused focal attention kernel and the
// standalone normalise / select kernels, so that both give the same bits.
//
// FastOCR (technical summary, Focal-Guided Pruning): the focal score of an
// image token is the attention its query heads give it: per head a softmax
// of the logits over the candidate segment, summed over the heads of a kv
// head's group.
//
// Input logits are raw fp32 q.k dot products (exact bf16 products, fp32
// sums).  Per head: the max, then sum_i 2^((x_i - max) * scale * log2 e) in
// fp64 in a fixed order (focal_stats); per token: the heads' probabilities
// summed in fp64 and rounded to fp32 once.
#pragma once

#include "common.h"

namespace kvsel {

// logit(hh, i) for head hh < nh of the output row and token i < cnt.  Per
// head: m = max_i logit (fp32) and Z = sum_i 2^((logit - m) * c) in fp64,
// with a summation order that does not depend on NT (any NT dividing 1024):
// virtual thread v in [0, 1024) adds i = v, v + 1024, ... in order, each
// virtual wave of 64 is reduced by wave_sum_d, and the 16 virtual-wave sums
// are added in order.  Up to NH heads are done per pass over the tokens.
// Writes s_m[hh] = m and s_iz[hh] = 1 / Z (0 when Z = 0).
template <int NT, int NH, typename LF>
__device__ void focal_stats(LF logit, int nh, int cnt, double c, double *s_m, double *s_iz) {
  constexpr int NW = NT / 64, R = 1024 / NT;
  static_assert(NT % 64 == 0 && 1024 % NT == 0, "block size must divide 1024");
  __shared__ float s_wm[NH][NW];
  __shared__ double s_wz[NH][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int h0 = 0; h0 < nh; h0 += NH) {
    const int hn = min(NH, nh - h0);
    float mx[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) mx[hh] = -INFINITY;
    for (int i = tid; i < cnt; i += NT) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        if (hh < hn) mx[hh] = fmaxf(mx[hh], logit(h0 + hh, i));
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      mx[hh] = wave_max_f(mx[hh]);
      if (lane == 0) s_wm[hh][w] = mx[hh];
    }
    __syncthreads();
    double md[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float m = s_wm[hh][0];
      for (int j = 1; j < NW; ++j) m = fmaxf(m, s_wm[hh][j]);
      md[hh] = (double)m;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double part[NH];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) part[hh] = 0.0;
      for (int i = tid + r * NT; i < cnt; i += 1024) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          if (hh < hn) part[hh] += exp2_acc(((double)logit(h0 + hh, i) - md[hh]) * c);
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        part[hh] = wave_sum_d(part[hh]);
        if (lane == 0) s_wz[hh][w + r * NW] = part[hh];
      }
    }
    __syncthreads();
    if (tid < hn) {
      float m = s_wm[tid][0];
      for (int j = 1; j < NW; ++j) m = fmaxf(m, s_wm[tid][j]);
      double z = 0.0;
      for (int j = 0; j < 16; ++j) z += s_wz[tid][j];
      s_m[h0 + tid] = (double)m;
      s_iz[h0 + tid] = z > 0.0 ? 1.0 / z : 0.0;
    }
    __syncthreads();
  }
}

template <typename LF>
__device__ __forceinline__ double focal_score(LF logit, int nh, int i, double c, const double *s_m,
                                              const double *s_iz) {
  double sc = 0.0;
  for (int hh = 0; hh < nh; ++hh) sc += exp2_acc(((double)logit(hh, i) - s_m[hh]) * c) * s_iz[hh];
  return sc;
}

}  // namespace kvsel
