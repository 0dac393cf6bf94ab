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
// fp64 with the reduction order of a 1024-thread block (vsum1024); per token:
// the heads' probabilities summed in fp64 and rounded to fp32 once.
#pragma once

#include "common.h"

namespace kvsel {

// logit(hh, i) for head hh < nh of the output row and segment token i < cnt
template <int NT, typename LF>
__device__ void focal_stats(LF logit, int nh, int cnt, double c, double *s_m, double *s_iz, float *redf,
                            double *redd) {
  for (int hh = 0; hh < nh; ++hh) {
    const float mx = vmax<NT>([&](int i) { return logit(hh, i); }, cnt, redf);
    const double md = (double)mx;
    const double z = vsum1024<NT>([&](int i) { return exp2_acc(((double)logit(hh, i) - md) * c); }, cnt, redd);
    if (threadIdx.x == 0) {
      s_m[hh] = md;
      s_iz[hh] = z > 0.0 ? 1.0 / z : 0.0;
    }
  }
  __syncthreads();
}

template <typename LF>
__device__ __forceinline__ double focal_score(LF logit, int nh, int i, double c, const double *s_m,
                                              const double *s_iz) {
  double sc = 0.0;
  for (int hh = 0; hh < nh; ++hh) sc += exp2_acc(((double)logit(hh, i) - s_m[hh]) * c) * s_iz[hh];
  return sc;
}

}  // namespace kvsel
