// Focal score from stored logits, and the group-sum / average-pool post-pass.
//
// FastOCR (technical summary, Focal-Guided Pruning): focal layers rank the
// image tokens by the attention they receive.  Here each query head's
// probabilities over the candidate segment (or over every row it sees) are
// summed over the heads that share a kv head.
// FastKV section 2A: the saliency is averaged over a window of queries; the
// average pool of width 7 smooths it along the sequence.
//
// Precision: the logits are raw fp32 q.k dot products of bf16 inputs (exact
// products, fp32 sums); the max, the shift, exp, the normaliser and the head
// sum are evaluated in fp64, and the score is rounded to fp32 once, so the
// score's error is set by the fp32 dot product alone.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

constexpr int kNormThreads = 256;
constexpr int kMaxHeadsPerOut = 64;

__global__ __launch_bounds__(kNormThreads) void focal_norm_kernel(NormArgs a) {
  const int o = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ double s_m[kMaxHeadsPerOut], s_iz[kMaxHeadsPerOut];
  __shared__ float s_red[kNormThreads / 64];
  __shared__ double s_redd[kNormThreads / 64];

  const int n = clampi(a.seq_len[b], 0, a.cap_rows);
  const int s0 = clampi(a.seg_begin[b], 0, n);
  const int s1 = clampi(a.seg_end[b], s0, n);
  // logit row layout: segment mode stores rows [s0, s1) at 0; context mode rows [0, n) at 0.
  // Device values beyond the host bounds are clamped to the scratch and output strides.
  const int64_t ldo = a.scores != nullptr ? a.ld : a.ld64;
  const int cnt = (int)min((int64_t)(a.norm == KVSEL_NORM_SEGMENT ? s1 - s0 : n), a.ld_logits);
  const int off = a.norm == KVSEL_NORM_SEGMENT ? 0 : s0;
  const int seg = (int)min(min((int64_t)(s1 - s0), (int64_t)(cnt - off)), ldo);

  for (int hh = 0; hh < a.heads_per_out; ++hh) {
    const int h = o * a.heads_per_out + hh;
    const float *row = a.logits + ((size_t)b * a.hq + h) * a.ld_logits;
    float mx = -INFINITY;
    for (int i = tid; i < cnt; i += kNormThreads) mx = fmaxf(mx, row[i]);
    mx = block_max(mx, s_red);
    double z = 0.0;
    const double md = (double)mx;
    for (int i = tid; i < cnt; i += kNormThreads) z += exp(((double)row[i] - md) * a.scale);
    z = block_sum_d(z, s_redd);
    if (tid == 0) {
      s_m[hh] = md;
      s_iz[hh] = z > 0.0 ? 1.0 / z : 0.0;
    }
  }
  __syncthreads();
  for (int i = tid; i < seg; i += kNormThreads) {
    double sc = 0.0;
    for (int hh = 0; hh < a.heads_per_out; ++hh) {
      const int h = o * a.heads_per_out + hh;
      const float x = a.logits[((size_t)b * a.hq + h) * a.ld_logits + off + i];
      sc += exp(((double)x - s_m[hh]) * a.scale) * s_iz[hh];
    }
    if (a.scores != nullptr)
      a.scores[((size_t)b * a.n_out + o) * a.ld + i] = (float)sc;
    else
      a.scores64[((size_t)b * a.n_out + o) * a.ld64 + i] = sc;
  }
}

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

hipError_t launch_focal_norm(const NormArgs &a, int batch, hipStream_t s) {
  if (a.heads_per_out > kMaxHeadsPerOut) return hipErrorInvalidValue;
  hipLaunchKernelGGL(focal_norm_kernel, dim3(a.n_out, batch), dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs &a, int batch, int max_seg_len, hipStream_t s) {
  const int bx = (max_seg_len + 255) / 256;
  hipLaunchKernelGGL(pool_kernel, dim3(bx > 0 ? bx : 1, a.n_out, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
