// Focal score normalisation, alone or fused with the exact top-k, one
// work-group per (sequence, output row), reading logits stored by the
// attention, logits or shared-prefix kernel (the path for shapes the fused
// focal attention kernel does not take: split attention, context
// normalisation, long segments, and the focal layers of a shared-prefix
// cascade).
//
// FastOCR (technical summary, Focal-Guided Pruning): a focal layer ranks the
// image tokens by the attention its queries give them and keeps the top tau;
// Cross-Step Fixation Reuse: the previous step's set warm-starts the choice.
// The arithmetic is focal.h's; selection is radix.h's.
#include "common.h"
#include "focal.h"
#include "kvsel_internal.h"
#include "radix.h"

namespace kvsel {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kMaxHeadsPerOut = 64;
// the fused selection: 512 threads (the statistics' virtual threads, one
// each) when the launch has a row per CU or more, so that four work-groups
// share a compute unit; 1024 for fewer rows (more threads per row).  Same
// bits either way.  The keys sit in dynamic LDS sized to the longest segment
// a row can hold (its logits row).
constexpr int kSelectThreads = kStatThreads;
inline __host__ __device__ int select_cap(int64_t ld_logits) { return (int)min(ld_logits, (int64_t)kSelMaxSeg); }

struct FocalRow {
  int cnt, off, seg;
};

__device__ __forceinline__ FocalRow focal_row(const SelArgs &a, int b, int64_t ld_out) {
  FocalRow r;
  const int n = clampi(a.seq_len[b], 0, a.cap_rows);
  const int s0 = clampi(a.seg_begin[b], 0, n);
  const int s1 = clampi(a.seg_end[b], s0, n);
  // logit rows: segment mode holds rows [s0, s1) at 0, context mode rows [0, n) at 0
  r.cnt = (int)min((int64_t)(a.norm == KVSEL_NORM_SEGMENT ? s1 - s0 : n), a.ld_logits);
  r.off = a.norm == KVSEL_NORM_SEGMENT ? 0 : s0;
  r.seg = (int)min((int64_t)min(s1 - s0, r.cnt - r.off), ld_out);
  return r;
}

// grid (output rows, sequences): scores only
__global__ __launch_bounds__(kSelThreads) void focal_norm_kernel(SelArgs a) {
  __shared__ double s_m[kMaxHeadsPerOut], s_iz[kMaxHeadsPerOut];
  const int o = blockIdx.x, b = blockIdx.y;
  const FocalRow r = focal_row(a, b, a.scores != nullptr ? a.ld : a.ld64);
  const double c = a.scale * 1.4426950408889634;
  const float *base = a.logits + ((size_t)b * a.hq + o * a.heads_per_out) * a.ld_logits;
  auto stat_logit = [&](int hh, int i) { return base[(size_t)hh * a.ld_logits + i]; };
  focal_stats<kSelThreads, 4>(stat_logit, a.heads_per_out, r.cnt, c, s_m, s_iz);
  const float *lg = base + r.off;
  auto seg_logit = [&](int hh, int i) { return lg[(size_t)hh * a.ld_logits + i]; };
  for (int i0 = threadIdx.x; i0 < r.seg; i0 += kSelThreads * kStatBatch)
    focal_scores_batch(seg_logit, a.heads_per_out, i0, kSelThreads, r.seg, c, s_m, s_iz, [&](int i, double sc) {
      if (a.scores != nullptr)
        a.scores[((size_t)b * a.n_out + o) * a.ld + i] = (float)sc;
      else
        a.scores64[((size_t)b * a.n_out + o) * a.ld64 + i] = sc;
    });
}

// grid (kv heads, sequences): scores + top-k of the group
template <int NT>
__global__ __launch_bounds__(NT) void focal_select_kernel(SelArgs a) {
  extern __shared__ uint32_t s_keys[];   // select_cap(ld_logits) keys
  __shared__ RadixShared<NT> sh;
  __shared__ double s_m[8], s_iz[8];
  const int g = blockIdx.x, b = blockIdx.y;
  FocalRow r = focal_row(a, b, a.scores != nullptr ? a.ld : (int64_t)kSelMaxSeg);
  r.seg = min(r.seg, select_cap(a.ld_logits));
  const double c = a.scale * 1.4426950408889634;
  const float *base = a.logits + ((size_t)b * a.hq + g * a.heads_per_out) * a.ld_logits;
  auto stat_logit = [&](int hh, int i) { return base[(size_t)hh * a.ld_logits + i]; };
  focal_stats<NT, 4>(stat_logit, a.heads_per_out, r.cnt, c, s_m, s_iz);
  const float *lg = base + r.off;
  auto seg_logit = [&](int hh, int i) { return lg[(size_t)hh * a.ld_logits + i]; };
  float *so = a.scores != nullptr ? a.scores + ((size_t)b * a.n_out + g) * a.ld : nullptr;
  for (int i0 = threadIdx.x; i0 < r.seg; i0 += NT * kStatBatch)
    focal_scores_batch(seg_logit, a.heads_per_out, i0, NT, r.seg, c, s_m, s_iz, [&](int i, double sc) {
      const float f = (float)sc;
      s_keys[i] = okey(f);
      if (so != nullptr) so[i] = f;
    });
  __syncthreads();
  auto key = [&](int i) -> uint32_t { return s_keys[i]; };
  const size_t row = (size_t)b * a.n_out + g;
  BlockSync<NT> grp;
  radix_topk<NT, true, 25>(grp, key, r.seg, a.k, a.warm != nullptr ? a.warm + row * a.k : nullptr, a.idx + row * a.k, sh,
                           s_keys);
}

}  // namespace

hipError_t launch_focal_norm(const SelArgs &a, int batch, hipStream_t s) {
  if (a.heads_per_out > kMaxHeadsPerOut) return hipErrorInvalidValue;
  hipLaunchKernelGGL(focal_norm_kernel, dim3(a.n_out, batch), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_focal_select(const SelArgs &a, int batch, hipStream_t s) {
  if (a.heads_per_out > 8) return hipErrorInvalidValue;
  const size_t dyn = (size_t)select_cap(a.ld_logits) * sizeof(uint32_t);
  if ((int64_t)a.n_out * batch < 256)
    hipLaunchKernelGGL(focal_select_kernel<2 * kSelectThreads>, dim3(a.n_out, batch), dim3(2 * kSelectThreads), dyn, s,
                       a);
  else
    hipLaunchKernelGGL(focal_select_kernel<kSelectThreads>, dim3(a.n_out, batch), dim3(kSelectThreads), dyn, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
