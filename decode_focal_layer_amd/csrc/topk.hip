// Exact top-k per row with the lower index kept among equal scores, output
// ascending.
//
// FastOCR (technical summary, Focal-Guided Pruning): keep the top tau of the
// image tokens; Cross-Step Fixation Reuse: the previous step's set is a warm
// start.  FastKV 2A: keep the top-ranked tokens.
//
// One work-group per row.  Rows that fit are staged in LDS as order-preserving
// keys once; longer rows are read from global memory on every pass.  The
// selection itself is radix_topk (radix.h).
#include "common.h"
#include "kvsel_internal.h"
#include "radix.h"

namespace kvsel {

namespace {

constexpr int kLdsKeys = 12288;   // rows up to this length are staged in LDS (48 KiB)

template <int NT, bool IN_LDS>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t s_keys[IN_LDS ? kLdsKeys : 1];
  __shared__ RadixShared<NT> sh;
  const int row = blockIdx.x;
  const float *src = a.scores + (size_t)row * a.ld;
  if (IN_LDS) {
    for (int i = threadIdx.x; i < a.n; i += NT) s_keys[i] = okey(src[i]);
    __syncthreads();
  }
  auto key = [&](int i) -> uint32_t { return IN_LDS ? s_keys[i] : okey(src[i]); };
  const uint32_t theta = a.warm != nullptr ? warm_theta<NT>(key, a.warm + (size_t)row * a.k, a.n, a.k, sh) : 0u;
  radix_topk<NT>(key, a.n, a.k, theta, a.idx + (size_t)row * a.k, sh);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.n <= kLdsKeys) {
    hipLaunchKernelGGL((topk_kernel<1024, true>), dim3(a.rows), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL((topk_kernel<1024, false>), dim3(a.rows), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvsel
