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

// rows up to this length are staged in LDS (144 KiB of dynamic LDS; gfx950
// gives a work-group up to 160 KiB)
constexpr int kLdsKeys = 36864;

template <int NT, bool IN_LDS>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ RadixShared<NT> sh;
  const int row = blockIdx.x;
  const float *src = a.scores + (size_t)row * a.ld;
  const int n = a.n_row != nullptr ? clampi(a.n_row[row], 0, a.n) : a.n;   // this row's candidates
  // a cold row's candidate range (every key), taken while staging
  uint32_t lo = 0xffffffffu, hi = 0u;
  if (IN_LDS) {
    // 32 loads in flight per thread before the LDS stores (one memory latency
    // for a whole row of up to 32768 keys)
    constexpr int B = 32;
    for (int base = 0; base < n; base += B * NT) {
      float v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int i = base + j * NT + threadIdx.x;
        v[j] = i < n ? src[i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int i = base + j * NT + threadIdx.x;
        if (i < n) {
          const uint32_t x = okey(v[j]);
          s_keys[i] = x;
          lo = min(lo, x);
          hi = max(hi, x);
        }
      }
    }
    __syncthreads();
  }
  auto key = [&](int i) -> uint32_t { return IN_LDS ? s_keys[i] : okey(src[i]); };
  BlockSync<NT> grp;
  int32_t *dst = a.idx + (size_t)row * a.k;
  if (IN_LDS && a.warm == nullptr && n > a.k) {
    // cold: the range is known, so the selection starts at the digit passes
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      sh.w1[w] = lo;
      sh.w2[w] = hi;
    }
    __syncthreads();
    lo = 0xffffffffu;
    hi = 0u;
    for (int i = 0; i < NT / 64; ++i) {
      lo = min(lo, sh.w1[i]);
      hi = max(hi, sh.w2[i]);
    }
    __syncthreads();
    radix_select<NT, IN_LDS>(grp, key, n, a.k, 0u, lo, hi, (uint32_t)n, dst, sh);
    return;
  }
  radix_topk<NT, IN_LDS>(grp, key, n, a.k, a.warm != nullptr ? a.warm + (size_t)row * a.k : nullptr, dst, sh);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.n <= kLdsKeys) {
    // LDS above 64 KiB must be allowed (once per device)
    const hipError_t e = allow_dynamic_lds((const void *)topk_kernel<1024, true>, kLdsKeys * 4);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_kernel<1024, true>), dim3(a.rows), dim3(1024), (size_t)a.n * 4, s, a);
  } else {
    hipLaunchKernelGGL((topk_kernel<1024, false>), dim3(a.rows), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvsel
