// Exact top-k per row with the lower index kept among equal scores, output
// ascending.
//
// FastOCR (technical summary, Focal-Guided Pruning): keep the top tau of the
// image tokens; Cross-Step Fixation Reuse: the previous step's set is a warm
// start.  FastKV 2A: keep the top-ranked tokens.
//
// Short rows: one work-group per row.  Rows that fit are staged in LDS as
// order-preserving keys once; the selection itself is radix_topk (radix.h).
//
// Long rows (n > kLdsKeys): two kernels, the kernel boundary being the only
// synchronisation between them.
//  1. slices: many work-groups per row, each a slice of kSliceKeys keys, count
//     the keys of every coarse bin -- the top 11 bits of the key (sign,
//     exponent, three mantissa bits) -- in LDS (four copies of each bin, so
//     lanes of a wave adding to one bin mostly hit different words) and store
//     the slice's 2048 counts to its own workspace slot.
//  2. select: one work-group per row sums its slices' counts, finds the coarse
//     bin holding the k-th largest key, and runs the exact radix select over
//     the keys from that bin's lower edge up (theta) with the range bounded by
//     the highest non-empty bin, so that its digit passes see only about k
//     keys plus one bin's worth.  The warm start is not used on this path (it
//     never changes the result).
#include "common.h"
#include "kvsel_internal.h"
#include "radix.h"

namespace kvsel {

namespace {

// rows up to this length are staged in LDS (144 KiB of dynamic LDS; gfx950
// gives a work-group up to 160 KiB)
constexpr int kLdsKeys = 36864;
// keys per thread held in registers by the staged output (kLdsKeys / 1024, odd)
constexpr int kStageC = 37;

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
      for (int j = 0; j < B; ++j) v[j] = src[min(base + j * NT + (int)threadIdx.x, n - 1)];   // unbranched reads
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
    radix_select<NT, IN_LDS, kStageC>(grp, key, n, a.k, 0u, lo, hi, (uint32_t)n, dst, sh, IN_LDS ? s_keys : nullptr);
    return;
  }
  radix_topk<NT, IN_LDS, kStageC>(grp, key, n, a.k, a.warm != nullptr ? a.warm + (size_t)row * a.k : nullptr, dst, sh,
                                  IN_LDS ? s_keys : nullptr);
}

constexpr int kCoarseBins = 2048;   // key >> 21
constexpr int kCoarseShift = 21;
constexpr int kSliceThreads = 256;
constexpr int kSliceKeys = 8192;
constexpr int kBinCopies = 4;

__device__ __forceinline__ int row_len(const TopkArgs &a, int row) {
  return a.n_row != nullptr ? clampi(a.n_row[row], 0, a.n) : a.n;
}

// grid (slices, rows): coarse-bin counts of one slice
__global__ __launch_bounds__(kSliceThreads) void topk_slice_kernel(TopkArgs a, uint32_t *counts, int nslices) {
  __shared__ uint32_t h[kCoarseBins * kBinCopies];
  const int sl = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < kCoarseBins * kBinCopies; i += kSliceThreads) h[i] = 0u;
  __syncthreads();
  const int n = row_len(a, row);
  const int i0 = sl * kSliceKeys, i1 = min(n, i0 + kSliceKeys);
  const float *src = a.scores + (size_t)row * a.ld;
  const uint32_t copy = (uint32_t)(tid & (kBinCopies - 1));
  constexpr int B = kSliceKeys / kSliceThreads;   // keys per thread, all loads in flight together
  float v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) v[j] = src[min(i0 + j * kSliceThreads + tid, max(i1 - 1, 0))];   // unbranched reads
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int i = i0 + j * kSliceThreads + tid;
    if (i < i1) atomicAdd(&h[(okey(v[j]) >> kCoarseShift) * kBinCopies + copy], 1u);
  }
  __syncthreads();
  uint32_t *dst = counts + ((size_t)row * nslices + sl) * kCoarseBins;
  for (int b = tid; b < kCoarseBins; b += kSliceThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < kBinCopies; ++r) c += h[b * kBinCopies + r];
    dst[b] = c;
  }
}

// grid (rows): the exact top-k of a row (keys read from global memory) from
// its slices' coarse counts
template <int NT>
__global__ __launch_bounds__(NT) void topk_select_kernel(TopkArgs a, const uint32_t *counts, int nslices) {
  __shared__ RadixShared<NT> sh;
  uint32_t *s_hist = sh.hist;   // the coarse counts; free again before the radix select needs it
  static_assert(sizeof(sh.hist) / sizeof(sh.hist[0]) == kCoarseBins, "one count per coarse bin");
  const int row = blockIdx.x, t = threadIdx.x;
  const float *src = a.scores + (size_t)row * a.ld;
  const int n = row_len(a, row);
  int32_t *dst = a.idx + (size_t)row * a.k;
  BlockSync<NT> grp;
  if (n <= a.k) {   // every candidate kept
    for (int i = t; i < a.k; i += NT) dst[i] = i < n ? i : -1;
    return;
  }
  const int ns = (n + kSliceKeys - 1) / kSliceKeys;
  const uint32_t *rc = counts + (size_t)row * nslices * kCoarseBins;
  for (int b = t; b < kCoarseBins; b += NT) {
    uint32_t c = 0;
    constexpr int U = 16;   // slices read per step, all loads in flight together
    for (int s0 = 0; s0 < ns; s0 += U) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s0 + u < ns ? rc[(size_t)(s0 + u) * kCoarseBins + b] : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) c += v[u];
    }
    s_hist[b] = c;
  }
  if (t == 0) sh.misc[6] = 0u;
  grp.sync();
  // the bin holding the k-th largest key: participant t owns bins [t*per, (t+1)*per)
  constexpr int per = kCoarseBins / NT;
  static_assert(kCoarseBins % NT == 0, "whole bins per participant");
  uint32_t c = 0, top_nz = 0;
  for (int i = 0; i < per; ++i) {
    const uint32_t hc = s_hist[t * per + i];
    c += hc;
    if (hc != 0u) top_nz = (uint32_t)(t * per + i);
  }
  uint32_t total;
  const uint32_t below = excl_scan<NT>(grp, c, sh.w1, total);
  const uint32_t above = total - below - c;
  if (above < (uint32_t)a.k && (uint32_t)a.k <= above + c) {
    uint32_t run = above;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t hc = s_hist[t * per + i];
      if (run + hc >= (uint32_t)a.k) {
        sh.misc[0] = (uint32_t)(t * per + i);
        sh.misc[2] = run + hc;   // keys in this bin and above it
        break;
      }
      run += hc;
    }
  }
  const uint32_t wtop = wave_max_u32(top_nz);
  if ((t & 63) == 0) atomicMax(&sh.misc[6], wtop);
  grp.sync();
  const uint32_t b1 = sh.misc[0], ncand = sh.misc[2], btop = sh.misc[6];
  grp.sync();
  const uint32_t theta = b1 << kCoarseShift;
  const uint32_t hi = btop >= (uint32_t)(kCoarseBins - 1) ? 0xffffffffu : ((btop + 1u) << kCoarseShift) - 1u;
  auto key = [&](int i) -> uint32_t { return okey(src[i]); };
  radix_select<NT, false>(grp, key, n, a.k, theta, theta, hi, ncand, dst, sh);
}

}  // namespace

size_t topk_workspace_bytes(int rows, int n) {
  if (n <= kLdsKeys) return 0;
  const size_t nslices = ((size_t)n + kSliceKeys - 1) / kSliceKeys;
  return (size_t)rows * nslices * kCoarseBins * sizeof(uint32_t);
}

hipError_t launch_topk(const TopkArgs &a, void *ws, hipStream_t s) {
  if (a.n > kLdsKeys) {   // rows too long for LDS: the two-kernel path
    const int nslices = (a.n + kSliceKeys - 1) / kSliceKeys;
    uint32_t *counts = static_cast<uint32_t *>(ws);
    hipLaunchKernelGGL(topk_slice_kernel, dim3(nslices, a.rows), dim3(kSliceThreads), 0, s, a, counts, nslices);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_select_kernel<1024>), dim3(a.rows), dim3(1024), 0, s, a, (const uint32_t *)counts,
                       nslices);
    return hipGetLastError();
  }
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
