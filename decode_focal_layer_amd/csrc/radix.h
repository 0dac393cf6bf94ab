// Exact top-k of one row held as order-preserving uint32 keys, for one
// work-group: ties to the lower index, output ascending.
//
// The k-th largest key T is found by a radix select (digits of 11, 11 and 10
// bits, LDS histograms); a final pass over the row in index order keeps every
// key > T and the first (k - #keys > T) keys equal to T, placing them with
// wave ballots, so the output is ascending without a sort.  Only keys >= theta
// are ranked; theta must not exceed the k-th largest key (a warm start's
// minimum does not: at least k keys reach it).
#pragma once

#include "common.h"

namespace kvsel {

// float -> uint32 with the same order (negative floats below positive ones)
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
struct RadixShared {
  uint32_t hist[2048];
  uint32_t w1[NT / 64];
  uint32_t w2[NT / 64];
  uint32_t misc[4];
};

// exclusive scan of one value per thread in thread order; total returned
template <int NT>
__device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t *ws, uint32_t &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) ws[w] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = ws[i];
    pre += i < w ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// theta from a warm selection: the smallest key at the warm indices, or 0 (rank
// everything) if they are not strictly ascending and inside [0, n).
template <int NT, typename KeyFn>
__device__ uint32_t warm_theta(KeyFn key, const int32_t *wi, int n, int k, RadixShared<NT> &sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t bad = 0, mn = 0xffffffffu;
  for (int j = threadIdx.x; j < k; j += NT) {
    const int x = wi[j];
    if (x < 0 || x >= n) {
      bad = 1;
    } else {
      if (j + 1 < k && wi[j + 1] <= x) bad = 1;
      mn = min(mn, key(x));
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    bad |= __shfl_xor(bad, o);
    mn = min(mn, (uint32_t)__shfl_xor(mn, o));
  }
  __syncthreads();
  if (lane == 0) {
    sh.w1[w] = bad;
    sh.w2[w] = mn;
  }
  __syncthreads();
  uint32_t b2 = 0, m2 = 0xffffffffu;
  for (int i = 0; i < NT / 64; ++i) {
    b2 |= sh.w1[i];
    m2 = min(m2, sh.w2[i]);
  }
  __syncthreads();
  return b2 ? 0u : m2;
}

// keys: key(i) for i in [0, n).  Writes k indices to dst (ascending); when
// n < k the n indices are followed by -1.
template <int NT, typename KeyFn>
__device__ void radix_topk(KeyFn key, int n, int k, uint32_t theta, int32_t *dst, RadixShared<NT> &sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) dst[i] = i < n ? i : -1;
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass], nb = 1 << kBits[pass];
    for (int i = tid; i < nb; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t x = key(i);
      if (x >= theta && (x & pmask) == prefix) atomicAdd(&sh.hist[(x >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [t*per, (t+1)*per); count of the bins above its range
    const int per = nb / NT;
    uint32_t c = 0;
    for (int i = 0; i < per; ++i) c += sh.hist[tid * per + i];
    uint32_t total;
    const uint32_t below = excl_scan<NT>(c, sh.w1, total);
    const uint32_t above = total - below - c;
    if (above < (uint32_t)krem && (uint32_t)krem <= above + c) {
      uint32_t run = above;
      for (int i = per - 1; i >= 0; --i) {
        const uint32_t hcount = sh.hist[tid * per + i];
        if (run + hcount >= (uint32_t)krem) {
          sh.misc[0] = (uint32_t)(tid * per + i);
          sh.misc[1] = run;
          break;
        }
        run += hcount;
      }
    }
    __syncthreads();
    prefix |= sh.misc[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem -= (int)sh.misc[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t keq = (uint32_t)krem;   // keys equal to T to keep (>= 1)

  uint32_t written = 0, eq_seen = 0;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int base = 0; base < n && written < (uint32_t)k; base += NT) {
    const int i = base + tid;
    const uint32_t x = i < n ? key(i) : 0u;
    const bool gt = i < n && x > T;
    const bool eq = i < n && x == T;
    const uint64_t meq = __ballot(eq);
    if (lane == 0) sh.w1[w] = (uint32_t)__popcll(meq);
    __syncthreads();
    uint32_t eq_pre = 0, eq_tot = 0;
    for (int j = 0; j < NT / 64; ++j) {
      eq_pre += j < w ? sh.w1[j] : 0u;
      eq_tot += sh.w1[j];
    }
    eq_pre += (uint32_t)__popcll(meq & lt);
    const bool take = gt || (eq && eq_seen + eq_pre < keq);
    const uint64_t mt = __ballot(take);
    if (lane == 0) sh.w2[w] = (uint32_t)__popcll(mt);
    __syncthreads();
    uint32_t t_pre = 0, t_tot = 0;
    for (int j = 0; j < NT / 64; ++j) {
      t_pre += j < w ? sh.w2[j] : 0u;
      t_tot += sh.w2[j];
    }
    t_pre += (uint32_t)__popcll(mt & lt);
    if (take && written + t_pre < (uint32_t)k) dst[written + t_pre] = i;
    written += t_tot;
    eq_seen += eq_tot;
    __syncthreads();
  }
}

}  // namespace kvsel
