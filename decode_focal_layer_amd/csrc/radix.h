// Exact top-k of one row held as order-preserving uint32 keys, for one
// work-group: ties to the lower index, output ascending.
//
// The k-th largest key T is found by a radix select over (key - min), where
// min and max are taken over the candidate keys first: the digits (11 bits,
// from the top of the candidates' range down) then spread over the range the
// row actually occupies.  Scores of one softmax share a few float exponents,
// so digits taken from the raw key would put nearly every key into a handful
// of histogram bins (serialised LDS atomics).  The output pass gives each
// wave a contiguous range of indices, read 64 consecutive keys at a time (no
// LDS bank conflicts, coalesced global reads): the waves count their keys > T
// and == T, and each then places its chosen indices in order with ballot
// masks -- so the output is ascending and ties go to the lower index.  Only
// keys >= theta are ranked; theta must not exceed the k-th largest key (a warm
// start's minimum does not: at least k keys reach it).
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

// f(i, key(i)) for i = tid, tid + NT, ... below n; each thread issues B key
// reads before using them (one memory latency per B keys)
template <int NT, int B, typename KeyFn, typename F>
__device__ __forceinline__ void each_key(KeyFn key, int n, F f) {
  for (int base = 0; base < n; base += B * NT) {
    uint32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * NT + (int)threadIdx.x;
      x[j] = i < n ? key(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * NT + (int)threadIdx.x;
      if (i < n) f(i, x[j]);
    }
  }
}

// the calling wave walks [i0, i1) 64 consecutive keys at a time:
// f(i, valid, key) in every lane, the same number of calls in each lane
template <int B, typename KeyFn, typename F>
__device__ __forceinline__ void each_key_wave(KeyFn key, int i0, int i1, F f) {
  const int lane = threadIdx.x & 63;
  for (int base = i0; base < i1; base += B * 64) {
    uint32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * 64 + lane;
      x[j] = i < i1 ? key(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int b2 = base + j * 64;
      if (b2 < i1) f(b2 + lane, b2 + lane < i1, x[j]);
    }
  }
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
// n <= k all n indices are kept, followed by -1.
template <int NT, typename KeyFn>
__device__ void radix_topk(KeyFn key, int n, int k, uint32_t theta, int32_t *dst, RadixShared<NT> &sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) dst[i] = i < n ? i : -1;
    return;
  }
  // ---- range of the candidate keys ----
  constexpr int B = 8;
  uint32_t lo = 0xffffffffu, hi = 0u;
  each_key<NT, B>(key, n, [&](int, uint32_t x) {
    if (x >= theta) {
      lo = min(lo, x);
      hi = max(hi, x);
    }
  });
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor(lo, o));
    hi = max(hi, (uint32_t)__shfl_xor(hi, o));
  }
  if (lane == 0) {
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
  const uint32_t range = hi - lo;
  const int nbits = range == 0u ? 0 : 32 - __clz(range);

  // ---- radix select of the k-th largest (key - lo) among candidates ----
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  for (int top = nbits; top > 0; top -= 11) {
    const int bits = top < 11 ? top : 11;
    const int shift = top - bits;
    const int nb = 1 << bits;
    for (int i = tid; i < nb; i += NT) sh.hist[i] = 0;
    __syncthreads();
    each_key<NT, B>(key, n, [&](int, uint32_t x) {
      const uint32_t r = x - lo;
      if (x >= theta && (r & pmask) == prefix) atomicAdd(&sh.hist[(r >> shift) & (nb - 1)], 1u);
    });
    __syncthreads();
    // thread t owns bins [t*per, (t+1)*per) (empty past nb); bins above its range
    const int per = (nb + NT - 1) / NT;
    uint32_t c = 0;
    for (int i = 0; i < per; ++i) {
      const int bi = tid * per + i;
      c += bi < nb ? sh.hist[bi] : 0u;
    }
    uint32_t total;
    const uint32_t below = excl_scan<NT>(c, sh.w1, total);
    const uint32_t above = total - below - c;
    if (above < (uint32_t)krem && (uint32_t)krem <= above + c) {
      uint32_t run = above;
      for (int i = per - 1; i >= 0; --i) {
        const int bi = tid * per + i;
        const uint32_t hcount = bi < nb ? sh.hist[bi] : 0u;
        if (run + hcount >= (uint32_t)krem) {
          sh.misc[0] = (uint32_t)bi;
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
  const uint32_t T = lo + prefix;        // the k-th largest key
  const uint32_t keq = (uint32_t)krem;   // keys equal to T to keep (>= 1)

  // ---- ordered output: wave w owns indices [w*cw, (w+1)*cw), walked 64 at a time ----
  constexpr int NW = NT / 64;
  const int cw = (n + NW * 64 - 1) / (NW * 64) * 64;
  const int w0 = min(n, w * cw), w1 = min(n, w0 + cw);
  uint32_t cg = 0, ce = 0;   // this wave's keys above T and equal to T
  each_key_wave<B>(key, w0, w1, [&](int, bool valid, uint32_t x) {
    cg += (uint32_t)__popcll(__ballot(valid && x > T));
    ce += (uint32_t)__popcll(__ballot(valid && x == T));
  });
  if (lane == 0) {
    sh.w1[w] = cg;
    sh.w2[w] = ce;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int i = 0; i < w; ++i) {
    gt_before += sh.w1[i];
    eq_before += sh.w2[i];
  }
  const uint64_t lt = (1ull << lane) - 1ull;   // lanes below this one
  // taken keys before this wave: all of its larger keys and the equal keys up to keq
  uint32_t pos = gt_before + (eq_before < keq ? eq_before : keq);
  uint32_t eq_seen = eq_before;
  each_key_wave<B>(key, w0, w1, [&](int i, bool valid, uint32_t x) {
    const bool eq = valid && x == T;
    const uint64_t me = __ballot(eq);
    const bool take = valid && (x > T || (eq && eq_seen + (uint32_t)__popcll(me & lt) < keq));
    const uint64_t mt = __ballot(take);
    if (take) {
      const uint32_t p = pos + (uint32_t)__popcll(mt & lt);
      if (p < (uint32_t)k) dst[p] = i;
    }
    pos += (uint32_t)__popcll(mt);
    eq_seen += (uint32_t)__popcll(me);
  });
}

}  // namespace kvsel
