// Exact top-k of one row held as order-preserving uint32 keys: ties to the
// lower index, output ascending.
//
// The selection runs on a group of NTS threads (whole waves) with its own
// barrier: a whole work-group (BlockSync) or a set of waves inside a
// work-group whose other waves keep streaming (WaveSetSync).
//
// The k-th largest key T is found by a radix select over (key - lo), where lo
// and hi bound the candidate keys: the digits (11 bits, from the top of the
// candidates' range down) spread over the range the row occupies, because the
// scores of one softmax share a few float exponents and digits taken from the
// raw key would pile nearly every key into a handful of histogram bins
// (serialised LDS atomics).  Once the bin holding T has at most kListCap
// candidates they are collected into LDS and ranked exactly, which replaces
// the remaining digit passes.  The output pass gives each thread a contiguous
// range of indices: the threads count their keys > T and == T, exclusive
// scans place them, and each writes its chosen indices in order -- so the
// output is ascending and ties go to the lower index.  Only keys >=
// theta are ranked; theta must not exceed the k-th largest key (a warm start's
// minimum does not: at least k keys reach it).
#pragma once

#include "common.h"

namespace kvsel {

// float -> uint32 with the same order (negative floats below positive ones)
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// candidates of the digit bin holding T collected for an exact rank
constexpr int kListCap = 256;

template <int NTS>
struct RadixShared {
  uint32_t hist[2048];
  uint32_t sink[64];   // the histogram passes' adds of keys outside the bin (never read)
  uint32_t w1[NTS / 64];
  uint32_t w2[NTS / 64];
  uint32_t w3[NTS / 64];
  uint32_t misc[8];
  alignas(16) uint32_t list_key[kListCap];   // read four at a time by the rank
  alignas(16) int32_t list_idx[kListCap];
};

// All threads of the work-group take part.
template <int NTS>
struct BlockSync {
  __device__ int t() const { return (int)threadIdx.x; }
  __device__ void sync() const { __syncthreads(); }
};

// NTS / 64 waves of a work-group take part (rank = the wave's place in the
// set); they meet on an LDS counter that only grows.  Every wave of the set
// calls sync() equally often, so each wait ends once the last of them has
// arrived; waves outside the set never wait on it.  The fences order LDS only
// (the set shares data through LDS), so a wait never includes the wave's
// outstanding global loads or stores.
template <int NTS>
struct WaveSetSync {
  int rank;
  uint32_t *ctr;
  uint32_t target;
  __device__ int t() const { return rank * 64 + (int)(threadIdx.x & 63); }
  __device__ void sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    target += NTS / 64;
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while ((uint32_t)__builtin_amdgcn_readfirstlane(
               (int)__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < target)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
};

// exclusive scan of one value per participant in participant order; total
// returned.  ws holds NTS / 64 words.
template <int NTS, typename Grp>
__device__ __forceinline__ uint32_t excl_scan(Grp &grp, uint32_t v, uint32_t *ws, uint32_t &total) {
  const int t = grp.t(), w = t >> 6;
  const uint32_t x = wave_incl_scan_u32(v);
  if ((t & 63) == 63) ws[w] = x;
  grp.sync();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NTS / 64; ++i) {
    const uint32_t s = ws[i];
    pre += i < w ? s : 0u;
    tot += s;
  }
  grp.sync();
  total = tot;
  return pre + x - v;
}

// exclusive scans of two values per participant (one pair of barriers)
template <int NTS, typename Grp>
__device__ __forceinline__ void excl_scan2(Grp &grp, uint32_t a, uint32_t b, uint32_t *wa, uint32_t *wb,
                                           uint32_t &pa, uint32_t &pb) {
  const int t = grp.t(), w = t >> 6;
  const uint32_t xa = wave_incl_scan_u32(a), xb = wave_incl_scan_u32(b);
  if ((t & 63) == 63) {
    wa[w] = xa;
    wb[w] = xb;
  }
  grp.sync();
  uint32_t sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NTS / 64; ++i) {
    sa += i < w ? wa[i] : 0u;
    sb += i < w ? wb[i] : 0u;
  }
  grp.sync();
  pa = sa + xa - a;
  pb = sb + xb - b;
}

// f(i, key(i)) for i = t, t + NTS, ... below n; each thread issues B key
// reads before using them (one memory latency per B keys).  The reads past n
// read key n - 1 instead of being skipped: a read under a branch would be
// waited for before the next one is issued.
template <int NTS, int B, typename KeyFn, typename F>
__device__ __forceinline__ void each_key(int t, KeyFn key, int n, F f) {
  for (int base = 0; base < n; base += B * NTS) {
    uint32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) x[j] = key(min(base + j * NTS + t, n - 1));
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * NTS + t;
      if (i < n) f(i, x[j]);
    }
  }
}

// the calling wave walks [i0, i1) 64 consecutive keys at a time:
// f(i, valid, key) in every lane, the same number of calls in each lane
// (reads past i1 read key i1 - 1, unbranched, as in each_key)
template <int B, typename KeyFn, typename F>
__device__ __forceinline__ void each_key_wave(KeyFn key, int i0, int i1, F f) {
  const int lane = threadIdx.x & 63;
  for (int base = i0; base < i1; base += B * 64) {
    uint32_t x[B];
#pragma unroll
    for (int j = 0; j < B; ++j) x[j] = key(min(base + j * 64 + lane, i1 - 1));
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int b2 = base + j * 64;
      if (b2 < i1) f(b2 + lane, b2 + lane < i1, x[j]);
    }
  }
}

// theta from a warm selection: the smallest key at the warm indices, or 0 (rank
// everything) if they are not strictly ascending and inside [0, n).
template <int NTS, typename Grp, typename KeyFn>
__device__ uint32_t warm_theta(Grp &grp, KeyFn key, const int32_t *wi, int n, int k, RadixShared<NTS> &sh) {
  const int t = grp.t(), w = t >> 6;
  uint32_t bad = 0, mn = 0xffffffffu;
  for (int j = t; j < k; j += NTS) {
    const int x = wi[j];
    if (x < 0 || x >= n) {
      bad = 1;
    } else {
      if (j + 1 < k && wi[j + 1] <= x) bad = 1;
      mn = min(mn, key(x));
    }
  }
  bad = wave_max_u32(bad);
  mn = wave_min_u32(mn);
  if ((t & 63) == 0) {
    sh.w1[w] = bad;
    sh.w2[w] = mn;
  }
  grp.sync();
  uint32_t b2 = 0, m2 = 0xffffffffu;
  for (int i = 0; i < NTS / 64; ++i) {
    b2 |= sh.w1[i];
    m2 = min(m2, sh.w2[i]);
  }
  grp.sync();
  return b2 ? 0u : m2;
}

// lo, hi and the count of the keys >= theta (hi < lo when there are none)
template <int NTS, typename Grp, typename KeyFn>
__device__ void key_range(Grp &grp, KeyFn key, int n, uint32_t theta, uint32_t &lo, uint32_t &hi, uint32_t &ncand,
                          RadixShared<NTS> &sh) {
  const int t = grp.t(), w = t >> 6;
  uint32_t l = 0xffffffffu, h = 0u, c = 0u;
  each_key<NTS, 8>(t, key, n, [&](int, uint32_t x) {
    if (x >= theta) {
      l = min(l, x);
      h = max(h, x);
      ++c;
    }
  });
  l = wave_min_u32(l);
  h = wave_max_u32(h);
  c = wave_reduce_u32(c, [](uint32_t a, uint32_t b) { return a + b; });
  if ((t & 63) == 0) {
    sh.w1[w] = l;
    sh.w2[w] = h;
    sh.w3[w] = c;
  }
  grp.sync();
  lo = 0xffffffffu;
  hi = 0u;
  ncand = 0u;
  for (int i = 0; i < NTS / 64; ++i) {
    lo = min(lo, sh.w1[i]);
    hi = max(hi, sh.w2[i]);
    ncand += sh.w3[i];
  }
  grp.sync();
}

struct RadixT {
  uint32_t T, keq;
};

// After a histogram pass over nb bins (bin nb - 1 the highest): the bin
// holding the krem-th largest of the counted keys.  Participant t owns bins
// [t*per, (t+1)*per); the one whose bins hold that key writes sh.misc[0] =
// the bin, misc[1] = the keys in the bins above it, misc[2] = the keys in it,
// which the participants read after their next sync.
template <int NTS, typename Grp>
__device__ __forceinline__ void pick_bin(Grp &grp, RadixShared<NTS> &sh, int nb, uint32_t krem) {
  const int t = grp.t();
  const int per = (nb + NTS - 1) / NTS;
  uint32_t c = 0;
  for (int i = 0; i < per; ++i) {
    const int bi = t * per + i;
    c += bi < nb ? sh.hist[bi] : 0u;
  }
  uint32_t total;
  const uint32_t below = excl_scan<NTS>(grp, c, sh.w1, total);
  const uint32_t above = total - below - c;   // candidates in bins above this participant's
  if (above < krem && krem <= above + c) {
    uint32_t run = above;
    for (int i = per - 1; i >= 0; --i) {
      const int bi = t * per + i;
      const uint32_t hcount = bi < nb ? sh.hist[bi] : 0u;
      if (run + hcount >= krem) {
        sh.misc[0] = (uint32_t)bi;
        sh.misc[1] = run;
        sh.misc[2] = hcount;
        break;
      }
      run += hcount;
    }
  }
}

// An empty candidate list: its count is zero, and slots past the collected
// ones rank below every candidate (key 0, last index).  The caller syncs
// before collecting.
template <int NTS, typename Grp>
__device__ __forceinline__ void list_reset(Grp &grp, RadixShared<NTS> &sh) {
  const int t = grp.t();
  if (t == 0) sh.misc[3] = 0;
  for (int i = t; i < kListCap; i += NTS) {
    sh.list_key[i] = 0u;
    sh.list_idx[i] = 0x7fffffff;
  }
}

// The krem-th of the nl collected candidates in (key descending, index
// ascending) order: its key T, and keq = krem minus the candidates with a
// larger key (how many keys equal to T are taken).  The rank of item j is the
// number of items with a larger key, or an equal key and a lower index.  Four
// adjacent participants take item j, each a quarter of the list (four items
// per LDS access, several in flight), and add their counts with two lane
// exchanges.  Ends with sh free again.
template <int NTS, typename Grp>
__device__ __forceinline__ RadixT rank_list(Grp &grp, RadixShared<NTS> &sh, int nl, uint32_t krem) {
  const int t = grp.t();
  const int nl4 = (nl + 3) & ~3;   // whole groups of four (the padding ranks below everything)
  for (int jj = t; jj < 4 * nl; jj += NTS) {
    const int j = jj >> 2, q = jj & 3;
    const uint32_t xj = sh.list_key[j];
    const int ij = sh.list_idx[j];
    uint32_t r = 0, gt = 0;
#pragma unroll 2
    for (int i = 4 * q; i < nl4; i += 16) {
      const uint4 xi = *reinterpret_cast<const uint4 *>(&sh.list_key[i]);
      const int4 ii = *reinterpret_cast<const int4 *>(&sh.list_idx[i]);
      gt += (xi.x > xj ? 1u : 0u) + (xi.y > xj ? 1u : 0u) + (xi.z > xj ? 1u : 0u) + (xi.w > xj ? 1u : 0u);
      r += ((xi.x > xj || (xi.x == xj && ii.x < ij)) ? 1u : 0u) + ((xi.y > xj || (xi.y == xj && ii.y < ij)) ? 1u : 0u) +
           ((xi.z > xj || (xi.z == xj && ii.z < ij)) ? 1u : 0u) + ((xi.w > xj || (xi.w == xj && ii.w < ij)) ? 1u : 0u);
    }
    r += (uint32_t)__shfl_xor((int)r, 1);
    r += (uint32_t)__shfl_xor((int)r, 2);
    gt += (uint32_t)__shfl_xor((int)gt, 1);
    gt += (uint32_t)__shfl_xor((int)gt, 2);
    if (q == 0 && r == krem - 1u) {
      sh.misc[4] = xj;
      sh.misc[5] = krem - gt;
    }
  }
  grp.sync();
  const RadixT res{sh.misc[4], sh.misc[5]};
  grp.sync();   // sh is free again
  return res;
}

// The k-th largest key T among the candidates (keys >= theta) of key(i), i in
// [0, n), and keq, how many keys equal to T the top k hold (>= 1); n > k >= 1.
// lo <= every candidate key <= hi, and nin >= the number of candidates (at
// least k of them).  LDS_KEYS: key(i) reads LDS; otherwise global memory,
// with more reads in flight per lane.  LIST: the digit passes stop once the
// bin holding T has at most this many candidates, which are then collected
// and ranked (0: digit passes until T is known, for keys whose passes are
// cheap).  Ends with sh free again.
template <int NTS, bool LDS_KEYS = true, int LIST = kListCap, typename Grp, typename KeyFn>
__device__ RadixT radix_find(Grp &grp, KeyFn key, int n, int k, uint32_t theta, uint32_t lo, uint32_t hi, uint32_t nin,
                             RadixShared<NTS> &sh) {
  static_assert(LIST >= 0 && LIST <= kListCap, "the candidate list holds kListCap keys");
  constexpr int B = LDS_KEYS ? 8 : 32;
  constexpr int NW = NTS / 64;
  const int t = grp.t(), lane = t & 63, w = t >> 6;
  const uint32_t range = hi - lo;
  int top = range == 0u ? 0 : 32 - __clz(range);
  uint32_t prefix = 0, pmask = 0;   // digits of (key - lo) fixed so far
  uint32_t krem = (uint32_t)k;      // keys still to take inside the prefix's bin
  auto in_bin = [&](uint32_t x) { return x >= theta && ((x - lo) & pmask) == prefix; };

  // ---- digit passes until the bin holding T is small ----
  while (top > 0 && nin > (uint32_t)LIST) {
    const int bits = top < 11 ? top : 11;
    const int shift = top - bits;
    const int nb = 1 << bits;
    for (int i = t; i < nb; i += NTS) sh.hist[i] = 0;
    grp.sync();
    // a key of the bin: x - base below 2^span (any key when span reaches 32);
    // every key adds one, those outside the bin to this lane's sink word (no
    // branch around the add)
    const uint32_t base = lo + prefix;
    const int span = shift + bits;
    each_key<NTS, B>(t, key, n, [&](int, uint32_t x) {
      const uint32_t d = x - base;
      const bool in = x >= theta && (span >= 32 || (d >> span) == 0u);
      atomicAdd(in ? &sh.hist[d >> shift] : &sh.sink[lane], 1u);
    });
    grp.sync();
    pick_bin<NTS>(grp, sh, nb, krem);
    grp.sync();
    prefix |= sh.misc[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem -= sh.misc[1];
    nin = sh.misc[2];
    top -= bits;
    grp.sync();
  }

  uint32_t T, keq;
  if (top == 0) {
    T = lo + prefix;   // every digit fixed: the bin is one key value
    keq = krem;
  } else {
    // ---- at most kListCap candidates left in the bin: collect and rank them ----
    list_reset<NTS>(grp, sh);
    grp.sync();
    {
      // wave w walks its contiguous range 64 keys at a time, B chunks per
      // batch: the batch's matches counted from ballots, their slots taken
      // with one add to the counter, then written
      const int cw = (n + NW * 64 - 1) / (NW * 64) * 64;
      const int w0 = min(n, w * cw), w1 = min(n, w0 + cw);
      const uint64_t below = (1ull << lane) - 1ull;
      for (int b0 = w0; b0 < w1; b0 += B * 64) {
        uint32_t x[B];
#pragma unroll
        for (int j = 0; j < B; ++j) x[j] = key(min(b0 + j * 64 + lane, w1 - 1));   // unbranched reads
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < B; ++j) cnt += (uint32_t)__popcll(__ballot(b0 + j * 64 + lane < w1 && in_bin(x[j])));
        if (cnt == 0u) continue;
        uint32_t slot0 = 0;
        if (lane == 0) slot0 = atomicAdd(&sh.misc[3], cnt);
        slot0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot0);
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const int i = b0 + j * 64 + lane;
          const bool m = i < w1 && in_bin(x[j]);
          const uint64_t mask = __ballot(m);
          const uint32_t slot = slot0 + (uint32_t)__popcll(mask & below);
          if (m && slot < (uint32_t)kListCap) {
            sh.list_key[slot] = x[j];
            sh.list_idx[slot] = i;
          }
          slot0 += (uint32_t)__popcll(mask);
        }
      }
    }
    grp.sync();
    // the digit passes stopped at a bin of at most LIST keys: all of them collected
    if (grp.t() == 0) KVSEL_CHECK(sh.misc[3] <= (uint32_t)kListCap, kDbgCount, sh.misc[3]);
    const RadixT r = rank_list<NTS>(grp, sh, min((int)sh.misc[3], kListCap), krem);
    T = r.T;
    keq = r.keq;
  }
  return RadixT{T, keq};
}

// The k largest of key(i), i in [0, n), among the candidates (keys >= theta),
// written ascending to dst; arguments as for radix_find.  Output, keys in
// global memory: per-wave ranges walked 64 consecutive keys at a time, so
// that the reads coalesce and each wave's chosen indices leave in contiguous
// runs.  Keys in LDS: per-participant ranges of C keys (C odd: the lanes of a
// wave read different banks); with stage (the LDS array the keys live in,
// writable once they are read) and C <= STAGE_C, each participant holds its
// keys in registers (read once for the count and the output) while the
// chosen indices are placed in that array, which is then copied out in order
// (coalesced).
template <int NTS, bool LDS_KEYS = true, int STAGE_C = 0, int LIST = kListCap, typename Grp, typename KeyFn>
__device__ void radix_select(Grp &grp, KeyFn key, int n, int k, uint32_t theta, uint32_t lo, uint32_t hi, uint32_t nin,
                             int32_t *dst, RadixShared<NTS> &sh, uint32_t *stage = nullptr) {
  constexpr int B = LDS_KEYS ? 8 : 32;
  constexpr int NW = NTS / 64;
  const int t = grp.t(), lane = t & 63, w = t >> 6;
  const RadixT found = radix_find<NTS, LDS_KEYS, LIST>(grp, key, n, k, theta, lo, hi, nin, sh);
  const uint32_t T = found.T, keq = found.keq;
  if constexpr (LDS_KEYS) {
    // ---- ordered output: participant t owns the indices [t*C, (t+1)*C) ----
    // It counts its keys above T and equal to T, the exclusive scans of those
    // counts place it, and it takes its chosen indices in order: ascending
    // output, and the equal keys taken are the lowest-indexed keq.
    const int C = ((n + NTS - 1) / NTS) | 1;
    const int i0 = min(n, t * C), i1 = min(n, i0 + C);
    if (STAGE_C > 0 && stage != nullptr && C <= STAGE_C) {
      // the participant's keys read once, into registers
      constexpr int SC = STAGE_C > 0 ? STAGE_C : 1;
      uint32_t x[SC];
#pragma unroll
      for (int j = 0; j < SC; ++j) x[j] = key(min(i0 + j, n - 1));
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        cg += (i0 + j < i1 && x[j] > T) ? 1u : 0u;
        ce += (i0 + j < i1 && x[j] == T) ? 1u : 0u;
      }
      uint32_t gt_before, eq_before;
      // (its barriers also free the key array: every participant has read its keys)
      excl_scan2<NTS>(grp, cg, ce, sh.w1, sh.w2, gt_before, eq_before);
      uint32_t pos = gt_before + (eq_before < keq ? eq_before : keq);
      uint32_t eq_seen = eq_before;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        if (i0 + j < i1) {
          bool take = x[j] > T;
          if (x[j] == T) {
            take = eq_seen < keq;
            ++eq_seen;
          }
          if (take) {
            KVSEL_CHECK(pos < (uint32_t)k, kDbgOutSlot, pos);
            stage[pos++] = (uint32_t)(i0 + j);
          }
        }
      }
      grp.sync();
      for (int i = t; i < k; i += NTS) dst[i] = (int32_t)stage[i];
      grp.sync();   // sh is free again
      return;
    }
    uint32_t cg = 0, ce = 0;
    for (int b0 = i0; b0 < i1; b0 += B) {
      uint32_t x[B];
#pragma unroll
      for (int j = 0; j < B; ++j) x[j] = key(min(b0 + j, n - 1));
#pragma unroll
      for (int j = 0; j < B; ++j) {
        cg += (b0 + j < i1 && x[j] > T) ? 1u : 0u;
        ce += (b0 + j < i1 && x[j] == T) ? 1u : 0u;
      }
    }
    uint32_t gt_before, eq_before;
    excl_scan2<NTS>(grp, cg, ce, sh.w1, sh.w2, gt_before, eq_before);
    uint32_t pos = gt_before + (eq_before < keq ? eq_before : keq);
    uint32_t eq_seen = eq_before;
    {
      for (int b0 = i0; b0 < i1; b0 += B) {
        uint32_t x[B];
#pragma unroll
        for (int j = 0; j < B; ++j) x[j] = key(min(b0 + j, n - 1));
#pragma unroll
        for (int j = 0; j < B; ++j) {
          if (b0 + j < i1) {
            bool take = x[j] > T;
            if (x[j] == T) {
              take = eq_seen < keq;
              ++eq_seen;
            }
            if (take) {
              KVSEL_CHECK(pos < (uint32_t)k, kDbgOutSlot, pos);
              if (pos < (uint32_t)k) dst[pos] = b0 + j;
              ++pos;
            }
          }
        }
      }
    }
  } else {
    // ---- ordered output: wave w owns indices [w*cw, (w+1)*cw), walked 64 at a time ----
    // The waves count their keys above T and equal to T, and each then places
    // its chosen indices in order with ballot masks.
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
    grp.sync();
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
        KVSEL_CHECK(p < (uint32_t)k, kDbgOutSlot, p);
        if (p < (uint32_t)k) dst[p] = i;
      }
      pos += (uint32_t)__popcll(mt);
      eq_seen += (uint32_t)__popcll(me);
    });
  }
  grp.sync();   // sh is free again
}

// Top-k of a whole row with a block of NTS threads: warm theta (optional),
// candidate range, radix select.  When n <= k all n indices are kept,
// followed by -1.  LDS_KEYS as for radix_select.
template <int NTS, bool LDS_KEYS = true, int STAGE_C = 0, int LIST = kListCap, typename Grp, typename KeyFn>
__device__ void radix_topk(Grp &grp, KeyFn key, int n, int k, const int32_t *warm, int32_t *dst, RadixShared<NTS> &sh,
                           uint32_t *stage = nullptr) {
  const int t = grp.t();
  if (n <= k) {
    for (int i = t; i < k; i += NTS) dst[i] = i < n ? i : -1;
    return;
  }
  const uint32_t theta = warm != nullptr ? warm_theta<NTS>(grp, key, warm, n, k, sh) : 0u;
  uint32_t lo, hi, ncand;
  key_range<NTS>(grp, key, n, theta, lo, hi, ncand, sh);
  radix_select<NTS, LDS_KEYS, STAGE_C, LIST>(grp, key, n, k, theta, lo, hi, ncand, dst, sh, stage);
}

}  // namespace kvsel
