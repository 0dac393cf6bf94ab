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

// Cold rows of n <= NT * C keys (no warm start): the keys stay in registers
// from the load to the output, so no pass reads or writes them in LDS.
// Thread t holds keys t + j*NT (j < C): for each j the 64 lanes of a wave
// hold 64 consecutive indices, which is what the ballot-based collection and
// the ordered output need.  The selection is that of radix_find: digit
// passes (11 bits, from the top of the row's key range) until the bin
// holding the k-th largest key has at most kListCap keys, which are then
// collected and ranked.  The output counts each 64-key chunk's keys above T
// and equal to T, scans the counts in index order, and each wave writes its
// chosen indices: ascending, and the equal keys taken are the lowest-indexed.
template <int NT, int C>
__global__ __launch_bounds__(NT) void topk_regs_kernel(TopkArgs a) {
  constexpr int NW = NT / 64;
  static_assert(C * NW <= NT, "one chunk count per participant in the output scan");
  __shared__ RadixShared<NT> sh;
  __shared__ uint32_t s_cg[C * NW], s_ce[C * NW];
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float *src = a.scores + (size_t)row * a.ld;
  const int n = a.n_row != nullptr ? clampi(a.n_row[row], 0, a.n) : a.n;
  int32_t *dst = a.idx + (size_t)row * a.k;
  BlockSync<NT> grp;
  if (n <= a.k) {   // every candidate kept
    for (int i = t; i < a.k; i += NT) dst[i] = i < n ? i : -1;
    return;
  }
  uint32_t x[C];
  {
    float v[C];
#pragma unroll
    for (int j = 0; j < C; ++j) v[j] = src[min(t + j * NT, n - 1)];   // unbranched reads, all in flight
#pragma unroll
    for (int j = 0; j < C; ++j) x[j] = okey(v[j]);
  }
  auto valid = [&](int j) { return t + j * NT < n; };
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    lo = valid(j) ? min(lo, x[j]) : lo;
    hi = valid(j) ? max(hi, x[j]) : hi;
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.w1[w] = lo;
    sh.w2[w] = hi;
  }
  grp.sync();
  lo = 0xffffffffu;
  hi = 0u;
  for (int i = 0; i < NW; ++i) {
    lo = min(lo, sh.w1[i]);
    hi = max(hi, sh.w2[i]);
  }
  grp.sync();

  // ---- the k-th largest key T, and keq: how many keys equal to T are taken ----
  const uint32_t range = hi - lo;
  int top = range == 0u ? 0 : 32 - __clz(range);
  uint32_t prefix = 0, pmask = 0;   // digits of (key - lo) fixed so far
  uint32_t krem = (uint32_t)a.k;    // keys still to take inside the prefix's bin
  uint32_t nin = (uint32_t)n;       // keys in the prefix's bin
  while (top > 0 && nin > (uint32_t)kListCap) {
    const int bits = top < 11 ? top : 11;
    const int shift = top - bits;
    const int nb = 1 << bits;
    for (int i = t; i < nb; i += NT) sh.hist[i] = 0;
    grp.sync();
    // keys of the bin: x - base below 2^span; the others add to this lane's
    // sink word (no branch around the add)
    const uint32_t base = lo + prefix;
    const int span = shift + bits;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const uint32_t d = x[j] - base;
      const bool in = valid(j) && (span >= 32 || (d >> span) == 0u);
      atomicAdd(in ? &sh.hist[d >> shift] : &sh.sink[lane], 1u);
    }
    grp.sync();
    pick_bin<NT>(grp, sh, nb, krem);
    grp.sync();
    prefix |= sh.misc[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem -= sh.misc[1];
    nin = sh.misc[2];
    top -= bits;
    grp.sync();
  }
  const uint64_t below = (1ull << lane) - 1ull;   // lanes below this one
  uint32_t T, keq;
  if (top == 0) {
    T = lo + prefix;   // every digit fixed: the bin is one key value
    keq = krem;
  } else {
    // collect the bin's keys (at most kListCap): each wave counts its matches
    // from ballots, takes their slots with one add, then writes them
    list_reset<NT>(grp, sh);
    grp.sync();
    auto in_bin = [&](int j) { return valid(j) && ((x[j] - lo) & pmask) == prefix; };
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) cnt += (uint32_t)__popcll(__ballot(in_bin(j)));
    if (cnt != 0u) {
      uint32_t slot0 = 0;
      if (lane == 0) slot0 = atomicAdd(&sh.misc[3], cnt);
      slot0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot0);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const bool m = in_bin(j);
        const uint64_t mask = __ballot(m);
        const uint32_t slot = slot0 + (uint32_t)__popcll(mask & below);
        if (m && slot < (uint32_t)kListCap) {
          sh.list_key[slot] = x[j];
          sh.list_idx[slot] = t + j * NT;
        }
        slot0 += (uint32_t)__popcll(mask);
      }
    }
    grp.sync();
    if (t == 0) KVSEL_CHECK(sh.misc[3] <= (uint32_t)kListCap, kDbgCount, sh.misc[3]);
    const RadixT r = rank_list<NT>(grp, sh, min((int)sh.misc[3], kListCap), krem);
    T = r.T;
    keq = r.keq;
  }

  // ---- ordered output: chunk q = j*NW + w holds indices j*NT + 64w + [0, 64) ----
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const uint32_t g = (uint32_t)__popcll(__ballot(valid(j) && x[j] > T));
    const uint32_t e = (uint32_t)__popcll(__ballot(valid(j) && x[j] == T));
    if (lane == 0) {
      s_cg[j * NW + w] = g;
      s_ce[j * NW + w] = e;
    }
  }
  grp.sync();
  {
    const uint32_t g = t < C * NW ? s_cg[t] : 0u, e = t < C * NW ? s_ce[t] : 0u;
    uint32_t gb, eb;
    excl_scan2<NT>(grp, g, e, sh.w1, sh.w2, gb, eb);
    if (t < C * NW) {
      s_cg[t] = gb;
      s_ce[t] = eb;
    }
  }
  grp.sync();
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const uint32_t gb = s_cg[j * NW + w], eb = s_ce[j * NW + w];   // before this chunk
    const bool eq = valid(j) && x[j] == T;
    const uint64_t em = __ballot(eq);
    const bool take = valid(j) && (x[j] > T || (eq && eb + (uint32_t)__popcll(em & below) < keq));
    const uint64_t tm = __ballot(take);
    const uint32_t slot = gb + (eb < keq ? eb : keq) + (uint32_t)__popcll(tm & below);
    KVSEL_CHECK(!take || slot < (uint32_t)a.k, kDbgOutSlot, slot);
    if (take) dst[slot] = t + j * NT;
  }
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
  if (a.warm == nullptr && a.n <= 32 * 1024) {   // cold rows: keys held in registers
    const dim3 g(a.rows), blk(1024);
    if (a.n <= 4 * 1024)
      hipLaunchKernelGGL((topk_regs_kernel<1024, 4>), g, blk, 0, s, a);
    else if (a.n <= 8 * 1024)
      hipLaunchKernelGGL((topk_regs_kernel<1024, 8>), g, blk, 0, s, a);
    else if (a.n <= 16 * 1024)
      hipLaunchKernelGGL((topk_regs_kernel<1024, 16>), g, blk, 0, s, a);
    else
      hipLaunchKernelGGL((topk_regs_kernel<1024, 32>), g, blk, 0, s, a);
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
