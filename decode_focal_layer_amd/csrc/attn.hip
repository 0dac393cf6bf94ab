// Split-KV decode attention over a paged bf16 cache, dense or over a
// gathered row set, with an optional fused output of the raw q.k logits
// that the focal score is computed from.
//
// FastOCR (technical summary, Focal-Guided Pruning): focal layers attend over
// the full cache and choose from that attention; every other layer attends
// only over the pruned set.  FastKV section 2B: decode over the retained KV.
//
// Work decomposition:
//  * grid = (splits, kv heads, sequences).  When there are enough (sequence,
//    kv head) pairs to fill the chip, each pair gets one large work-group and
//    writes its output directly; otherwise the pair's "virtual rows" (the kept
//    rows, then the always-attended rows before and after the candidate
//    segment; or every row for dense attention) are split over several
//    work-groups whose partial (max, sum, accumulator) records are merged by
//    the last of them to finish.  No work-group waits on another.
//  * prologue: the work-group resolves its rows to physical cache rows
//    (index -> block table -> block) into LDS once, so the streaming loop
//    issues only K/V loads.
//  * a lane group of 16 lanes owns one row at a time: a lane holds 8 of the
//    128 dims (one 16-byte load per K row and per V row, so a wave reads four
//    consecutive 256-byte rows per load instruction), the 16-lane dot product
//    is reduced with DPP row operations, and each lane group keeps its own
//    online-softmax state (max, sum, 8 accumulator dims per query head of the
//    group), so the loop has no cross-group synchronisation.
//  * rows are handed out in chunks of 4*U consecutive rows per wave from an
//    LDS counter.  The hardware issues older waves' loads first, so a static
//    split leaves the younger waves (and with them the CU's memory traffic)
//    trailing by a quarter of the loop; taking the next chunk on demand ends
//    every wave within one chunk of the others.  The chunk a wave gets varies
//    from run to run, so the output's rounding (not its row set) may too.
//    Deterministic launches (a.det) give wave w the chunks w, w + waves, ...
//    instead: the same sums in the same order on every run.
//  * the lane-group states are merged in registers (the four groups of a
//    wave) and in LDS (across waves).
#include <type_traits>

#include "common.h"
#include "focal.h"
#include "kvsel_internal.h"
#include "radix.h"

// Launch shape (defaults chosen by measurement on MI355X; overridable at build
// time for sweeps): threads per work-group for groups of <= 2 query heads,
// rows per lane group per loop iteration, and resident waves per CU the split
// count aims for.
#ifndef KVSEL_ATTN_NT2
#define KVSEL_ATTN_NT2 1024
#endif
#ifndef KVSEL_ATTN_U
#define KVSEL_ATTN_U 4
#endif
#ifndef KVSEL_ATTN_WAVES_PER_CU
#define KVSEL_ATTN_WAVES_PER_CU 16
#endif
// split records merged by the last work-group of each pair (1) or by a
// second kernel (0)
#ifndef KVSEL_ATTN_FUSED_MERGE
#define KVSEL_ATTN_FUSED_MERGE 1
#endif
// minimum resident waves per SIMD the compiler must allow for (0: no bound)
#ifndef KVSEL_ATTN_WPE
#define KVSEL_ATTN_WPE 0
#endif

namespace kvsel {

namespace {

constexpr int kTabLds = 2048;   // block tables up to this many entries are staged in LDS

struct SeqView {
  int n, s0, s1, nR;
};

// bounds of sequence b from its raw seq_len / segment values, clamped
__device__ __forceinline__ SeqView seq_view_of(const AttnArgs &a, int n_raw, int s0_raw, int s1_raw, bool dense) {
  SeqView v;
  const int cap = a.max_blocks * kBlk;
  v.n = clampi(n_raw, 0, cap);
  v.s0 = clampi(s0_raw, 0, v.n);
  v.s1 = clampi(s1_raw, v.s0, v.n);
  v.nR = dense ? v.n : (a.k + v.s0 + (v.n - v.s1));
  return v;
}

// The first virtual row from which every row is this sequence's own (past the
// rows shared across sequences, a.shared_rows > 0): those are read once and
// may be streamed past the caches.  Virtual rows: dense, the logical rows;
// else the kept segment rows, then [0, s0), then [s1, n).  Kept rows are
// never counted as own here (they come first).
__device__ __forceinline__ int own_rows_from(const AttnArgs &a, const SeqView &v, bool dense) {
  const int sh = a.shared_rows;
  if (dense) return min(sh, v.n);
  if (sh >= v.n) return v.nR;                          // nothing of its own
  if (sh > v.s1) return a.k + v.s0 + (sh - v.s1);      // [s1, sh) shared, then own
  if (sh > v.s0) return a.k + v.s0;                    // [0, s0) shared, [s1, n) own
  return a.k + sh;                                     // [sh, s0) and [s1, n) own
}

__device__ __forceinline__ SeqView seq_view(const AttnArgs &a, int b, bool dense) {
  return seq_view_of(a, a.seq_len[b], a.seg_begin[b], a.seg_end[b], dense);
}

__device__ __forceinline__ uint32_t row_to_phys(const AttnArgs &a, int b, int g, int row) {
  if (row < 0) return kNoRow;
  const int blk = a.block_table[(size_t)b * a.max_blocks + (row >> 4)];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return kNoRow;
  return ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// dot product of 8 bf16 pairs packed in two uint4 (v_dot2_f32_bf16: exact
// bf16 products, fp32 accumulation)
__device__ __forceinline__ float dot8(const uint4 &x, const uint4 &y) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.x), __builtin_bit_cast(bf16x2, y.x), 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.y), __builtin_bit_cast(bf16x2, y.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.z), __builtin_bit_cast(bf16x2, y.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.w), __builtin_bit_cast(bf16x2, y.w), s, false);
  return s;
}

// full 128-dim dots of one row (this lane's 8 dims + 15 others) for each head
template <int G>
__device__ __forceinline__ void dot_rows(const uint4 (&qr)[G], const uint4 &kr, float (&dot)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = row16_sum(dot8(qr[h], kr));
}

// The running max is a lazy reference: it moves only when a row's logit
// exceeds it by more than this many log2 units, so most iterations skip the
// accumulator rescale; probabilities relative to it stay below 2^8.
constexpr float kLazy = 8.f;
constexpr float kNegBig = -1e30f;   // finite "empty" max: 2^(kNegBig - x) == 0, no NaN

#if KVSEL_ATTN_WPE > 0
#define KVSEL_ATTN_OCC __attribute__((amdgpu_waves_per_eu(KVSEL_ATTN_WPE)))
#else
#define KVSEL_ATTN_OCC
#endif

// A split record word, stored and loaded at agent scope: the work-group that
// merges a pair's records may run on another XCD, whose L2 is not coherent
// with this one's for ordinary accesses; agent-scope accesses are (stores
// write through, loads miss a line they cannot trust).
__device__ __forceinline__ void rec_store(float *p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rec_load(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Combine the split records of (sequence b, kv head g) into out / lse:
// thread x < G*128 of the caller's nt threads takes head x / 128, dim x % 128.
template <int G>
__device__ __forceinline__ void merge_records(const AttnArgs &a, int b, int g, int nact, int tid, int nt) {
  if (tid == 0) KVSEL_CHECK(nact >= 0 && nact <= a.nsplit, kDbgCount, nact);
  for (int x = tid; x < G * kD; x += nt) {
    const int h = x / kD, dim = x % kD;
    const size_t hb = (size_t)b * a.hq + g * G + h;
    const float *rec0 = a.rec + hb * a.nsplit * kRec;
    float M = kNegBig;
    // unrolled: the records' loads go out together instead of one per latency
#pragma unroll 8
    for (int sp = 0; sp < nact; ++sp) M = fmaxf(M, rec_load(rec0 + sp * kRec + kD));
    float L = 0.f, A = 0.f;
#pragma unroll 8
    for (int sp = 0; sp < nact; ++sp) {
      const float c = fast_exp2(rec_load(rec0 + sp * kRec + kD) - M);
      L += rec_load(rec0 + sp * kRec + kD + 1) * c;
      A += rec_load(rec0 + sp * kRec + dim) * c;
    }
    if (a.mass != nullptr) {
      if (dim == 0) a.mass[hb] = L > 0.f ? A / L : 0.f;
    } else {
      a.out[hb * kD + dim] = L > 0.f ? A / L : 0.f;
    }
    if (dim == 0 && a.lse != nullptr) a.lse[hb] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

// MODE 0: attention only.  MODE 1: also store the raw logits to the global
// scratch.  MODE 2 (one split only): keep the segment logits in LDS and end
// with the focal selection of this (sequence, kv head).  MODE 3 (dense): the
// share of each head's attention on the candidate segment -- attention whose
// value rows are the segment's indicator, so V is never read; the share is
// dim 0 of that output.  STREAM: K/V rows are
// loaded non-temporally (each is read once), so they do not evict the data
// that is reused from launch to launch (block tables, kept indices, queries);
// off when rows are shared by many sequences (a shared prefix), which should
// stay cached -- then only the chunks made wholly of a sequence's own rows
// (past the shared ones, own_rows_from) are streamed.  Measured on MI355X:
// +8% for C1 decode and C3, and -8% for C4 if the shared prefix were streamed
// too.
template <int G, int NT, int U, int MODE, bool STREAM>
__global__ __launch_bounds__(NT) KVSEL_ATTN_OCC void attn_kernel(AttnArgs a) {
  constexpr int NW = NT / 64;    // waves
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = tid >> 4, sub = tid & 15;
  const bool dense = a.dense != 0;

  __shared__ uint32_t s_prow[kAttnMaxRps];
  __shared__ int32_t s_tab[kTabLds];
  __shared__ float s_acc[NW][G][kD];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ uint32_t s_next;          // next chunk to hand out
  extern __shared__ float s_logit[];   // MODE 2: [G][seg_cap]
  // MODE 2: chunks after the segment, waves done with the segment, the
  // selectors' barrier counter, the per-wave segment maxima
  __shared__ uint32_t s_next2, s_p1done, s_selctr;
  __shared__ float s_wmax[MODE == 2 ? NW : 1][G];
  __shared__ uint32_t s_simd_n[4], s_simd_done[4];   // MODE 2: waves per SIMD, and done with phase 1

  const int start = split * a.rps;
  constexpr int RPT = kAttnMaxRps / NT;
  constexpr int TPT = kTabLds / NT;

  // Prologue.  Every load it needs is issued before any result is used: the
  // sequence bounds, the query, the block table (into LDS when it fits) and
  // the kept indices of this split's rows, read at clamped addresses so that
  // no load waits for another.  Then each virtual row is resolved to its
  // physical row in LDS, and the streaming loop issues only K/V loads.
  const int n_raw = a.seq_len[b], s0_raw = a.seg_begin[b], s1_raw = a.seg_end[b];
  const uint16_t *qbase = a.q + ((size_t)b * a.hq + g * G) * kD + sub * 8;
  uint4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qr[h] = *reinterpret_cast<const uint4 *>(qbase + h * kD);
  const bool tab_lds = a.max_blocks <= kTabLds;
  const int32_t *tab = a.block_table + (size_t)b * a.max_blocks;
  int tv[TPT];
  if (tab_lds) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) tv[i] = tab[min(tid + i * NT, a.max_blocks - 1)];
  }
  int iv[RPT];
  if (!dense && a.k > 0) {   // k = 0: idx may be null and no row is read from it
    const int32_t *ib = a.idx + ((size_t)b * a.hkv + g) * a.k;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      if (i * NT < a.rps) iv[i] = ib[min(start + tid + i * NT, a.k - 1)];
  }
  const SeqView v = seq_view_of(a, n_raw, s0_raw, s1_raw, dense);
  const int cnt = max(0, min(a.rps, v.nR - start));   // rows of this split
  if (tid == 0) KVSEL_CHECK(cnt <= kAttnMaxRps, kDbgLds, cnt);
  // chunks starting at or past this split-local row hold only rows read once
  // (all of them when STREAM)
  const int own_from = STREAM ? 0 : own_rows_from(a, v, dense) - start;
  constexpr int CH = 4 * U;              // rows per chunk
  const int nch = (cnt + CH - 1) / CH;   // chunks of this split

  int lo = 0, hi = 0;   // logical rows whose logits are stored, at row - lo (dense only)
  if (MODE == 2) {
    lo = v.s0;
    hi = v.s0 + min(v.s1 - v.s0, a.seg_cap);
  } else if (MODE == 1) {
    if (a.logit_mode == 1) { lo = v.s0; hi = v.s1; }
    else { lo = 0; hi = v.n; }
  } else if (MODE == 3) {   // the segment, whose attention share is measured
    lo = v.s0;
    hi = v.s1;
  }

  if (tab_lds) {
#pragma unroll
    for (int i = 0; i < TPT; ++i)
      if (tid + i * NT < a.max_blocks) s_tab[tid + i * NT] = tv[i];
  }
  if (tid == 0) s_next = NW;   // chunks 0 .. NW-1 start the waves
  int c1 = nch;                // MODE 2: chunks up to the segment's end
  if (MODE == 2) {
    c1 = min(nch, (hi - start + CH - 1) / CH);
    if (tid == 0) {
      s_next2 = c1;
      s_p1done = 0;
      s_selctr = 0;
    }
    if (tid < 4) s_simd_n[tid] = s_simd_done[tid] = 0u;
  }
  __syncthreads();
  // MODE 2: the SIMD this wave runs on (hardware wave id register, SIMD_ID
  // field); only used to spread the selecting waves over the SIMDs
  const uint32_t simd = MODE == 2 ? (uint32_t)__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3u : 0u;
  if (MODE == 2 && lane == 0) atomicAdd(&s_simd_n[simd], 1u);
  // Each virtual row of this split to its physical cache row, in LDS.  The
  // table entries of up to eight of a thread's rows are read unconditionally
  // (a clamped, valid address for a row that is not used) before any of them
  // is, so their latencies overlap instead of adding up.
  constexpr int RG = RPT < 8 ? RPT : 8;
#pragma unroll
  for (int i0 = 0; i0 < RPT; i0 += RG) {
    if (i0 * NT >= a.rps) break;
    int rowv[RG], blkv[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      const int i = i0 + u, t = tid + i * NT;
      int row = -1;
      if (i * NT < a.rps && t < cnt) {
        const int j = start + t;   // virtual row
        if (dense) row = j;
        else if (j < a.k) row = (iv[i] >= 0 && iv[i] < v.s1 - v.s0) ? v.s0 + iv[i] : -1;
        else if (j < a.k + v.s0) row = j - a.k;
        else row = v.s1 + (j - a.k - v.s0);
      }
      rowv[u] = row;
    }
    if (tab_lds) {
#pragma unroll
      for (int u = 0; u < RG; ++u) blkv[u] = s_tab[max(rowv[u], 0) >> 4];
    } else {
#pragma unroll
      for (int u = 0; u < RG; ++u) blkv[u] = tab[max(rowv[u], 0) >> 4];
    }
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      const int i = i0 + u, t = tid + i * NT;
      if (i * NT < a.rps && t < cnt) {
        const int row = rowv[u], blk = blkv[u];
        uint32_t pr = kNoRow;
        if (row >= 0 && blk >= 0 && (int64_t)blk < a.num_blocks)
          pr = ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
        s_prow[t] = pr;
      }
    }
  }

  float m[G], l[G], acc[G][8];
  float smax[G];   // MODE 2: largest segment logit per head seen by this lane group
#pragma unroll
  for (int h = 0; h < G; ++h) {
    smax[h] = -INFINITY;
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  const uint16_t *kbase = a.k_pool + sub * 8;
  const uint16_t *vbase = a.v_pool + sub * 8;

  // Chunk c is rows [c*CH, (c+1)*CH) of this split; lane group grp takes
  // rows c*CH + grp%4 + 4*u, so each load instruction of a wave covers four
  // consecutive rows.
#define KVSEL_ROWT(base, u) ((base) + (grp & 3) + 4 * (u))
  // K/V rows of one chunk into registers; NTL: loaded non-temporally (each row
  // is read once: do not displace reused lines)
  auto load_rows_as = [&](auto nt, int base, uint4 (&kr)[U], uint4 (&vr)[U], bool (&ok)[U]) {
    constexpr bool NTL = decltype(nt)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = KVSEL_ROWT(base, u);
      // unbranched LDS read (a read under a branch is waited for at once)
      const uint32_t pr_t = s_prow[max(min(t, cnt - 1), 0)];
      const uint32_t pr = t < cnt ? pr_t : kNoRow;
      ok[u] = pr != kNoRow;
      KVSEL_CHECK(!ok[u] || (uint64_t)pr < (uint64_t)a.num_blocks * (uint64_t)a.hkv * kBlk, kDbgKvRow, pr);
      // a row that is not attended reads this lane's query (a valid, finite
      // 16 bytes) and gets probability 0
      const uint16_t *kp = ok[u] ? kbase + (size_t)pr * kD : qbase;
      const uint16_t *vp = ok[u] ? vbase + (size_t)pr * kD : qbase;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      if (NTL)
        kr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp)));
      else
        kr[u] = *reinterpret_cast<const uint4 *>(kp);
      if (MODE == 3)
        vr[u] = make_uint4(0u, 0u, 0u, 0u);   // not read
      else if (NTL)
        vr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp)));
      else
        vr[u] = *reinterpret_cast<const uint4 *>(vp);
    }
  };
  // the chunk's rows streamed when they all lie past the shared rows (uniform)
  auto load_rows = [&](int base, uint4 (&kr)[U], uint4 (&vr)[U], bool (&ok)[U]) {
    if (STREAM || base >= own_from)
      load_rows_as(std::true_type{}, base, kr, vr, ok);
    else
      load_rows_as(std::false_type{}, base, kr, vr, ok);
  };
  // online softmax over the chunk's rows
  auto consume = [&](int base, const uint4 (&kr)[U], const uint4 (&vr)[U], const bool (&ok)[U]) {
    float dot[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) dot_rows<G>(qr, kr[u], dot[u]);
    if (MODE == 1 || MODE == 2) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = start + KVSEL_ROWT(base, u);   // dense: logical row = virtual row
        if (MODE == 2 && ok[u] && row >= lo && row < hi) {
#pragma unroll
          for (int h = 0; h < G; ++h) smax[h] = fmaxf(smax[h], dot[u][h]);
        }
        // a segment row of this split whose block is missing is not attended:
        // its logit is -inf (probability 0), so no stale value is ranked
        if (sub < G && KVSEL_ROWT(base, u) < cnt && row >= lo && row < hi) {
          float dv = dot[u][0];
#pragma unroll
          for (int h = 1; h < G; ++h) dv = sub == h ? dot[u][h] : dv;
          if (!ok[u]) dv = -INFINITY;
          if (MODE == 2) {
            KVSEL_CHECK(row - lo < a.seg_cap, kDbgLds, row - lo);
            s_logit[sub * a.seg_cap + (row - lo)] = dv;
          }
          else if (row - lo < a.ld_logits)
            a.logits[((size_t)b * a.hq + g * G + sub) * a.ld_logits + (row - lo)] = dv;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s[U];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = ok[u] ? dot[u][h] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      if (mx > m[h] + kLazy) {   // move the reference (rare after the first rows)
        const float c = fast_exp2(m[h] - mx);
        l[h] *= c;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= c;
        m[h] = mx;
      }
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = fast_exp2(s[u] - m[h]);
        l[h] += p[u];
      }
      if constexpr (MODE == 3) {
        // the indicator row: 1 in dim 0 (lane sub 0) for segment rows
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int row = start + KVSEL_ROWT(base, u);
          acc[h][0] = fmaf(p[u], (sub == 0 && row >= lo && row < hi) ? 1.f : 0.f, acc[h][0]);
        }
        continue;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint4 w = vr[u];
        acc[h][0] = fmaf(p[u], bf_lo(w.x), acc[h][0]);
        acc[h][1] = fmaf(p[u], bf_hi(w.x), acc[h][1]);
        acc[h][2] = fmaf(p[u], bf_lo(w.y), acc[h][2]);
        acc[h][3] = fmaf(p[u], bf_hi(w.y), acc[h][3]);
        acc[h][4] = fmaf(p[u], bf_lo(w.z), acc[h][4]);
        acc[h][5] = fmaf(p[u], bf_hi(w.z), acc[h][5]);
        acc[h][6] = fmaf(p[u], bf_lo(w.w), acc[h][6]);
        acc[h][7] = fmaf(p[u], bf_hi(w.w), acc[h][7]);
      }
    }
  };

  // Chunks c .. cend-1, handed out by *ctr.  A wave leaves once the counter
  // has passed cend: the counter only grows, and a wave takes a new chunk
  // only after finishing one.
  auto run = [&](uint32_t *ctr, int c, int cend) {
    if (a.det) {   // a fixed share per wave (modes 0, 1 and 3 only)
      for (; c < cend; c += NW) {
        uint4 kr[U], vr[U];
        bool ok[U];
        load_rows(c * CH, kr, vr, ok);
        consume(c * CH, kr, vr, ok);
      }
      return;
    }
    while (c < cend) {
      uint32_t nxt = 0;
      if (lane == 0) nxt = atomicAdd(ctr, 1u);   // its latency hides behind the loads
      uint4 kr[U], vr[U];
      bool ok[U];
      load_rows(c * CH, kr, vr, ok);
      consume(c * CH, kr, vr, ok);
      c = __builtin_amdgcn_readfirstlane((int)nxt);
    }
  };
  if constexpr (MODE == 2) {
    // Phase 1: the chunks up to the end of the segment, whose logits the
    // selection needs.  Phase 2: the rest.  The last four waves to finish
    // phase 1 wait for the others, then select while the remaining waves
    // stream phase 2's rows; they join phase 2 when done.  (FastOCR,
    // Focal-Guided Pruning: the focal layer attends over the full cache and
    // selects from that attention.)
    run(&s_next, wave, c1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = wave_max_f(smax[h]);
      if (lane == 0) s_wmax[wave][h] = mx;
    }
    uint32_t ticket = 0, tsimd = 0;
    if (lane == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");   // this wave's logits are in LDS
      ticket = __hip_atomic_fetch_add(&s_p1done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      tsimd = atomicAdd(&s_simd_done[simd], 1u);
    }
    ticket = (uint32_t)__builtin_amdgcn_readfirstlane((int)ticket);
    tsimd = (uint32_t)__builtin_amdgcn_readfirstlane((int)tsimd);
    // Eight selectors: the last two waves of each SIMD to finish phase 1 (two
    // per SIMD, so the selection spreads over all of them) when every SIMD
    // holds at least two of the work-group's waves, else the last eight waves
    // to finish.
    constexpr int NSEL = kStatThreads / 64;
    static_assert(MODE != 2 || NW >= NSEL, "the fused selection needs kStatThreads / 64 waves");
    const bool by_simd = s_simd_n[0] >= 2u && s_simd_n[1] >= 2u && s_simd_n[2] >= 2u && s_simd_n[3] >= 2u;
    const bool selector = by_simd ? tsimd + 2u >= s_simd_n[simd] : ticket >= (uint32_t)(NW - NSEL);
    if (selector) {
      // every wave increments s_p1done once, after its last phase-1 chunk
      while ((uint32_t)__builtin_amdgcn_readfirstlane(
                 (int)__hip_atomic_load(&s_p1done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < (uint32_t)NW)
        __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      __shared__ FocalSelShared<G> s_fsel;
      WaveSetSync<kStatThreads> grp{by_simd ? (int)(simd * 2u + (tsimd + 2u - s_simd_n[simd])) : (int)ticket - (NW - NSEL),
                                    &s_selctr, 0u};
      float mh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s_wmax[0][h];
        for (int w2 = 1; w2 < NW; ++w2) mx = fmaxf(mx, s_wmax[w2][h]);
        mh[h] = mx;
      }
      const int seg = hi - lo;
      const size_t row = (size_t)b * a.hkv + g;
      float *so = a.sel_scores != nullptr ? a.sel_scores + row * a.sel_ld : nullptr;
      const int seg_out = so != nullptr ? (int)min((int64_t)seg, a.sel_ld) : 0;
      // the selection goes first at the issue arbiter: the streaming waves
      // mostly wait on memory
      __builtin_amdgcn_s_setprio(3);
      focal_select_fused<G>(grp, s_logit, a.seg_cap, seg, a.scale * 1.4426950408889634, mh,
                            a.sel_warm != nullptr ? a.sel_warm + row * a.sel_k : nullptr, a.sel_k,
                            a.sel_idx + row * a.sel_k, so, seg_out, s_fsel);
      __builtin_amdgcn_s_setprio(0);
    }
    uint32_t first = 0;
    if (lane == 0) first = atomicAdd(&s_next2, 1u);
    run(&s_next2, __builtin_amdgcn_readfirstlane((int)first), nch);
  } else {
    run(&s_next, wave, nch);
  }
#undef KVSEL_ROWT

  // merge the four lane groups of each wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo_ = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ca = fast_exp2(m[h] - mn), cb = fast_exp2(mo - mn);
      l[h] = l[h] * ca + lo_ * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * ca + ao * cb;
      }
      m[h] = mn;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][sub * 8 + e] = acc[h][e];
      if (sub == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  // merge the waves; one split: final output, else this split's partial record
  for (int x = tid; x < G * kD; x += NT) {
    const int h = x / kD, dim = x % kD;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = fast_exp2(s_m[w][h] - M);
      L += s_l[w][h] * c;
      A += s_acc[w][h][dim] * c;
    }
    const size_t hb = (size_t)b * a.hq + g * G + h;
    if (a.nsplit == 1) {
      if (MODE == 3) {
        if (dim == 0) a.mass[hb] = L > 0.f ? A / L : 0.f;
      } else {
        a.out[hb * kD + dim] = L > 0.f ? A / L : 0.f;
      }
      if (dim == 0 && a.lse != nullptr) a.lse[hb] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
    } else {
      float *rec = a.rec + (hb * a.nsplit + split) * kRec;
      rec_store(rec + dim, A);
      if (dim == 0) {
        rec_store(rec + kD, M);
        rec_store(rec + kD + 1, L);
      }
    }
  }
#if KVSEL_ATTN_FUSED_MERGE
  // Split records: the last of the pair's work-groups to finish merges them.
  // Each thread waits until its record stores are complete (written through
  // to the agent-coherent level), then one thread counts the work-group in;
  // the one that brings the count to nsplit resets it to zero for the next
  // call and reads every record with agent-scope loads.  No work-group waits
  // for another, and no cache is written back or invalidated.
  if (a.nsplit > 1) {
    __shared__ uint32_t s_last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      uint32_t *ctr = a.counters + (size_t)b * a.hkv + g;
      const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // the pair's counter started this call at zero: below nsplit at every arrival
      KVSEL_CHECK(prev < (uint32_t)a.nsplit, kDbgCounter, prev);
      const uint32_t last = prev == (uint32_t)a.nsplit - 1u ? 1u : 0u;
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (s_last) merge_records<G>(a, b, g, v.nR <= 0 ? 0 : min(a.nsplit, (v.nR + a.rps - 1) / a.rps), tid, NT);
  }
#endif
}

// merge of the split records: grid (kv heads, sequences), G*128 threads
template <int G>
__global__ __launch_bounds__(G * kD) void attn_merge_kernel(AttnArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const SeqView v = seq_view(a, b, a.dense != 0);
  merge_records<G>(a, b, g, v.nR <= 0 ? 0 : min(a.nsplit, (v.nR + a.rps - 1) / a.rps), threadIdx.x, G * kD);
}

// logits only: grid = (row chunks, kv heads, sequences); rows [lo, hi)
template <int G>
__global__ __launch_bounds__(256) void logits_kernel(AttnArgs a) {
  constexpr int NG = 16, U = 4;
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const SeqView v = seq_view(a, b, true);
  int lo, hi;
  if (a.logit_mode == 1) { lo = v.s0; hi = v.s1; }
  else { lo = 0; hi = v.n; }
  const int r0 = lo + chunk * a.rps;
  const int cnt = min(a.rps, hi - r0);
  if (cnt <= 0) return;
  uint4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qr[h] = *reinterpret_cast<const uint4 *>(a.q + ((size_t)b * a.hq + g * G + h) * kD + sub * 8);
  const uint16_t *kbase = a.k_pool + sub * 8;
  for (int base = 0; base < cnt; base += NG * U) {
    uint4 kr[U];
    uint32_t pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + grp + NG * u;
      const uint32_t pt = row_to_phys(a, b, g, r0 + min(t, cnt - 1));   // unbranched table read
      pr[u] = t < cnt ? pt : kNoRow;
      kr[u] = pr[u] != kNoRow ? *reinterpret_cast<const uint4 *>(kbase + (size_t)pr[u] * kD)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot[G];
      dot_rows<G>(qr, kr[u], dot);
      float dsel = dot[0];
#pragma unroll
      for (int h = 1; h < G; ++h) dsel = sub == h ? dot[h] : dsel;
      const int t = base + grp + NG * u;
      // a row whose block is missing is not attended: logit -inf
      if (t < cnt && sub < G && r0 + t - lo < a.ld_logits)
        a.logits[((size_t)b * a.hq + g * G + sub) * a.ld_logits + (r0 + t - lo)] = pr[u] != kNoRow ? dsel : -INFINITY;
    }
  }
}

// threads per attention work-group for a head group size
#ifndef KVSEL_ATTN_NT4
#define KVSEL_ATTN_NT4 512
#endif
#ifndef KVSEL_ATTN_U4
#define KVSEL_ATTN_U4 KVSEL_ATTN_U
#endif
#ifndef KVSEL_ATTN_WAVES_PER_CU4
#define KVSEL_ATTN_WAVES_PER_CU4 8
#endif
constexpr int attn_threads(int G) { return G <= 2 ? KVSEL_ATTN_NT2 : (G <= 4 ? KVSEL_ATTN_NT4 : 256); }
constexpr int attn_unroll(int G) { return G == 3 || G == 4 ? KVSEL_ATTN_U4 : KVSEL_ATTN_U; }
constexpr int attn_waves_per_cu(int G) {
  return G == 3 || G == 4 ? KVSEL_ATTN_WAVES_PER_CU4 : KVSEL_ATTN_WAVES_PER_CU;
}

template <int G>
hipError_t launch_attn_g(const AttnArgs &a, int batch, hipStream_t s) {
  constexpr int NT = attn_threads(G);
  constexpr int U = attn_unroll(G);
  const bool stream = a.shared_rows == 0;   // rows shared across sequences stay cached
  dim3 grid(a.nsplit, a.hkv, batch);
  if (a.sel_idx != nullptr) {
    if (a.det) return hipErrorInvalidValue;   // the fused focal pass takes rows on demand
    if constexpr (NT < kStatThreads) {
      return hipErrorInvalidValue;   // the fused selection needs kStatThreads / 64 waves
    } else {
    if (a.nsplit != 1) return hipErrorInvalidValue;
    const size_t dyn = (size_t)G * a.seg_cap * sizeof(float);
    if (dyn > kFusedLdsBytes) return hipErrorInvalidValue;
    // the LDS above 64 KiB must be allowed (once per device)
    for (const void *f : {(const void *)attn_kernel<G, NT, U, 2, true>, (const void *)attn_kernel<G, NT, U, 2, false>}) {
      const hipError_t e = allow_dynamic_lds(f, (int)kFusedLdsBytes);
      if (e != hipSuccess) return e;
    }
    if (stream)
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 2, true>), grid, dim3(NT), dyn, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 2, false>), grid, dim3(NT), dyn, s, a);
    return hipGetLastError();
    }
  }
  if (a.mass != nullptr) {
    if (a.dense == 0 || a.logits != nullptr) return hipErrorInvalidValue;
    if (stream)
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 3, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 3, false>), grid, dim3(NT), 0, s, a);
  } else if (a.logits != nullptr) {
    if (stream)
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 1, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 1, false>), grid, dim3(NT), 0, s, a);
  } else {
    // Many (sequence, kv head) pairs of few rows each (a branched decode: 4096
    // pairs of ~680 rows) run on 512-thread work-groups, whose prologue and
    // merge are cheaper and four of which share a CU: 142.8 against 141.0 C4
    // steps/s.  C1's 256 pairs of ~1500 rows keep 1024 threads (-11% at 512).
    constexpr int kManyPairs = 2048;
    if constexpr (G == 2 && NT == 1024) {
      if ((int64_t)batch * a.hkv >= kManyPairs && a.nsplit == 1) {
        if (stream)
          hipLaunchKernelGGL((attn_kernel<G, 512, U, 0, true>), grid, dim3(512), 0, s, a);
        else
          hipLaunchKernelGGL((attn_kernel<G, 512, U, 0, false>), grid, dim3(512), 0, s, a);
        return hipGetLastError();
      }
    }
    if (stream)
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 0, true>), grid, dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<G, NT, U, 0, false>), grid, dim3(NT), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1 || KVSEL_ATTN_FUSED_MERGE) return e;
  hipLaunchKernelGGL(attn_merge_kernel<G>, dim3(a.hkv, batch), dim3(G * kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int batch, int hkv, int hq, int max_rows, int logit_mode, int max_seg_len,
                   int max_seq_len) {
  AttnPlan p;
  const int64_t pairs = (int64_t)batch * hkv;
  const int G = hq / hkv;
  // work-group slots: 256 CUs x the waves per CU aimed for / waves per work-group
  const int64_t slots = 256 * (attn_waves_per_cu(G) / (attn_threads(G) / 64));
  int64_t nsplit = (slots + pairs - 1) / pairs;
  // keep at least 256 rows per split, and at most kAttnMaxRps
  const int64_t by_rows = ((int64_t)max_rows + 255) / 256;
  if (nsplit > by_rows) nsplit = by_rows;
  if (nsplit < 1) nsplit = 1;
  int64_t rps = ((int64_t)max_rows + nsplit - 1) / nsplit;
  if (rps > kAttnMaxRps) {
    rps = kAttnMaxRps;
    nsplit = ((int64_t)max_rows + rps - 1) / rps;
  }
  if (rps < 1) rps = 1;
  p.rps = (int)rps;
  p.nsplit = (int)nsplit;
  p.ld_logits = logit_mode == 1 ? max_seg_len : (logit_mode == 2 ? max_seq_len : 0);
  size_t off = 0;
  p.off_counters = off;
  off = kCounterBytes;
  p.off_rec = off;
  if (p.nsplit > 1) off = align_up(off + (size_t)batch * hq * p.nsplit * kRec * sizeof(float));
  p.off_logits = off;
  if (logit_mode) off = align_up(off + (size_t)batch * hq * p.ld_logits * sizeof(float));
  p.off_extra = off;
  p.total = off;
  return p;
}

hipError_t launch_attn(const AttnArgs &a, int batch, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_attn_g<1>(a, batch, s);
    case 2: return launch_attn_g<2>(a, batch, s);
    case 3: return launch_attn_g<3>(a, batch, s);
    case 4: return launch_attn_g<4>(a, batch, s);
    case 5: return launch_attn_g<5>(a, batch, s);
    case 6: return launch_attn_g<6>(a, batch, s);
    case 7: return launch_attn_g<7>(a, batch, s);
    case 8: return launch_attn_g<8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_logits(const AttnArgs &a, int batch, int group, int max_rows, hipStream_t s) {
  const int chunks = (max_rows + a.rps - 1) / a.rps;
  dim3 grid(chunks > 0 ? chunks : 1, a.hkv, batch), block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL(logits_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(logits_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(logits_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(logits_kernel<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(logits_kernel<5>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(logits_kernel<6>, grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL(logits_kernel<7>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(logits_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvsel
