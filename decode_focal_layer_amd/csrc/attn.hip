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
//    work-groups whose partial (max, sum, accumulator) records are merged by a
//    second small kernel.  No work-group waits on another.
//  * prologue: the work-group resolves its rows to physical cache rows
//    (index -> block table -> block) into LDS once, so the streaming loop
//    issues only K/V loads.
//  * a lane group of 16 lanes owns one row at a time: a lane holds 8 of the
//    128 dims (one 16-byte load per K row and per V row, so a wave reads four
//    consecutive 256-byte rows per load instruction), the 16-lane dot product
//    is reduced with DPP row operations, and each lane group keeps its own
//    online-softmax state (max, sum, 8 accumulator dims per query head of the
//    group), so the loop has no cross-group synchronisation.
//  * the lane-group states are merged in registers (the four groups of a
//    wave) and in LDS (across waves).
#include "common.h"
#include "kvsel_internal.h"

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

namespace kvsel {

namespace {

constexpr int kTabLds = 2048;   // block tables up to this many entries are staged in LDS

struct SeqView {
  int n, s0, s1, nR;
};

__device__ __forceinline__ SeqView seq_view(const AttnArgs &a, int b, bool dense) {
  SeqView v;
  const int cap = a.max_blocks * kBlk;
  v.n = clampi(a.seq_len[b], 0, cap);
  v.s0 = clampi(a.seg_begin[b], 0, v.n);
  v.s1 = clampi(a.seg_end[b], v.s0, v.n);
  v.nR = dense ? v.n : (a.k + v.s0 + (v.n - v.s1));
  return v;
}

// virtual row j -> logical row (or -1)
__device__ __forceinline__ int virt_to_row(const AttnArgs &a, const SeqView &v, int b, int g, int j,
                                           bool dense) {
  if (dense) return j;
  if (j < a.k) {
    const int r = a.idx[((size_t)b * a.hkv + g) * a.k + j];
    return (r >= 0 && r < v.s1 - v.s0) ? v.s0 + r : -1;
  }
  if (j < a.k + v.s0) return j - a.k;
  return v.s1 + (j - a.k - v.s0);
}

__device__ __forceinline__ uint32_t row_to_phys(const AttnArgs &a, int b, int g, int row) {
  if (row < 0) return kNoRow;
  const int blk = a.block_table[(size_t)b * a.max_blocks + (row >> 4)];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return kNoRow;
  return ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
}

template <int G>
__device__ __forceinline__ void dot_rows(const float (&qf)[G][8], const uint4 &kr, float (&dot)[G]) {
  float kf[8];
  unpack8(kr, kf);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float s = qf[h][0] * kf[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) s = fmaf(qf[h][e], kf[e], s);
    dot[h] = row16_sum(s);
  }
}

template <int G, int NT, int U>
__global__ __launch_bounds__(NT) void attn_kernel(AttnArgs a) {
  constexpr int NG = NT / 16;    // lane groups
  constexpr int NW = NT / 64;    // waves
  constexpr int ITER = NG * U;   // rows per iteration of the work-group
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = tid >> 4, sub = tid & 15;
  const bool dense = a.dense != 0;

  __shared__ uint32_t s_prow[kAttnMaxRps];
  __shared__ int32_t s_tab[kTabLds];
  __shared__ float s_acc[NW][G][kD];
  __shared__ float s_m[NW][G], s_l[NW][G];

  const SeqView v = seq_view(a, b, dense);
  const int start = split * a.rps;
  const int cnt = max(0, min(a.rps, v.nR - start));   // rows of this split

  int lo = 0, hi = 0;   // logical rows whose logits are stored, at row - lo (dense only)
  if (a.logits != nullptr) {
    if (a.logit_mode == 1) { lo = v.s0; hi = v.s1; }
    else { lo = 0; hi = v.n; }
  }

  // Prologue: the kept indices and the block table are loaded together (one
  // memory latency), then each virtual row is resolved to its physical row.
  {
    constexpr int RPT = kAttnMaxRps / NT;
    const bool tab_lds = a.max_blocks <= kTabLds;
    int lr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int t = tid + i * NT;
      lr[i] = t < cnt ? virt_to_row(a, v, b, g, start + t, dense) : -1;
    }
    if (tab_lds)
      for (int i = tid; i < a.max_blocks; i += NT) s_tab[i] = a.block_table[(size_t)b * a.max_blocks + i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int t = tid + i * NT;
      if (t < cnt) {
        const int row = lr[i];
        uint32_t pr = kNoRow;
        if (row >= 0) {
          const int blk = tab_lds ? s_tab[row >> 4] : a.block_table[(size_t)b * a.max_blocks + (row >> 4)];
          if (blk >= 0 && (int64_t)blk < a.num_blocks)
            pr = ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
        }
        s_prow[t] = pr;
      }
    }
  }

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qv = *reinterpret_cast<const uint4 *>(a.q + ((size_t)b * a.hq + g * G + h) * kD + sub * 8);
    unpack8(qv, qf[h]);
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  const uint16_t *kbase = a.k_pool + sub * 8;
  const uint16_t *vbase = a.v_pool + sub * 8;
  for (int base = 0; base < cnt; base += ITER) {
    uint4 kr[U], vr[U];
    uint32_t pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + grp + NG * u;
      pr[u] = t < cnt ? s_prow[t] : kNoRow;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pr[u] != kNoRow) {
        kr[u] = *reinterpret_cast<const uint4 *>(kbase + (size_t)pr[u] * kD);
        vr[u] = *reinterpret_cast<const uint4 *>(vbase + (size_t)pr[u] * kD);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float dot[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) dot_rows<G>(qf, kr[u], dot[u]);
    if (a.logits != nullptr) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = start + base + grp + NG * u;   // dense: logical row = virtual row
        if (base + grp + NG * u < cnt && sub < G && pr[u] != kNoRow && row >= lo && row < hi &&
            row - lo < a.ld_logits) {
          float dv = dot[u][0];
#pragma unroll
          for (int h = 1; h < G; ++h) dv = sub == h ? dot[u][h] : dv;
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
        s[u] = pr[u] != kNoRow ? dot[u][h] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      const float mn = fmaxf(m[h], mx);
      if (mn != -INFINITY) {
        const float c = fast_exp2(m[h] - mn);   // m = -inf -> 0
        float ps = 0.f;
        float p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u] = fast_exp2(s[u] - mn);
          ps += p[u];
        }
        l[h] = l[h] * c + ps;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= c;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float vf[8];
          unpack8(vr[u], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p[u], vf[e], acc[h][e]);
        }
        m[h] = mn;
      }
    }
  }

  // merge the four lane groups of each wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo_ = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ca = rescale(m[h], mn), cb = rescale(mo, mn);
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
      const float c = rescale(s_m[w][h], M);
      L += s_l[w][h] * c;
      A += s_acc[w][h][dim] * c;
    }
    const size_t hb = (size_t)b * a.hq + g * G + h;
    if (a.nsplit == 1) {
      a.out[hb * kD + dim] = L > 0.f ? A / L : 0.f;
      if (dim == 0 && a.lse != nullptr) a.lse[hb] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
    } else {
      float *rec = a.rec + (hb * a.nsplit + split) * kRec;
      rec[dim] = A;
      if (dim == 0) {
        rec[kD] = M;
        rec[kD + 1] = L;
      }
    }
  }
}

// merge of the split records: grid (kv heads, sequences), G*128 threads
template <int G>
__global__ __launch_bounds__(G * kD) void attn_merge_kernel(AttnArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int h = threadIdx.x / kD, dim = threadIdx.x % kD;
  const SeqView v = seq_view(a, b, a.dense != 0);
  const int nact = v.nR <= 0 ? 0 : min(a.nsplit, (v.nR + a.rps - 1) / a.rps);
  const size_t hb = (size_t)b * a.hq + g * G + h;
  const float *rec0 = a.rec + hb * a.nsplit * kRec;
  float M = -INFINITY;
  for (int sp = 0; sp < nact; ++sp) M = fmaxf(M, rec0[sp * kRec + kD]);
  float L = 0.f, A = 0.f;
  for (int sp = 0; sp < nact; ++sp) {
    const float c = rescale(rec0[sp * kRec + kD], M);
    L += rec0[sp * kRec + kD + 1] * c;
    A += rec0[sp * kRec + dim] * c;
  }
  a.out[hb * kD + dim] = L > 0.f ? A / L : 0.f;
  if (dim == 0 && a.lse != nullptr) a.lse[hb] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
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
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qv = *reinterpret_cast<const uint4 *>(a.q + ((size_t)b * a.hq + g * G + h) * kD + sub * 8);
    unpack8(qv, qf[h]);
  }
  const uint16_t *kbase = a.k_pool + sub * 8;
  for (int base = 0; base < cnt; base += NG * U) {
    uint4 kr[U];
    uint32_t pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + grp + NG * u;
      pr[u] = t < cnt ? row_to_phys(a, b, g, r0 + t) : kNoRow;
      kr[u] = pr[u] != kNoRow ? *reinterpret_cast<const uint4 *>(kbase + (size_t)pr[u] * kD)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot[G];
      dot_rows<G>(qf, kr[u], dot);
      float dsel = dot[0];
#pragma unroll
      for (int h = 1; h < G; ++h) dsel = sub == h ? dot[h] : dsel;
      const int t = base + grp + NG * u;
      if (t < cnt && sub < G && pr[u] != kNoRow && r0 + t - lo < a.ld_logits)
        a.logits[((size_t)b * a.hq + g * G + sub) * a.ld_logits + (r0 + t - lo)] = dsel;
    }
  }
}

// threads per attention work-group for a head group size
constexpr int attn_threads(int G) {
  return G <= 2 ? KVSEL_ATTN_NT2 : (G == 4 ? (KVSEL_ATTN_NT2 < 512 ? KVSEL_ATTN_NT2 : 512) : 256);
}

template <int G>
hipError_t launch_attn_g(const AttnArgs &a, int batch, hipStream_t s) {
  constexpr int NT = attn_threads(G);
  dim3 grid(a.nsplit, a.hkv, batch);
  hipLaunchKernelGGL((attn_kernel<G, NT, KVSEL_ATTN_U>), grid, dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
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
  const int64_t slots = 256 * (KVSEL_ATTN_WAVES_PER_CU / (attn_threads(G) / 64));
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
    case 4: return launch_attn_g<4>(a, batch, s);
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
    case 4: hipLaunchKernelGGL(logits_kernel<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(logits_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvsel
