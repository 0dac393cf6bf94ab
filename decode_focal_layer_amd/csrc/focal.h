// Focal score arithmetic shared by the fused focal attention kernel and the
// standalone normalise / select kernels, so that both give the same bits.
//
// FastOCR (technical summary, Focal-Guided Pruning): the focal score of an
// image token is the attention its query heads give it: per head a softmax
// of the logits over the candidate segment, summed over the heads of a kv
// head's group.
//
// Input logits are raw fp32 q.k dot products (exact bf16 products, fp32
// sums).  Per head h: m_h = max_i x_hi; the fp32 term e_hi = 2^((x_hi - m_h) c)
// (c = scale * log2 e, see focal_term); Z_h = sum_i e_hi in fp64 in a fixed
// order.  Per token: the score sum_h e_hi / Z_h in fp64, rounded to fp32 once.
#pragma once

#include "common.h"
#include "radix.h"

namespace kvsel {

// The normaliser's summation order: virtual thread v in [0, 512) adds its
// tokens i = v, v + 512, ... in order; each virtual wave's 64 partial sums are
// reduced by wave_sum_d; the eight wave sums are added in order.  Any group of
// threads that runs virtual thread v as its thread v gets the same bits.
constexpr int kStatThreads = 512;

// The term 2^((x - m) c) for fp32 x and m (m is a float held in a double),
// c = ch + cl split into two floats.  The exponent is formed with fp32
// error-free steps (TwoSum for x - m, a fused multiply-add for the product's
// rounding error) to far below fp32 precision; its leading float goes through
// the hardware exp2 and the small remainder r through 1 + r ln 2.  About two
// fp32 ulps in all, with no fp64 arithmetic.  A logit of -inf (a row that is
// not attended, e.g. its cache block is missing) gives exactly 0: the
// error-free steps would otherwise form -inf - (-inf).
__device__ __forceinline__ float focal_term(float x, double m, double c) {
  const float mf = (float)m;
  const float ch = (float)c, cl = (float)(c - (double)ch);
  const float d = x - mf;   // d + de = x - mf exactly
  const float bv = d - x;
  const float de = (x - (d - bv)) + (-mf - bv);
  const float y = d * ch;   // y + yl ~ (d + de) (ch + cl)
  const float yl = fmaf(d, ch, -y) + fmaf(d, cl, de * ch);
  const float e = __builtin_amdgcn_exp2f(y) * fmaf(yl, 0.6931471805599453f, 1.0f);
  return x == -INFINITY ? 0.f : e;
}

// logit(hh, i) for head hh < nh of the output row and token i < cnt.  Writes
// s_m[hh] = m_h and s_iz[hh] = 1 / Z_h (0 when Z_h = 0).  Run by a whole
// block of NT >= 256 threads; up to NH heads per pass over the tokens.  The
// logits are read kStatBatch tokens at a time, every read unbranched (at a
// clamped token and head) so that they are all in flight together; the
// normaliser still adds each thread's tokens in increasing order.
constexpr int kStatBatch = 8;
template <int NT, int NH, typename LF>
__device__ void focal_stats(LF logit, int nh, int cnt, double c, double *s_m, double *s_iz) {
  constexpr int NW = NT / 64, SW = kStatThreads / 64, BS = kStatBatch;
  static_assert(NT % 64 == 0 && NT >= kStatThreads, "block of at least kStatThreads threads");
  __shared__ float s_wm[NH][NW];
  __shared__ double s_wz[NH][SW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int h0 = 0; h0 < nh; h0 += NH) {
    const int hn = min(NH, nh - h0);
    float mx[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) mx[hh] = -INFINITY;
    for (int i0 = tid; i0 < cnt; i0 += NT * BS) {
      float v[BS][NH];
#pragma unroll
      for (int j = 0; j < BS; ++j) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) v[j][hh] = logit(h0 + min(hh, hn - 1), min(i0 + j * NT, cnt - 1));
      }
#pragma unroll
      for (int j = 0; j < BS; ++j) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          if (hh < hn && i0 + j * NT < cnt) mx[hh] = fmaxf(mx[hh], v[j][hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      mx[hh] = wave_max_f(mx[hh]);
      if (lane == 0) s_wm[hh][w] = mx[hh];
    }
    __syncthreads();
    double md[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float m = s_wm[hh][0];
      for (int j = 1; j < NW; ++j) m = fmaxf(m, s_wm[hh][j]);
      md[hh] = (double)m;
    }
    if (tid < kStatThreads) {
      double part[NH];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) part[hh] = 0.0;
      for (int i0 = tid; i0 < cnt; i0 += kStatThreads * BS) {
        float v[BS][NH];
#pragma unroll
        for (int j = 0; j < BS; ++j) {
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
            v[j][hh] = logit(h0 + min(hh, hn - 1), min(i0 + j * kStatThreads, cnt - 1));
        }
#pragma unroll
        for (int j = 0; j < BS; ++j) {   // tokens i0, i0 + kStatThreads, ... in order
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
            if (hh < hn && i0 + j * kStatThreads < cnt) part[hh] += (double)focal_term(v[j][hh], md[hh], c);
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        part[hh] = wave_sum_d(part[hh]);
        if (lane == 0) s_wz[hh][w] = part[hh];
      }
    }
    __syncthreads();
    if (tid < hn) {
      double z = 0.0;
      for (int j = 0; j < SW; ++j) z += s_wz[tid][j];
      s_m[h0 + tid] = md[tid];
      s_iz[h0 + tid] = z > 0.0 ? 1.0 / z : 0.0;
    }
    __syncthreads();
  }
}

// scores of tokens i0, i0 + stride, ... (kStatBatch of them, those below cnt)
// from the statistics: per token the fp64 sum over the heads in order; the
// reads of one head go out together.  f(i, score) for each token below cnt.
template <typename LF, typename F>
__device__ __forceinline__ void focal_scores_batch(LF logit, int nh, int i0, int stride, int cnt, double c,
                                                   const double *s_m, const double *s_iz, F f) {
  constexpr int BS = kStatBatch;
  double sc[BS];
#pragma unroll
  for (int j = 0; j < BS; ++j) sc[j] = 0.0;
  for (int hh = 0; hh < nh; ++hh) {
    float v[BS];
#pragma unroll
    for (int j = 0; j < BS; ++j) v[j] = logit(hh, min(i0 + j * stride, cnt - 1));
    const double m = s_m[hh], iz = s_iz[hh];
#pragma unroll
    for (int j = 0; j < BS; ++j) sc[j] += (double)focal_term(v[j], m, c) * iz;
  }
#pragma unroll
  for (int j = 0; j < BS; ++j)
    if (i0 + j * stride < cnt) f(i0 + j * stride, sc[j]);
}

// LDS state of the fused selection (one kv head's group of G heads)
template <int G>
struct FocalSelShared {
  RadixShared<kStatThreads> rx;
  double z[G][kStatThreads / 64];
  uint32_t lo[kStatThreads / 64], hi[kStatThreads / 64], wmin[kStatThreads / 64], wbad[kStatThreads / 64];
};

// warm indices read per selection thread (k up to this many times kStatThreads)
constexpr int kWarmPerThread = 2;

// Focal selection of one (sequence, kv head) inside the attention kernel, run
// by a set of eight waves (grp, kStatThreads participants) while the other
// waves of the work-group stream.  s_logit holds the G heads' segment logits
// at h * cap + i (i < seg); they are overwritten (terms, then keys in head 0's
// row).  mh[h] is the logits' max per head.  warm (null: none) is the
// previous selection of this row, k indices; a warm set that is not strictly
// ascending inside [0, seg) is ignored (theta = 0), as is one with k beyond
// kWarmPerThread * 256.  Writes k ascending indices to dst (all seg tokens
// then -1 when seg <= k) and, if so != null, the scores of tokens i < seg_out.
template <int G, typename Grp>
__device__ void focal_select_fused(Grp &grp, float *s_logit, int cap, int seg, double c, const float *mh,
                                   const int32_t *warm, int k, int32_t *dst, float *so, int seg_out,
                                   FocalSelShared<G> &fs) {
  constexpr int NTS = kStatThreads;
  const int t = grp.t(), w = t >> 6;
  // the warm indices are loaded now and used after the score pass
  const bool use_warm = warm != nullptr && k <= kWarmPerThread * NTS;
  int wv[kWarmPerThread], wn[kWarmPerThread];
#pragma unroll
  for (int j = 0; j < kWarmPerThread; ++j) {
    const int i = t + j * NTS;
    wv[j] = 0;
    wn[j] = 0x7fffffff;
    if (use_warm && i < k) {
      wv[j] = warm[i];
      if (i + 1 < k) wn[j] = warm[i + 1];
    }
  }
  double md[G];
#pragma unroll
  for (int h = 0; h < G; ++h) md[h] = (double)mh[h];
  // Pass A: terms (stored in place) and the normalisers' partial sums.  BA
  // tokens per step, so their reads and exponentials overlap; each thread
  // still adds its tokens in increasing order.
  constexpr int BA = 8;
  double z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) z[h] = 0.0;
  for (int base = t; base < seg; base += BA * NTS) {
    float e[BA][G];
#pragma unroll
    for (int j = 0; j < BA; ++j) {
      const int i = min(base + j * NTS, seg - 1);
#pragma unroll
      for (int h = 0; h < G; ++h) e[j][h] = s_logit[h * cap + i];
    }
#pragma unroll
    for (int j = 0; j < BA; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) e[j][h] = focal_term(e[j][h], md[h], c);
    }
#pragma unroll
    for (int j = 0; j < BA; ++j) {
      const int i = base + j * NTS;
      if (i < seg) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s_logit[h * cap + i] = e[j][h];
          z[h] += (double)e[j][h];
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    z[h] = wave_sum_d(z[h]);
    if ((t & 63) == 0) fs.z[h][w] = z[h];
  }
  grp.sync();
  double iz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    double zz = 0.0;
    for (int j = 0; j < NTS / 64; ++j) zz += fs.z[h][j];
    iz[h] = zz > 0.0 ? 1.0 / zz : 0.0;
  }
  // pass B: scores -> keys (head 0's row) and their range
  uint32_t *keys = reinterpret_cast<uint32_t *>(s_logit);
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int base = t; base < seg; base += BA * NTS) {
    float e[BA][G];
#pragma unroll
    for (int j = 0; j < BA; ++j) {
      const int i = min(base + j * NTS, seg - 1);
#pragma unroll
      for (int h = 0; h < G; ++h) e[j][h] = s_logit[h * cap + i];
    }
#pragma unroll
    for (int j = 0; j < BA; ++j) {
      const int i = base + j * NTS;
      double sc = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h) sc += (double)e[j][h] * iz[h];
      const float f = (float)sc;
      const uint32_t x = okey(f);
      if (i < seg) {
        keys[i] = x;
        if (so != nullptr && i < seg_out) so[i] = f;
        lo = min(lo, x);
        hi = max(hi, x);
      }
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if ((t & 63) == 0) {
    fs.lo[w] = lo;
    fs.hi[w] = hi;
  }
  grp.sync();
  lo = 0xffffffffu;
  hi = 0u;
  for (int j = 0; j < NTS / 64; ++j) {
    lo = min(lo, fs.lo[j]);
    hi = max(hi, fs.hi[j]);
  }
  if (seg <= k) {   // every token kept
    for (int i = t; i < k; i += NTS) dst[i] = i < seg ? i : -1;
    return;
  }
  // theta: the smallest key at the warm indices (a valid warm set has k
  // indices, so at least k keys reach it), or 0
  uint32_t theta = 0u;
  if (use_warm) {
    uint32_t bad = 0u, wmin = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kWarmPerThread; ++j) {
      if (t + j * NTS < k) {
        const int x = wv[j];
        if (x < 0 || x >= seg || wn[j] <= x) bad = 1u;
        else wmin = min(wmin, keys[x]);
      }
    }
    bad = wave_max_u32(bad);
    wmin = wave_min_u32(wmin);
    if ((t & 63) == 0) {
      fs.wbad[w] = bad;
      fs.wmin[w] = wmin;
    }
    grp.sync();
    bad = 0u;
    wmin = 0xffffffffu;
    for (int j = 0; j < NTS / 64; ++j) {
      bad |= fs.wbad[j];
      wmin = min(wmin, fs.wmin[j]);
    }
    theta = bad ? 0u : wmin;
  }
  if (theta > lo) lo = theta;
  auto key = [&](int i) -> uint32_t { return keys[i]; };
  radix_select<NTS, true, 25>(grp, key, seg, k, theta, lo, hi, (uint32_t)seg, dst, fs.rx, keys);
}

}  // namespace kvsel
