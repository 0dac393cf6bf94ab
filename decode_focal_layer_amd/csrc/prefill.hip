// Causal prefill attention over the propagated tokens, on MFMA.
//
// FastKV (section 2A, Token-Selective Propagation, two-stage prefill): after
// the TSP layer only the top-ranked tokens and the window tokens go on to
// the later layers, which run ordinary causal prefill attention over that
// shorter sequence.  The propagated tokens keep their order of position, so
// token i of the compacted sequence sees tokens 0..i.
//
// One work-group per (128 query rows, kv head, sequence), four waves of 32
// query rows.  A query row is a (position, head) pair of the kv head's
// group, numbered position-major, so a work-group covers 128/G positions
// for any group size G.  Keys go through LDS in tiles of 64:
//  * K row-major, bf16, the 16-byte chunks of a row XOR-swizzled by the key
//    (conflict-free writes of whole rows and reads of one chunk per key);
//  * V transposed, scaled by a power of two and converted to fp16, its key
//    order permuted so that P leaves the S product already in the operand
//    order of the P V product (no lane exchange).  The scale 2^-e is one per
//    work-group and only grows: e is 0 while the largest V magnitude seen is
//    in [2^-4, 2^15), else floor(log2) of it minus 14, so the scaled V stay
//    below 2^15 (inside fp16).  Scaled V of at least 2^-14 (fp16 normal) are
//    exact; smaller ones are off by less than 2^-20 of the largest magnitude,
//    for V of any magnitude (bf16 values below 2^-86 aside).  The first
//    tile's exact maximum sets e; after the P V products of each tile, each
//    wave tests the next tile's V (already in registers) against the
//    magnitude that would raise e and takes the exact maximum only if one
//    reaches it; the work-group reads the waves' reports after the barrier
//    before the stash, and when e grows O is rescaled by the exact power of
//    two.  O is multiplied by 2^e at the end.
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as A rows, query rows as
// B columns: each lane owns one query row and 16 keys of a 32-key block);
// online softmax per row in fp32 whose running max is moved only when a
// row's max grows by more than 8 (log2 units), so the O rescale is rare;
// O^T += V^T P with v_mfma_f32_32x32x16_f16, P rounded to nearest fp16
// (11 significant bits, P <= 256).  The
// next tile's K/V are fetched into registers while the current one runs.
// Work items (sequence, kv head, row block) are ordered head-major with each
// head's latest (heaviest) row blocks first, and cut into eight contiguous
// runs, one per XCD (work-groups are dealt to the XCDs in turn): each XCD
// then works through about one head at a time, whose K/V stays in its L2.
#include "common.h"
#include "kvsel_internal.h"
#include "mfma_common.h"
#include "mfma_kernels.h"

namespace kvsel {

namespace {

constexpr int kPThreads = 256;
constexpr int kPWaves = kPThreads / 64;
constexpr int kPRows = 32 * kPWaves;   // query rows per work-group
static_assert(kPWaves == 4, "the V maxima are gathered from four waves");
constexpr int kBN = 64;                // keys per tile
constexpr float kSlack = 8.f;          // log2 headroom of the running max (p <= 256 in fp16)
constexpr int kLgStride = 65;          // floats per staged logits row (64 keys + 1: distinct banks)
constexpr int kVExpNone = -1000;       // V scale exponent before any nonzero V

// byte offset of K chunk c (dims 8c .. 8c+7) of tile key r
__device__ __forceinline__ int k_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// byte offset of V^T element (dim d, tile position p); the 16-byte blocks of
// a row are XOR-swizzled by the dim, so that the 16-byte reads of 8 (or 16)
// consecutive dims fall in distinct banks
__device__ __forceinline__ int vt_off(int d, int p) {
  const int sw = (d ^ (d >> 3)) & 7;
  return d * 128 + ((((p >> 3) ^ sw) & 7) << 4) + (p & 7) * 2;
}

// tile position of keys 4q .. 4q+3 (q = 0..15).  Key 32*blk + 8*a + 4*hf + r
// comes out of S in lane half hf, register 4a + r of block blk; the P V
// product's k-step s takes register 8*(s&1) + i of block s>>1 from lane half
// hf as k-index hf*8 + i, so that key goes to position
// 32*blk + 16*(a>>1) + 8*hf + 4*(a&1) + r.
__device__ __forceinline__ int quad_pos(int q) {
  const int blk = q >> 3, a = (q & 7) >> 1, hf = q & 1;
  return blk * 32 + (a >> 1) * 16 + hf * 8 + (a & 1) * 4;
}

// staging of one tile: K chunk i = tid + 256u is (key i/16, chunk i%16); V
// holds keys 4*(tid/16) .. +3 of chunk tid%16.  Keys past the sequence read
// its last row (masked later).
struct Stage {
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

// byte offsets of this thread's rows from the tile's first row (K: u = 0..3,
// V: u = 4..7); keys past the sequence are clamped to its last row
struct StageOff {
  uint32_t o[8];
};

__device__ __forceinline__ StageOff stage_off(int t0, int n, int tid, uint32_t row_bytes) {
  StageOff s;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + kPThreads * u;
    s.o[u] = (uint32_t)(min(t0 + (i >> 4), n - 1) - t0) * row_bytes + (uint32_t)(i & 15) * 16u;
    s.o[4 + u] = (uint32_t)(min(t0 + (tid >> 4) * 4 + u, n - 1) - t0) * row_bytes + (uint32_t)(tid & 15) * 16u;
  }
  return s;
}

// tile base (uniform) + 32-bit per-thread offsets: scalar-base global loads
__device__ __forceinline__ Stage fetch(const uint8_t *kt, const uint8_t *vt, const StageOff &s) {
  auto ld = [](const uint8_t *p, uint32_t o) { return *reinterpret_cast<const uint4 *>(p + o); };
  return Stage{ld(kt, s.o[0]), ld(kt, s.o[1]), ld(kt, s.o[2]), ld(kt, s.o[3]),
               ld(vt, s.o[4]), ld(vt, s.o[5]), ld(vt, s.o[6]), ld(vt, s.o[7])};
}

// the largest bf16 magnitude (as bits) of this thread's staged V rows
__device__ __forceinline__ uint32_t v_max_bits(const Stage &st) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint4 vs[4] = {st.v0, st.v1, st.v2, st.v3};
  u16x2 m = {0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, word_of(vs[u], e) & 0x7fff7fffu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// 2^k as a float, k in [-126, 127]
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }

// The work-group's V scale exponent after a tile whose largest V magnitude
// has bf16 bits mx (uniform): unchanged for an all-zero tile; else at least
// floor(log2 max) - 14 (the scaled tile stays below 2^15 = inside fp16, inf
// and nan giving 114), 0 while the largest magnitude is in [2^-4, 2^15) (no
// scaling for V of ordinary size), and never below -100 (2^100 is a float).
// O is rescaled by the exact power of two when the exponent grows.
__device__ __forceinline__ int next_v_exp(int e, uint32_t mx, f32x16 (&acc)[4]) {
  if (mx == 0u) return e;
  const int ex = (int)(mx >> 7) - 127;   // floor(log2 |v|); -127 for bf16 subnormals, 128 for inf and nan
  const int want = (ex > 14 || ex < -4) ? max(ex - 14, -100) : 0;
  if (want <= e) return e;
  if (e != kVExpNone) {
    const int d = e - want;   // < 0
    const float f = d < -126 ? 0.f : pow2f(d);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[dt][j] *= f;
  }
  return want;
}

// bf16 bits of the smallest V magnitude that makes next_v_exp raise e: any
// nonzero one while none is set; else 2^(e+15), for e < 0 at most 2^-4
// (where e returns to 0); 0x8000 (above every bf16 magnitude) for none
__device__ __forceinline__ uint32_t v_grow_bits(int e) {
  if (e == kVExpNone) return 1u;
  const int t = e < 0 ? min(e + 15, -4) : e + 15;   // >= -85
  return t + 127 >= 255 ? 0x8000u : (uint32_t)(t + 127) << 7;
}

// the tile's K into LDS as it is
__device__ __forceinline__ void stash_k(const Stage &st, uint8_t *s_k, int tid) {
  const uint4 ks[4] = {st.k0, st.k1, st.k2, st.k3};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + kPThreads * u;
    *reinterpret_cast<uint4 *>(s_k + k_off(i >> 4, i & 15)) = ks[u];
  }
}

// the tile's V into LDS, transposed and converted to fp16 after scaling by
// sc (SCALED) or as it is
template <bool SCALED>
__device__ __forceinline__ void stash_v_as(const Stage &st, uint8_t *s_vt, int tid, float sc) {
  const int p = quad_pos(tid >> 4), vc = tid & 15;
  // fp16 pair of two bf16 values (as float bits)
  auto cv = [&](uint32_t a_bits, uint32_t b_bits) {
    return SCALED ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(a_bits) * sc,
                                                                            __uint_as_float(b_bits) * sc))
                  : f16_pair(a_bits, b_bits);
  };
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {   // dims vc*8 + 2*e2 (low halves) and + 1 (high halves)
    const uint32_t w0 = word_of(st.v0, e2), w1 = word_of(st.v1, e2);
    const uint32_t w2 = word_of(st.v2, e2), w3 = word_of(st.v3, e2);
    *reinterpret_cast<uint2 *>(s_vt + vt_off(vc * 8 + 2 * e2, p)) =
        make_uint2(cv(w0 << 16, w1 << 16), cv(w2 << 16, w3 << 16));
    *reinterpret_cast<uint2 *>(s_vt + vt_off(vc * 8 + 2 * e2 + 1, p)) =
        make_uint2(cv(w0 & 0xffff0000u, w1 & 0xffff0000u), cv(w2 & 0xffff0000u, w3 & 0xffff0000u));
  }
}

// the tile's V into LDS after scaling by 2^-e (exact; no scaling when e is 0
// or none is set yet; e uniform)
__device__ __forceinline__ void stash_v(const Stage &st, uint8_t *s_vt, int tid, int e) {
  if (e == 0 || e == kVExpNone)
    stash_v_as<false>(st, s_vt, tid, 1.f);
  else
    stash_v_as<true>(st, s_vt, tid, pow2f(-e));
}

// Whether one of this thread's staged V magnitudes reaches the bf16 bits t.
// A bf16 pair read as an fp16 pair keeps the order of its values among
// values of one sign, so the packed maximum and minimum over the raw words
// decide it for 0 < t <= 0x7c00; an fp16 nan among them (a bf16 magnitude
// above 0x7c00) counts as reaching.  The answer errs only towards yes: for t
// = 1 should fp16 denormals be flushed, and for t above 0x7c00 (the fp16
// pattern of t then a nan or -0), where every tile reaches.
__device__ __forceinline__ bool v_reaches(const Stage &st, uint32_t t) {
  typedef _Float16 hx2 __attribute__((ext_vector_type(2)));
  const uint4 vs[4] = {st.v0, st.v1, st.v2, st.v3};
  auto h = [&](int i) { return __builtin_bit_cast(hx2, word_of(vs[i >> 2], i & 3)); };
  hx2 mx = h(0), mn = h(0);
#pragma unroll
  for (int i = 1; i < 16; i += 2) {
    const hx2 x = h(i), y = i + 1 < 16 ? h(i + 1) : h(i);
    mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, x), y);
    mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, x), y);
  }
  const _Float16 th = __builtin_bit_cast(_Float16, (uint16_t)t);
  const bool r0 = !(mx.x < th), r1 = !(mx.y < th), r2 = !(mn.x > -th), r3 = !(mn.y > -th);
  return (r0 | r1) | (r2 | r3);   // no short circuit: one straight sequence
}

// This wave's report on a fetched tile's V, for the exponent update before
// its stash: the wave's largest magnitude (bits) when it reaches
// v_grow_bits(e), else 0 -- the exact maximum is taken only then, and
// whenever some wave reports one the largest report is the work-group's
// maximum.  Lane 0 writes it to s_wmax[wave].
__device__ __forceinline__ void report_v(const Stage &st, int e, uint32_t *s_wmax, int tid) {
  uint32_t wm = 0u;
  if (__ballot(v_reaches(st, v_grow_bits(e))) != 0) wm = wave_max_u32(v_max_bits(st));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = wm;
}

// the work-group's largest V magnitude from the waves' reports (uniform)
__device__ __forceinline__ uint32_t group_v_max(const uint32_t *s_wmax) {
  const uint4 m = *reinterpret_cast<const uint4 *>(s_wmax);
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)max(max(m.x, m.y), max(m.z, m.w)));
}

// The scale exponent from the first tile's exact largest V magnitude
__device__ __forceinline__ int first_v_exp(const Stage &st, uint32_t *s_wmax, int tid, f32x16 (&acc)[4]) {
  const uint32_t wm = wave_max_u32(v_max_bits(st));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = wm;
  __syncthreads();
  return next_v_exp(kVExpNone, group_v_max(s_wmax), acc);
}

// V rows of a shared-range tile that are not attended (vkeep bit u clear:
// row u of this thread) set to zero before the stash: p = 0 must not meet a
// non-finite value
__device__ __forceinline__ void zero_dropped_v(Stage &st, int vkeep) {
  if (vkeep == 0xf) return;
  const uint4 z = make_uint4(0, 0, 0, 0);
  if (!(vkeep & 1)) st.v0 = z;
  if (!(vkeep & 2)) st.v1 = z;
  if (!(vkeep & 4)) st.v2 = z;
  if (!(vkeep & 8)) st.v3 = z;
}

// O back from V scaled by 2^-e: O * 2^e (exact short of overflow)
__device__ __forceinline__ void unscale_v(f32x16 (&acc)[4], int e) {
  if (e == 0 || e == kVExpNone) return;
  const float f = pow2f(e);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[dt][j] *= f;
}

// One 64-key tile for this lane's query row: S^T = K Q^T from the LDS K
// tile, the online softmax, O^T += V^T P from the LDS V^T tile.  masked(bk, j)
// drops key 32*bk + 8*(j/4) + 4*hf + j%4 of the tile; it is evaluated only
// when need_mask.  on_dots(s) sees the raw dots before the mask; after_pv()
// runs once the P V products are issued (work that overlaps them).
template <typename MaskFn, typename DotsFn, typename AfterFn>
__device__ __forceinline__ void attend_tile(const uint8_t *s_k, const uint8_t *s_vt, const bf16x8 (&qop)[8], int col,
                                            int hf, float scale_log2, bool need_mask, MaskFn masked, DotsFn on_dots,
                                            AfterFn after_pv, f32x16 (&acc)[4], float &mrun, float &lsum) {
    // S^T, two 32-key blocks: s[bk][j] is key t0 + 32*bk + 8*(j/4) + 4*hf + j%4
    // (operands read one k-step ahead of the products that use them)
    f32x16 s[2] = {{}, {}};
    {
      auto kread = [&](int bk, int kk) {
        return *reinterpret_cast<const bf16x8 *>(s_k + k_off(bk * 32 + col, hf * 8 + kk));
      };
      bf16x8 c0 = kread(0, 0), c1 = kread(1, 0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bf16x8 n0, n1;
        if (kk < 7) {
          n0 = kread(0, kk + 1);
          n1 = kread(1, kk + 1);
        }
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c0, qop[kk], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1, qop[kk], s[1], 0, 0, 0);
        if (kk < 7) {
          c0 = n0;
          c1 = n1;
        }
      }
      // keep the order: reads of k-steps 0 and 1, then (2 products, 2 reads of the next step) ...
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int kk = 0; kk < 6; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    on_dots(s);
    if (need_mask) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (masked(bk, j)) s[bk][j] = -INFINITY;
    }
    float tm = s[0][0];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int j = 0; j < 16; ++j) tm = fmaxf(tm, s[bk][j]);
    tm = half_pair_max(tm) * scale_log2;   // the row's max in this tile, log2 units (scale > 0)
    // the running max moves only when a row's max grows by more than kSlack:
    // p then stays below 2^kSlack and the rescale is skipped on most tiles
    if (__ballot(tm > mrun + kSlack) != 0) {
      const float mnew = fmaxf(mrun, tm);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[dt][j] *= alpha;
    }
    const float neg = mrun == -INFINITY ? 0.f : -mrun;   // a row that has seen nothing yet keeps p = 0
    float ps = 0.f;
    f16x8 pop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(fmaf(s[ks >> 1][(ks & 1) * 8 + i], scale_log2, neg));
        ps += p[i];
      }
      const h2 p01 = __builtin_convertvector((f2){p[0], p[1]}, h2), p23 = __builtin_convertvector((f2){p[2], p[3]}, h2);
      const h2 p45 = __builtin_convertvector((f2){p[4], p[5]}, h2), p67 = __builtin_convertvector((f2){p[6], p[7]}, h2);
      pop[ks] = __builtin_shufflevector(__builtin_shufflevector(p01, p23, 0, 1, 2, 3),
                                        __builtin_shufflevector(p45, p67, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
    lsum += ps;
    {
      auto vread = [&](int dt, int ks) {
        return *reinterpret_cast<const f16x8 *>(s_vt + vt_off(dt * 32 + col, ks * 16 + hf * 8));
      };
      f16x8 c[4] = {vread(0, 0), vread(1, 0), vread(2, 0), vread(3, 0)};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        f16x8 nx[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          if (ks < 3) nx[dt] = vread(dt, ks + 1);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(c[dt], pop[ks], acc[dt], 0, 0, 0);
        }
        if (ks < 3)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) c[dt] = nx[dt];
      }
    }
    after_pv();
}

__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kBN * 256];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kD * kBN * 2];
  __shared__ __attribute__((aligned(16))) uint32_t s_wmax[kPWaves];   // each wave's report on the next tile's V

  const uint32_t L = blockIdx.x, per = gridDim.x >> 3;
  const uint32_t w = (L & 7u) * per + (L >> 3);   // this XCD's run, in order
  if (w >= (uint32_t)a.items) return;
  const int blk = a.nblk - 1 - (int)(w % (uint32_t)a.nblk);
  const int g = (int)((w / (uint32_t)a.nblk) % (uint32_t)a.hkv), b = (int)(w / ((uint32_t)a.nblk * a.hkv));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int G = a.group;
  const int64_t base = a.cu_seqlens[b];
  const int n = (int)min((int64_t)a.max_seqlen, max((int64_t)0, (int64_t)a.cu_seqlens[b + 1] - base));
  const int nrows = n * G;
  const int row0 = blk * kPRows;
  if (row0 >= nrows) return;   // the whole work-group
  const int kend = (min(row0 + kPRows, nrows) - 1) / G + 1;   // keys any row here sees

  // this lane's query row (B operand: dims hf*64 + kk*8 .. +8)
  const int rr = row0 + wave * 32 + col;
  const bool live = rr < nrows;
  const int pos = live ? rr / G : -1;   // -1 sees no key
  const int h = rr % G;
  const int wave_last = min(row0 + wave * 32 + 31, nrows - 1);
  const int wave_kend = wave_last >= row0 + wave * 32 ? wave_last / G + 1 : 0;   // keys this wave's rows see
  bf16x8 qop[8];
  if (live) {
    const uint4 *p = reinterpret_cast<const uint4 *>(a.q + ((base + pos) * a.hq + g * G + h) * kD + hf * 64);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, p[kk]);
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }


  float mrun = -INFINITY, lsum = 0.f;   // this row's running max; this lane's share of the sum
  f32x16 acc[4];                        // O^T: dims dt*32 + 8*(j/4) + 4*hf + j%4 of this row
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = {};

  // K/V rows of this (sequence, kv head): row r at byte (r * hkv) * 256
  const uint32_t row_bytes = (uint32_t)a.hkv * kD * 2;
  const uint8_t *kseq = reinterpret_cast<const uint8_t *>(a.k + (base * a.hkv + g) * kD);
  const uint8_t *vseq = reinterpret_cast<const uint8_t *>(a.v + (base * a.hkv + g) * kD);
  const StageOff full = stage_off(0, kBN, tid, row_bytes);   // a tile wholly inside the sequence
  auto fetch_tile = [&](int t0) {
    const size_t o = (size_t)t0 * row_bytes;
    KVSEL_CHECK(t0 >= 0 && t0 < n, kDbgKvRow, t0);   // a tile starts inside the sequence
    return fetch(kseq + o, vseq + o, t0 + kBN <= n ? full : stage_off(t0, n, tid, row_bytes));
  };

  const int wave_row0 = row0 + wave * 32;
  const bool wave_full = wave_row0 + 31 < nrows;
  const int wave_pos0 = wave_row0 / G;   // the wave's earliest position

  Stage st = fetch_tile(0);
  int ve = first_v_exp(st, s_wmax, tid, acc);   // V scale exponent (uniform)
  for (int t0 = 0; t0 < kend; t0 += kBN) {
    __syncthreads();   // the previous tile's reads are done; the waves' reports on this tile are in
    stash_k(st, s_k, tid);
    ve = next_v_exp(ve, group_v_max(s_wmax), acc);
    stash_v(st, s_vt, tid, ve);
    __syncthreads();
    const bool more = t0 + kBN < kend;
    if (more) st = fetch_tile(t0 + kBN);
    // the report on the next tile (read after the next first barrier)
    auto report = [&] {
      if (more) report_v(st, ve, s_wmax, tid);
    };
    if (t0 >= wave_kend) {   // every row of this wave is before the tile
      report();
      continue;
    }

    // the causal mask, only on tiles that reach past a row of this wave
    attend_tile(s_k, s_vt, qop, col, hf, a.scale_log2, !wave_full || t0 + kBN - 1 > wave_pos0,
                [&](int bk, int j) { return t0 + 32 * bk + 8 * (j >> 2) + 4 * hf + (j & 3) > pos; },
                [](const f32x16 (&)[2]) {}, report, acc, mrun, lsum);
  }

  const float lrow = half_pair_sum(lsum);
  if (!live) return;
  const int64_t orow = (base + pos) * a.hq + g * G + h;
  const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
  unscale_v(acc, ve);
  float *o = a.out + orow * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq)
      *reinterpret_cast<float4 *>(o + dt * 32 + 8 * jq + 4 * hf) =
          make_float4(acc[dt][4 * jq] * inv, acc[dt][4 * jq + 1] * inv, acc[dt][4 * jq + 2] * inv,
                      acc[dt][4 * jq + 3] * inv);
  if (hf == 0 && a.lse != nullptr)
    a.lse[orow] = lrow > 0.f ? (mrun + __log2f(lrow)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
// Every sequence's queries over one shared row range (a shared prefix read
// zero-copy through one block table): the part of each branch's attention
// that all branches have in common, computed once per kv head for all of
// them.  HPD-Parsing wiki, method item 2: the branches reuse the shared
// context's KV.  Query row rr = sequence * G + head of the group; no mask but
// the range's ends and invalid blocks.  Same tiles and tile step as the
// prefill kernel; the output is normalised over the range, with its lse, or
// (accumulate) folded into the attention over other rows already in out/lse.
// ---------------------------------------------------------------------------
// Tiles start on a cache-block boundary (keys before the part's first row are
// masked), so each load's block is uniform: K chunk u of thread t is key
// t0 + 16u + t/16, in block t0/16 + u; its V rows are keys t0 + 4(t/16) + u,
// all in block t0/16 + wave.  A load is then a scalar block base plus one
// per-thread offset.
//
// Segment logits go out a query row at a time: each wave stages its tile of
// dots (32 rows x 64 keys, rows padded to 65 floats so that the stores of a
// key column fall in distinct banks) in dynamic LDS, then writes each row's 64
// consecutive keys with one coalesced store.
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void shared_kernel(SharedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kBN * 256];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kD * kBN * 2];
  __shared__ int32_t s_tab[kSharedMaxBlocks];
  __shared__ __attribute__((aligned(16))) uint32_t s_wmax[kPWaves];   // each wave's report on the next tile's V
  extern __shared__ float s_lg[];            // logits asked for: [kPWaves][32][kLgStride]

  const uint32_t L = blockIdx.x, per = gridDim.x >> 3;
  const uint32_t w = (L & 7u) * per + (L >> 3);   // this XCD's run: one kv head's work together
  if (w >= (uint32_t)a.items) return;
  const int blk = (int)(w % (uint32_t)a.nblk);
  const int part = (int)((w / (uint32_t)a.nblk) % (uint32_t)a.splits);
  const int g = (int)(w / ((uint32_t)a.nblk * (uint32_t)a.splits));
  const int r0 = min(a.row_end, a.row_begin + part * a.chunk);   // this part's rows [r0, r1)
  const int r1 = min(a.row_end, r0 + a.chunk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int G = a.group;
  const int nrows = a.batch * G;
  const int row0 = blk * kPRows;
  if (row0 >= nrows) return;   // the whole work-group

  const int first = r0 >> 4;
  const int nb = r1 > r0 ? ((r1 - 1) >> 4) - first + 1 : 0;
  for (int i = tid; i < nb; i += kPThreads) s_tab[i] = a.table[first + i];

  const int rr = row0 + wave * 32 + col;
  const bool live = rr < nrows;
  const int b = rr / G, h = rr % G;
  const bool wave_live = row0 + wave * 32 + 31 < nrows;   // every row of this wave is a real query
  bf16x8 qop[8];
  if (live) {
    const uint4 *p = reinterpret_cast<const uint4 *>(a.q + ((size_t)b * a.hq + g * G + h) * kD + hf * 64);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, p[kk]);
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  __syncthreads();   // the block ids

  // block id of table entry first + ti (uniform), -1 when outside the range's
  // blocks or not a block of the pool
  auto block_id = [&](int ti) {
    const int32_t bi = __builtin_amdgcn_readfirstlane(ti < nb ? s_tab[ti] : -1);
    return bi >= 0 && (int64_t)bi < a.num_blocks ? bi : -1;
  };
  // this (block, kv head)'s 4 KiB run; the pool's first run for a skipped block
  auto run_of = [&](const uint16_t *pool, int32_t bi) {
    return reinterpret_cast<const uint8_t *>(pool) +
           (bi < 0 ? 0 : ((size_t)((uint32_t)bi * (uint32_t)a.hkv + (uint32_t)g) << 12));
  };
  const uint32_t koff = (uint32_t)(tid >> 4) * 256u + (uint32_t)(tid & 15) * 16u;
  const uint32_t voff = (uint32_t)((tid >> 4) & 3) * 1024u + (uint32_t)(tid & 15) * 16u;
  auto ld = [](const uint8_t *p, uint32_t o) { return *reinterpret_cast<const uint4 *>(p + o); };
  // the tile at t0 (a multiple of 16).  tmask bit i: key t0 + i is attended
  // (inside [r0, r1) and in a pool block; uniform).  vkeep bit u: V row u of
  // this thread is attended (the others are zeroed before the stash: p = 0
  // must not meet a non-finite value)
  auto fetch_tile = [&](int t0, uint64_t &tmask, int &vkeep) {
    const int tb = (t0 >> 4) - first;
    const int32_t b0 = block_id(tb), b1 = block_id(tb + 1), b2 = block_id(tb + 2), b3 = block_id(tb + 3);
    const uint8_t *k0 = run_of(a.k_pool, b0), *k1 = run_of(a.k_pool, b1);
    const uint8_t *k2 = run_of(a.k_pool, b2), *k3 = run_of(a.k_pool, b3);
    const int lo = max(r0 - t0, 0), hi = min(r1 - t0, kBN);   // keys t0 + [lo, hi) are in the range
    tmask = (b0 >= 0 ? 0xffffull : 0ull) | (b1 >= 0 ? 0xffffull << 16 : 0ull) | (b2 >= 0 ? 0xffffull << 32 : 0ull) |
            (b3 >= 0 ? 0xffffull << 48 : 0ull);
    tmask &= (hi >= kBN ? ~0ull : (1ull << hi) - 1ull) & ~((1ull << lo) - 1ull);
    const int32_t vb = wave == 0 ? b0 : wave == 1 ? b1 : wave == 2 ? b2 : b3;
    const uint8_t *vr = run_of(a.v_pool, vb);
    const int kv0 = t0 + 4 * (tid >> 4);
    vkeep = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) vkeep |= (vb >= 0 && kv0 + u >= r0 && kv0 + u < r1) ? 1 << u : 0;
    return Stage{ld(k0, koff), ld(k1, koff), ld(k2, koff), ld(k3, koff),
                 ld(vr, voff), ld(vr, voff + 256u), ld(vr, voff + 512u), ld(vr, voff + 768u)};
  };

  float mrun = -INFINITY, lsum = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = {};

  // raw dots of each row's segment keys inside [r0, r1), when asked for;
  // [wlo, whi) covers the segments of this wave's rows
  const bool want_lg = a.logits != nullptr;
  int wlo = 0, whi = 0;
  // this lane's row: its logits indexed by key (entry i is segment row lg0 + i)
  // and the keys it takes, [lk0, lk1); lane c of the wave holds row c's
  uint64_t lgb = 0;
  int lk0 = 0, lk1 = 0;
  if (want_lg) {
    int lg0 = 0, lg1 = 0;
    if (live) {
      lg0 = clampi(a.seg_begin[b], 0, a.row_end);
      lg1 = (int)min((int64_t)clampi(a.seg_end[b], lg0, a.row_end), (int64_t)lg0 + a.ld_logits);   // the row holds ld_logits
      lgb = reinterpret_cast<uint64_t>(a.logits + ((size_t)b * a.hq + g * G + h) * a.ld_logits - lg0);
    }
    const int k0 = max(lg0, r0), k1 = max(k0, min(lg1, r1));
    lk0 = k0;
    lk1 = k1;
    wlo = k1 > k0 ? k0 : 0x7fffffff;
    whi = k1 > k0 ? k1 : 0;
    for (int o = 32; o > 0; o >>= 1) {
      wlo = min(wlo, __shfl_xor(wlo, o));
      whi = max(whi, __shfl_xor(whi, o));
    }
  }

  const int tfirst = r0 & ~15;
  int vkeep = 0;
  uint64_t nmask = 0;
  Stage st = fetch_tile(tfirst, nmask, vkeep);
  zero_dropped_v(st, vkeep);
  int ve = first_v_exp(st, s_wmax, tid, acc);   // V scale exponent (uniform)
  for (int t0 = tfirst; t0 < r1; t0 += kBN) {
    __syncthreads();   // the previous tile's reads are done; the waves' reports on this tile are in
    stash_k(st, s_k, tid);
    ve = next_v_exp(ve, group_v_max(s_wmax), acc);
    stash_v(st, s_vt, tid, ve);
    __syncthreads();
    const uint64_t vmask = nmask;   // bit i: key t0 + i is attended
    const bool more = t0 + kBN < r1;
    if (more) st = fetch_tile(t0 + kBN, nmask, vkeep);
    // this lane half's bits: bit 8a + r of mb[bk] is key 32 bk + 8a + 4 hf + r
    // (constant shifts below; no per-lane 64-bit masks)
    const uint32_t mb0 = (uint32_t)(vmask >> (4 * hf)), mb1 = (uint32_t)(vmask >> (32 + 4 * hf));
    attend_tile(s_k, s_vt, qop, col, hf, a.scale_log2, !wave_live || vmask != ~0ull,
                [&](int bk, int j) {
                  return !live || (((bk ? mb1 : mb0) >> (8 * (j >> 2) + (j & 3))) & 1u) == 0u;
                },
                [&](const f32x16 (&s)[2]) {
                  if (!want_lg || t0 + kBN <= wlo || t0 >= whi) return;
                  float *st = s_lg + wave * (32 * kLgStride);
#pragma unroll
                  for (int bk = 0; bk < 2; ++bk)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                      st[col * kLgStride + 32 * bk + 8 * (j >> 2) + 4 * hf + (j & 3)] = s[bk][j];
                  __builtin_amdgcn_wave_barrier();
                  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                  const int key = t0 + lane;
                  const bool att = ((vmask >> lane) & 1ull) != 0ull;   // a skipped block's row: -inf
#pragma unroll
                  for (int rw = 0; rw < 32; ++rw) {
                    // row rw's base and range, from lane rw (uniform)
                    const uint32_t blo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lgb, rw);
                    const uint32_t bhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lgb >> 32), rw);
                    const int x0 = __builtin_amdgcn_readlane(lk0, rw), x1 = __builtin_amdgcn_readlane(lk1, rw);
                    float *base = reinterpret_cast<float *>(((uint64_t)bhi << 32) | blo);
                    const float v = st[rw * kLgStride + lane];
                    if (base != nullptr && key >= x0 && key < x1) base[key] = att ? v : -INFINITY;
                  }
                  __builtin_amdgcn_wave_barrier();
                  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                },
                [&] {   // the next tile: dropped rows zeroed, then the report (read after the next first barrier)
                  if (!more) return;
                  zero_dropped_v(st, vkeep);
                  report_v(st, ve, s_wmax, tid);
                },
                acc, mrun, lsum);
  }

  const float lrow = half_pair_sum(lsum);
  if (!live) return;
  unscale_v(acc, ve);
  const size_t orow = ((size_t)part * a.batch + b) * a.hq + g * G + h;
  float *o = a.out + orow * kD;
  const float lse_r = lrow > 0.f ? (mrun + __log2f(lrow)) * 0.6931471805599453f : -INFINITY;   // natural log
  if (a.accumulate) {
    // out/lse hold the attention over the other rows: the exact merge of the
    // two (each lane reads the elements it then writes; both lane halves read
    // lse before either writes it)
    const float lo = a.lse[orow];
    const float m = fmaxf(lo, lse_r);
    const float wo = m == -INFINITY ? 0.f : expf(lo - m), wr = m == -INFINITY ? 0.f : expf(lse_r - m);
    const float iz = m == -INFINITY ? 0.f : 1.f / (wo + wr);
    const float cr = lrow > 0.f ? wr * iz / lrow : 0.f, co = wo * iz;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        float4 *p = reinterpret_cast<float4 *>(o + dt * 32 + 8 * jq + 4 * hf);
        const float4 x = *p;
        *p = make_float4(x.x * co + acc[dt][4 * jq] * cr, x.y * co + acc[dt][4 * jq + 1] * cr,
                         x.z * co + acc[dt][4 * jq + 2] * cr, x.w * co + acc[dt][4 * jq + 3] * cr);
      }
    if (hf == 0) a.lse[orow] = m == -INFINITY ? -INFINITY : m + logf(wo + wr);
    return;
  }
  const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq)
      *reinterpret_cast<float4 *>(o + dt * 32 + 8 * jq + 4 * hf) =
          make_float4(acc[dt][4 * jq] * inv, acc[dt][4 * jq + 1] * inv, acc[dt][4 * jq + 2] * inv,
                      acc[dt][4 * jq + 3] * inv);
  if (hf == 0 && a.lse != nullptr) a.lse[orow] = lse_r;
}

// eight (sequence, head) rows per work-group, 32 threads of 4 floats per row;
// every thread reads all its parts before any thread writes, so out and
// lse_out may be one of the parts (in place)
__global__ __launch_bounds__(256) void merge_kernel(const float4 *o, const float *lse, int parts, int64_t rows,
                                                    float4 *out, float *lse_out) {
  const int64_t r = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int d4 = threadIdx.x & 31;
  float m = -INFINITY;
  if (r < rows)
    for (int p = 0; p < parts; ++p) m = fmaxf(m, lse[(size_t)p * rows + r]);
  float z = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < rows && m != -INFINITY)
    for (int p = 0; p < parts; ++p) {
      const float wp = expf(lse[(size_t)p * rows + r] - m);   // 0 for an empty part
      const float4 x = o[((size_t)p * rows + r) * 32 + d4];
      z += wp;
      acc.x += x.x * wp;
      acc.y += x.y * wp;
      acc.z += x.z * wp;
      acc.w += x.w * wp;
    }
  __syncthreads();
  if (r >= rows) return;
  if (m == -INFINITY) {
    out[r * 32 + d4] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d4 == 0) lse_out[r] = -INFINITY;
    return;
  }
  const float iz = 1.f / z;
  out[r * 32 + d4] = make_float4(acc.x * iz, acc.y * iz, acc.z * iz, acc.w * iz);
  if (d4 == 0) lse_out[r] = m + logf(z);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int batch, hipStream_t s) {
  if (a.group < 1 || a.max_seqlen < 1 || batch < 1) return hipErrorInvalidValue;
  PrefillArgs c = a;
  c.nblk = (int32_t)(((int64_t)a.max_seqlen * a.group + kPRows - 1) / kPRows);
  const int64_t items = (int64_t)c.nblk * a.hkv * batch;
  if (items >= 0x7ffffff0ll) return hipErrorInvalidValue;
  c.items = (int32_t)items;
  const int64_t grid = (items + 7) / 8 * 8;   // a multiple of the XCD count
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(kPThreads), 0, s, c);
  return hipGetLastError();
}

}  // namespace kvsel

namespace kvsel {

hipError_t launch_shared(const SharedArgs &a, hipStream_t s) {
  if (a.group < 1 || a.batch < 1 || a.hkv < 1 || a.row_begin < 0 || a.row_end < a.row_begin || a.splits < 1)
    return hipErrorInvalidValue;
  if (a.accumulate && (a.splits != 1 || a.lse == nullptr)) return hipErrorInvalidValue;
  if (a.row_end > a.row_begin && ((a.row_end - 1) >> 4) - (a.row_begin >> 4) + 1 > kSharedMaxBlocks)
    return hipErrorInvalidValue;
  SharedArgs c = a;
  // parts of whole 64-row tiles
  c.chunk = (int32_t)(((int64_t)(a.row_end - a.row_begin) + a.splits * kBN - 1) / (a.splits * kBN) * kBN);
  if (c.chunk < kBN) c.chunk = kBN;
  c.nblk = (int32_t)(((int64_t)a.batch * a.group + kPRows - 1) / kPRows);
  const int64_t items = (int64_t)c.nblk * a.hkv * a.splits;
  if (items >= 0x7ffffff0ll) return hipErrorInvalidValue;
  c.items = (int32_t)items;
  const int64_t grid = (items + 7) / 8 * 8;   // a multiple of the XCD count
  const int dyn = a.logits != nullptr ? kPWaves * 32 * kLgStride * (int)sizeof(float) : 0;
  if (dyn > 0) {
    const hipError_t e = allow_dynamic_lds((const void *)shared_kernel, dyn);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(shared_kernel, dim3((unsigned)grid), dim3(kPThreads), dyn, s, c);
  return hipGetLastError();
}

hipError_t launch_merge(const float *o, const float *lse, int parts, int64_t rows, float *out, float *lse_out,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (parts < 1 || parts > kMaxMergeParts) return hipErrorInvalidValue;
  const int64_t blocks = (rows + 7) / 8;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4 *>(o), lse,
                     parts, rows, reinterpret_cast<float4 *>(out), lse_out);
  return hipGetLastError();
}

}  // namespace kvsel
