// Draft verification attention on MFMA.
//
// HPD-Parsing wiki (P-MTP): each branch drafts several tokens and verifies
// them in parallel, accepting several per step.  The m drafts' queries
// (positions n-m .. n-1 of a branch whose last m rows are the drafts' own
// K/V) attend over the branch's attended rows -- the kept visual rows, every
// row outside the candidate segment -- and, causally, over the drafts up to
// their own position.
//
// For one (sequence, kv head) the m drafts x G heads form R <= 32 query rows
// (column c = r * G + h), a dense (keys x 128) * (128 x R) contraction:
//  * S = K Q^T with v_mfma_f32_32x32x16_bf16, the keys as the A rows and the
//    query rows as the B columns, so each lane holds one query column and 16
//    keys of every 32-key tile;
//  * an online softmax per column (fp32, running max and sum per lane; the
//    max moves only when it grows by more than 8 in log2 units, so O is
//    rarely rescaled and P stays below 256);
//  * O^T += V^T P with the same instruction: A = V^T (the tile's V rows,
//    transposed through LDS), B = P, where P is split into a bf16 high part
//    and a bf16 remainder (two products), so P keeps about 16 significant
//    bits; bf16 V is exact.
// Four waves per work-group take the 32-key tiles in turn, each with its own
// LDS tile: K arrives by coalesced loads (16 lanes per 256-byte row) and is
// read back in operand order; V is loaded in operand order (the two lane
// halves of a key read adjacent 16-byte pieces) and written transposed, its
// keys placed so that P leaves the S product already in operand order.  The
// next tile's K/V are loaded during the current tile's softmax and P V.  The
// waves merge their (max, sum, O) through LDS at the end.  The causal mask
// needs no positions: the segment is cut at n - m, so the drafts are the last
// m attended rows and virtual row j >= cnt - m is draft j - (cnt - m),
// visible to draft r when that is <= r.
#include "common.h"
#include "kvsel_internal.h"
#include "mfma_common.h"
#include "mfma_kernels.h"

namespace kvsel {

namespace {

constexpr int kVThreads = 256;
constexpr int kVWaves = kVThreads / 64;
constexpr float kSlack = 8.f;   // log2 headroom of the running max

// per-wave LDS tile of 32 keys: K [32 keys][16 chunks of 16 B], chunk c of
// key r in slot c ^ (r & 15); V^T [128 dims][32 positions] bf16, 64-byte
// rows, the 16-byte blocks of row q XOR-swizzled by q >> 2
constexpr int kKtBytes = 32 * 256;
constexpr int kVtBytes = kD * 32 * 2;
constexpr int kWaveTile = kKtBytes + kVtBytes;
constexpr int kTilesBytes = kVWaves * kWaveTile;   // the merge buffer reuses these bytes
static_assert(sizeof(float) * kVWaves * 32 * kD <= (size_t)kTilesBytes, "merge buffer");

__device__ __forceinline__ int kt_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// V^T row of dim d: dims d and d + 8 (the two lane halves' dims of one load)
// in adjacent rows
__device__ __forceinline__ int vt_row(int d) { return (d & ~15) + (d & 7) * 2 + ((d >> 3) & 1); }

// byte offset of V^T element (dim d, position p)
__device__ __forceinline__ int vt_off(int d, int p) {
  const int q = vt_row(d);
  return q * 64 + ((((p >> 3) ^ (q >> 2)) & 3) << 4) + (p & 7) * 2;
}

// position of tile key r = 8a + 4h + i: S leaves it in lane half h, register
// 4a + i; k-step s of P V takes registers 8s .. 8s+7 of each lane half as
// k-indices 8h .. 8h+7, so the key goes to position 16(a>>1) + 8h + 4(a&1) + i
__device__ __forceinline__ int key_pos(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + i;
}

// 8 floats -> high bf16 parts and bf16 remainders, packed as MFMA operands
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_rne(x[2 * i]), h1 = bf16_rne(x[2 * i + 1]);
    const uint32_t l0 = bf16_rne(x[2 * i] - bf16_val(h0)), l1 = bf16_rne(x[2 * i + 1] - bf16_val(h1));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

__global__ __launch_bounds__(kVThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void verify_kernel(VerifyArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int G = a.group, R = min(a.m * G - a.col0, 32);   // this block's columns: a.col0 + [0, R)

  __shared__ __attribute__((aligned(16))) uint8_t s_tiles[kTilesBytes];
  __shared__ float s_m[kVWaves][32], s_l[kVWaves][32];
  extern __shared__ uint32_t s_prow[];   // a.rows_cap physical rows
  uint8_t *kt = s_tiles + wave * kWaveTile;
  uint8_t *vt = kt + kKtBytes;

  // ---- rows: kept (segment-relative idx), before the segment, after it ----
  const int cap = a.max_blocks * kBlk;
  const int n = clampi(a.seq_len[b], 0, cap);
  const int lim = max(n - a.m, 0);   // the segment ends before the drafts: they are always attended
  const int s0 = clampi(a.seg_begin[b], 0, lim);
  const int s1 = clampi(a.seg_end[b], s0, lim);
  const int cnt = min(a.k + s0 + (n - s1), a.rows_cap);
  const int32_t *tab = a.block_table + (size_t)b * a.max_blocks;
  const int32_t *ib = a.k > 0 ? a.idx + ((size_t)b * a.hkv + g) * a.k : nullptr;
  // 8 rows per thread per batch: all index loads in flight together, then
  // all block-table loads (two memory latencies per 2048 rows)
  constexpr int kRB = 8;
  for (int j0 = 0; j0 < cnt; j0 += kRB * kVThreads) {
    int kidx[kRB], row[kRB], blk[kRB];
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kVThreads + tid;
      kidx[u] = (j < cnt && j < a.k) ? ib[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kVThreads + tid;
      if (j >= cnt) row[u] = -1;
      else if (j < a.k) row[u] = (kidx[u] >= 0 && kidx[u] < s1 - s0) ? s0 + kidx[u] : -1;
      else if (j < a.k + s0) row[u] = j - a.k;
      else row[u] = s1 + (j - a.k - s0);
    }
#pragma unroll
    for (int u = 0; u < kRB; ++u) blk[u] = row[u] >= 0 ? tab[row[u] >> 4] : -1;
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kVThreads + tid;
      if (j < cnt) {
        uint32_t pr = kNoRow;
        if (blk[u] >= 0 && (int64_t)blk[u] < a.num_blocks)
          pr = ((uint32_t)blk[u] * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row[u] & 15);
        KVSEL_CHECK(j < a.rows_cap, kDbgLds, j);
        s_prow[j] = pr;
      }
    }
  }

  // ---- this lane's query column (B operand of k-step kk: dims kk*16 + hf*8 .. +8) ----
  bf16x8 qop[8];
  const int qr = (a.col0 + col) / G, qh = (a.col0 + col) % G;   // the column's draft and head
  if (col < R) {
    const uint4 *p = reinterpret_cast<const uint4 *>(a.q + (((size_t)b * a.m + qr) * a.hq + g * G + qh) * kD + hf * 8);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, p[2 * kk]);
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  __syncthreads();

  float mrun = -INFINITY, lsum = 0.f;   // this column's running max and this lane's share of the sum
  f32x16 acc[4];                        // O^T tiles: dims dt*32 + 8*(j/4) + 4*hf + j%4, this column
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = {};
  const int last_vis = cnt - a.m + qr;  // virtual index of this column's draft: the last it sees

  // The tile's K: load i brings keys 4i .. 4i+3, 16 lanes per 256-byte row.
  // Its V: key t0 + col, dims kk*16 + hf*8 .. +8 (the lane's operand order).
  // A row not attended reads the queries (valid memory) and is masked.
  // (written out load by load: the staging stays in registers)
  uint4 k0, k1, k2, k3, k4, k5, k6, k7, vv[8];
  uint32_t tile_mask = 0;   // bit i: key t0 + i of the loaded tile is attended
  auto krow_of = [&](int kr) {   // K row (16-byte pieces) of virtual row kr, or the queries
    const uint32_t pk_r = s_prow[max(min(kr, cnt - 1), 0)];   // unbranched LDS read
    const uint32_t pk = kr < cnt ? pk_r : kNoRow;
    return reinterpret_cast<const uint4 *>(pk != kNoRow ? a.k_pool + (size_t)pk * kD : a.q);
  };
#define KVSEL_VERIFY_LOAD_TILE(T0)                                                                   \
  do {                                                                                               \
    const int t0_ = (T0);                                                                            \
    const int key_ = t0_ + col;                                                                      \
    const uint32_t prr_ = s_prow[max(min(key_, cnt - 1), 0)]; /* unbranched LDS read */              \
    const uint32_t pr_ = key_ < cnt ? prr_ : kNoRow;                                                 \
    tile_mask = (uint32_t)__ballot(pr_ != kNoRow); /* lanes 0..31 (hf = 0) cover the 32 keys */      \
    const uint4 *vrow_ = reinterpret_cast<const uint4 *>((pr_ != kNoRow ? a.v_pool + (size_t)pr_ * kD \
                                                                        : a.q) + hf * 8);            \
    vv[0] = vrow_[0]; vv[1] = vrow_[2]; vv[2] = vrow_[4]; vv[3] = vrow_[6];                          \
    vv[4] = vrow_[8]; vv[5] = vrow_[10]; vv[6] = vrow_[12]; vv[7] = vrow_[14];                       \
    const int kr_ = t0_ + (lane >> 4), c_ = lane & 15;                                               \
    k0 = krow_of(kr_)[c_]; k1 = krow_of(kr_ + 4)[c_]; k2 = krow_of(kr_ + 8)[c_];                     \
    k3 = krow_of(kr_ + 12)[c_]; k4 = krow_of(kr_ + 16)[c_]; k5 = krow_of(kr_ + 20)[c_];              \
    k6 = krow_of(kr_ + 24)[c_]; k7 = krow_of(kr_ + 28)[c_];                                          \
  } while (0)
  if (wave * 32 < cnt) KVSEL_VERIFY_LOAD_TILE(wave * 32);

  const int vpos = key_pos(col);
  for (int t0 = wave * 32; t0 < cnt; t0 += kVWaves * 32) {
    const uint32_t vmask = tile_mask;
    // this wave's tile into its LDS (the wave's own earlier reads are done:
    // a wave's LDS accesses complete in order)
    {
      const int r = lane >> 4, c = lane & 15;
      *reinterpret_cast<uint4 *>(kt + kt_off(r, c)) = k0;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 4, c)) = k1;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 8, c)) = k2;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 12, c)) = k3;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 16, c)) = k4;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 20, c)) = k5;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 24, c)) = k6;
      *reinterpret_cast<uint4 *>(kt + kt_off(r + 28, c)) = k7;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t w = word_of(vv[kk], e2);
        const int d = kk * 16 + hf * 8 + 2 * e2;
        *reinterpret_cast<uint16_t *>(vt + vt_off(d, vpos)) = (uint16_t)(w & 0xffffu);
        *reinterpret_cast<uint16_t *>(vt + vt_off(d + 1, vpos)) = (uint16_t)(w >> 16);
      }
    __builtin_amdgcn_wave_barrier();
    // the staging registers are free again: the next tile's loads go out now
    // and land during this tile's S, softmax and P V
    if (t0 + kVWaves * 32 < cnt) KVSEL_VERIFY_LOAD_TILE(t0 + kVWaves * 32);

    // S = K Q^T: s[j] is key t0 + 8*(j/4) + 4*hf + j%4, query column col
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(kt + kt_off(col, 2 * kk + hf));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], s, 0, 0, 0);
    }

    float x[16];
    float tm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      // attended, a real column, and not a draft after this column's own
      // (a row before the drafts always passes the last test)
      const int kr = 8 * (j >> 2) + 4 * hf + (j & 3);
      const bool vis = (((vmask >> kr) & 1u) != 0) & (col < R) & (t0 + kr <= last_vis);
      x[j] = vis ? s[j] * a.scale_log2 : -INFINITY;
      tm = fmaxf(tm, x[j]);
    }
    tm = half_pair_max(tm);
    // the running max moves only when a column's max grows by more than
    // kSlack (log2 units): p stays below 2^kSlack and O is rarely rescaled
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
    const float neg = mrun == -INFINITY ? 0.f : -mrun;   // a column that has seen nothing keeps p = 0
    float p0[8], p1[8];   // registers 0..7 and 8..15: the two k-steps of P V
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p0[j] = fast_exp2(x[j] + neg);
      p1[j] = fast_exp2(x[8 + j] + neg);
      ps += p0[j] + p1[j];
    }
    lsum += ps;
    // P as the B operand: k-step s takes this lane's registers 8s .. 8s+7
    bf16x8 b1h, b1l, b2h, b2l;
    split8(p0, b1h, b1l);
    split8(p1, b2h, b2l);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = dt * 32 + col;
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(vt + vt_off(d, hf * 8));
      const bf16x8 a2 = *reinterpret_cast<const bf16x8 *>(vt + vt_off(d, 16 + hf * 8));
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1h, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1l, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2h, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2l, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

#undef KVSEL_VERIFY_LOAD_TILE

  // ---- merge: the column's two half-sums, then the waves ----
  const float lcol = half_pair_sum(lsum);
  __syncthreads();   // every wave is done with its tile before s_o overwrites the tiles
  float *s_o = reinterpret_cast<float *>(s_tiles);   // [wave][column][dim ^ column]
  if (hf == 0) {
    s_m[wave][col] = mrun;
    s_l[wave][col] = lcol;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int d = dt * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
      s_o[(wave * 32 + col) * kD + (d ^ col)] = acc[dt][j];
    }
  __syncthreads();
  for (int x = tid; x < R * kD; x += kVThreads) {
    const int c = x / kD, d = x % kD;
    float M = s_m[0][c];
#pragma unroll
    for (int w = 1; w < kVWaves; ++w) M = fmaxf(M, s_m[w][c]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) {
      const float f = s_m[w][c] == -INFINITY ? 0.f : fast_exp2(s_m[w][c] - M);
      L += s_l[w][c] * f;
      A += s_o[(w * 32 + c) * kD + (d ^ c)] * f;
    }
    const int r = (a.col0 + c) / G, h = (a.col0 + c) % G;
    const size_t ob = ((size_t)b * a.m + r) * a.hq + g * G + h;
    a.out[ob * kD + d] = L > 0.f ? A / L : 0.f;
    if (d == 0 && a.lse != nullptr) a.lse[ob] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Up to 16 query columns (m * G <= 16): 16x16 MFMA tiles of 16 keys per wave.
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16: lane (kl, kb) = (lane & 15,
// lane >> 4) supplies K[key kl][32s + 8kb ..] and Q[column kl][32s + 8kb ..]
// and receives S for keys 4kb .. 4kb+3 of column kl -- exactly the P values
// it supplies as the B operand of v_mfma_f32_16x16x16_bf16 for O^T += V^T P,
// whose A operand (V^T[d][keys 4kb ..]) comes from a 4 KiB per-wave LDS
// tile.  Half the accumulators of the 32-column kernel: 16 waves per CU.
// ---------------------------------------------------------------------------

// threads per (branch, kv head) work-group: 256 ran draft verification at the
// C4 shape (4096 pairs of ~720 rows) at 110.3 against 109.4 steps/s for 512
#ifndef KVSEL_W16_THREADS
#define KVSEL_W16_THREADS 256
#endif
constexpr int kW16Threads = KVSEL_W16_THREADS;
constexpr int kW16Waves = kW16Threads / 64;
constexpr int kVt16Bytes = kD * 16 * 2;   // V^T [128 dims][16 keys] bf16 per wave
constexpr int kO16Bytes = (int)sizeof(float) * kW16Waves * 16 * kD;
constexpr int kLds16 = kW16Waves * kVt16Bytes > kO16Bytes ? kW16Waves * kVt16Bytes : kO16Bytes;

// byte offset of V^T element (dim d, key r): 32-byte rows of four 8-byte
// groups of 4 keys, the groups XOR-swizzled by (d >> 3) & 3
__device__ __forceinline__ int vt16_off(int d, int r) {
  return d * 32 + ((((r >> 2) ^ (d >> 3)) & 3) << 3) + (r & 3) * 2;
}

// 4 floats -> high bf16 parts and bf16 remainders
__device__ __forceinline__ void split4(const float (&x)[4], s16x4 &hi, s16x4 &lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t h0 = bf16_rne(x[2 * i]), h1 = bf16_rne(x[2 * i + 1]);
    const uint32_t l0 = bf16_rne(x[2 * i] - bf16_val(h0)), l1 = bf16_rne(x[2 * i + 1] - bf16_val(h1));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(s16x4, make_uint2(h[0], h[1]));
  lo = __builtin_bit_cast(s16x4, make_uint2(l[0], l[1]));
}

__global__ __launch_bounds__(kW16Threads) __attribute__((amdgpu_waves_per_eu(4, 4))) void verify16_kernel(VerifyArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kl = lane & 15, kb = lane >> 4;
  const int G = a.group, R = a.m * G;

  __shared__ __attribute__((aligned(16))) uint8_t s_tiles[kLds16];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[16 * kD * 2];   // [column][16-byte chunk c ^ column]
  __shared__ float s_m[kW16Waves][16], s_l[kW16Waves][16];
  extern __shared__ uint32_t s_prow[];   // a.rows_cap physical rows
  uint8_t *vt = s_tiles + wave * kVt16Bytes;

  // ---- rows: kept (segment-relative idx), before the segment, after it ----
  const int cap = a.max_blocks * kBlk;
  const int n = clampi(a.seq_len[b], 0, cap);
  const int lim = max(n - a.m, 0);   // the segment ends before the drafts: they are always attended
  const int s0 = clampi(a.seg_begin[b], 0, lim);
  const int s1 = clampi(a.seg_end[b], s0, lim);
  const int cnt = min(a.k + s0 + (n - s1), a.rows_cap);
  const int32_t *tab = a.block_table + (size_t)b * a.max_blocks;
  const int32_t *ib = a.k > 0 ? a.idx + ((size_t)b * a.hkv + g) * a.k : nullptr;
  constexpr int kRB = 8;   // rows per thread per batch: index loads together, then table loads
  for (int j0 = 0; j0 < cnt; j0 += kRB * kW16Threads) {
    int kidx[kRB], row[kRB], blk[kRB];
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kW16Threads + tid;
      kidx[u] = (j < cnt && j < a.k) ? ib[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kW16Threads + tid;
      if (j >= cnt) row[u] = -1;
      else if (j < a.k) row[u] = (kidx[u] >= 0 && kidx[u] < s1 - s0) ? s0 + kidx[u] : -1;
      else if (j < a.k + s0) row[u] = j - a.k;
      else row[u] = s1 + (j - a.k - s0);
    }
#pragma unroll
    for (int u = 0; u < kRB; ++u) blk[u] = row[u] >= 0 ? tab[row[u] >> 4] : -1;
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int j = j0 + u * kW16Threads + tid;
      if (j < cnt) {
        uint32_t pr = kNoRow;
        if (blk[u] >= 0 && (int64_t)blk[u] < a.num_blocks)
          pr = ((uint32_t)blk[u] * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row[u] & 15);
        KVSEL_CHECK(j < a.rows_cap, kDbgLds, j);
        s_prow[j] = pr;
      }
    }
  }

  // ---- the queries into LDS (column c: draft c / G, head c % G; zero past R) ----
  const int qr = kl / G;
  for (int x = tid; x < 16 * 16; x += kW16Threads) {
    const int c = x >> 4, ch = x & 15;   // column, 16-byte chunk
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c < R)
      v = reinterpret_cast<const uint4 *>(a.q + (((size_t)b * a.m + c / G) * a.hq + g * G + c % G) * kD)[ch];
    *reinterpret_cast<uint4 *>(s_q + c * 256 + ((ch ^ c) << 4)) = v;
  }
  __syncthreads();
  // B operand of S step s for column kl: dims 32s + 8kb .. +8 = chunk 4s + kb
  auto qop = [&](int st) {
    return *reinterpret_cast<const bf16x8 *>(s_q + kl * 256 + (((4 * st + kb) ^ kl) << 4));
  };

  float mrun = -INFINITY, lsum = 0.f;   // column kl's running max; this lane's share of its sum
  f32x4 acc[8];                         // O^T rows dt*16 + 4kb + j, column kl
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = {};
  const int last_vis = cnt - a.m + qr;  // virtual index of this column's draft: the last it sees

  // key t0 + kl: K and V pieces 32s + 8kb (64 contiguous bytes per row and
  // load); a row not attended reads the queries (valid memory) and is masked
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
  uint32_t tile_mask = 0;   // bit i: key t0 + i of the loaded tile is attended
#define KVSEL_VERIFY16_LOAD(T0)                                                                      \
  do {                                                                                               \
    const int key_ = (T0) + kl;                                                                      \
    const uint32_t prr_ = s_prow[max(min(key_, cnt - 1), 0)]; /* unbranched LDS read */              \
    const uint32_t pr_ = key_ < cnt ? prr_ : kNoRow;                                                 \
    tile_mask = (uint32_t)__ballot(pr_ != kNoRow) & 0xffffu; /* lanes 0..15 cover the 16 keys */     \
    const uint4 *kr_ = reinterpret_cast<const uint4 *>((pr_ != kNoRow ? a.k_pool + (size_t)pr_ * kD  \
                                                                      : a.q) + kb * 8);              \
    const uint4 *vr_ = reinterpret_cast<const uint4 *>((pr_ != kNoRow ? a.v_pool + (size_t)pr_ * kD  \
                                                                      : a.q) + kb * 8);              \
    k0 = kr_[0]; k1 = kr_[4]; k2 = kr_[8]; k3 = kr_[12];                                             \
    v0 = vr_[0]; v1 = vr_[4]; v2 = vr_[8]; v3 = vr_[12];                                             \
  } while (0)
  if (wave * 16 < cnt) KVSEL_VERIFY16_LOAD(wave * 16);

  for (int t0 = wave * 16; t0 < cnt; t0 += kW16Waves * 16) {
    const uint32_t vmask = tile_mask;
    // V^T of this wave's tile (the wave's own earlier reads are done)
    {
      const uint4 vs[4] = {v0, v1, v2, v3};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t w = word_of(vs[i], e2);
          const int d = 32 * i + 8 * kb + 2 * e2;
          *reinterpret_cast<uint16_t *>(vt + vt16_off(d, kl)) = (uint16_t)(w & 0xffffu);
          *reinterpret_cast<uint16_t *>(vt + vt16_off(d + 1, kl)) = (uint16_t)(w >> 16);
        }
    }
    __builtin_amdgcn_wave_barrier();
    // S^T = K Q^T: s[j] is key t0 + 4kb + j, column kl
    f32x4 s = {};
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0), qop(0), s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1), qop(1), s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k2), qop(2), s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k3), qop(3), s, 0, 0, 0);
    // the staging registers are free: the next tile's loads go out now
    if (t0 + kW16Waves * 16 < cnt) KVSEL_VERIFY16_LOAD(t0 + kW16Waves * 16);

    float x[4];
    float tm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * kb + j;
      const bool vis = (((vmask >> r) & 1u) != 0) & (kl < R) & (t0 + r <= last_vis);
      x[j] = vis ? s[j] * a.scale_log2 : -INFINITY;
      tm = fmaxf(tm, x[j]);
    }
    tm = half_pair_max(row_pair_max(tm));   // over the column's 16 keys (lanes kl + 16 kb)
    if (__ballot(tm > mrun + kSlack) != 0) {
      const float mnew = fmaxf(mrun, tm);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[dt][j] *= alpha;
    }
    const float neg = mrun == -INFINITY ? 0.f : -mrun;   // a column that has seen nothing keeps p = 0
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(x[j] + neg);
      lsum += p[j];
    }
    s16x4 ph, pl;
    split4(p, ph, pl);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const s16x4 av = *reinterpret_cast<const s16x4 *>(vt + vt16_off(dt * 16 + kl, 4 * kb));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, ph, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pl, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }
#undef KVSEL_VERIFY16_LOAD

  // ---- merge: the column's four lane shares, then the waves ----
  const float lcol = half_pair_sum(row_pair_sum(lsum));
  __syncthreads();   // every wave is done with its tile before s_o overwrites the tiles
  float *s_o = reinterpret_cast<float *>(s_tiles);   // [wave][column][dim ^ 4 column]
  if (kb == 0) {
    s_m[wave][kl] = mrun;
    s_l[wave][kl] = lcol;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = dt * 16 + 4 * kb + j;
      s_o[(wave * 16 + kl) * kD + (d ^ (kl << 2))] = acc[dt][j];
    }
  __syncthreads();
  for (int x = tid; x < R * kD; x += kW16Threads) {
    const int c = x / kD, d = x % kD;
    float M = s_m[0][c];
#pragma unroll
    for (int w = 1; w < kW16Waves; ++w) M = fmaxf(M, s_m[w][c]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kW16Waves; ++w) {
      const float f = s_m[w][c] == -INFINITY ? 0.f : fast_exp2(s_m[w][c] - M);
      L += s_l[w][c] * f;
      A += s_o[(w * 16 + c) * kD + (d ^ (c << 2))] * f;
    }
    const int r = c / G, h = c % G;
    const size_t ob = ((size_t)b * a.m + r) * a.hq + g * G + h;
    a.out[ob * kD + d] = L > 0.f ? A / L : 0.f;
    if (d == 0 && a.lse != nullptr) a.lse[ob] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs &a0, int batch, hipStream_t s) {
  if (a0.m < 1 || a0.group < 1 || a0.rows_cap < 1 || a0.rows_cap > kVerifyMaxRows) return hipErrorInvalidValue;
  // the row table is dynamic LDS beside up to 70 KiB of static LDS (allowed once per device)
  for (const void *f : {(const void *)verify_kernel, (const void *)verify16_kernel}) {
    const hipError_t e = allow_dynamic_lds(f, kVerifyMaxRows * (int)sizeof(uint32_t));
    if (e != hipSuccess) return e;
  }
  const size_t dyn = (size_t)a0.rows_cap * sizeof(uint32_t);
  if (a0.m * a0.group <= 16) {
    VerifyArgs a = a0;
    a.col0 = 0;
    hipLaunchKernelGGL(verify16_kernel, dim3(a.hkv, batch), dim3(kW16Threads), dyn, s, a);
    return hipGetLastError();
  }
  // query columns (draft x group head) 32 at a time: the columns are
  // independent, each launch reads the branch's rows once more
  for (int c0 = 0; c0 < a0.m * a0.group; c0 += 32) {
    VerifyArgs a = a0;
    a.col0 = c0;
    hipLaunchKernelGGL(verify_kernel, dim3(a.hkv, batch), dim3(kVThreads), dyn, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvsel
