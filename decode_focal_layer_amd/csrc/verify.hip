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
//    query rows as the B columns (as in the window scoring), so each lane
//    holds one query column and 16 keys of every 32-key tile.
//  * an online softmax per column (fp32, running max and sum per lane);
//  * O^T += V^T P with the same instruction: A = V^T (the tile's V rows,
//    transposed through LDS), B = P, where P is split into a bf16 high part
//    and a bf16 remainder (two products), so P keeps about 16 significant
//    bits; bf16 V is exact.
// Four waves per work-group take the 32-row tiles in turn and merge their
// (max, sum, O) through LDS at the end.  The causal mask needs no positions:
// the segment is cut at n - m, so the drafts are the last m attended rows
// and virtual row j >= cnt - m is draft j - (cnt - m), visible to draft r
// when that is <= r.
#include "common.h"
#include "kvsel_internal.h"
#include "mfma_kernels.h"

namespace kvsel {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kVThreads = 256;
constexpr int kVWaves = kVThreads / 64;
constexpr int kVtStride = 40;   // bf16 per transposed V row (32 keys + pad, 16-byte aligned rows)

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

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

// transposed V row of dim d: dims d and d + 8 (the two lane halves' dims of
// one load) in adjacent rows, so their writes fall in different banks
__device__ __forceinline__ int vt_row(int d) { return (d & ~15) + (d & 7) * 2 + ((d >> 3) & 1); }

// LDS: the rows and the V^T tiles while the tiles run, then the same bytes
// hold the waves' partial outputs for the merge (two work-groups per CU)
constexpr size_t kRowBytes = sizeof(uint32_t) * kVerifyMaxRows;
constexpr size_t kVtBytes = sizeof(uint16_t) * kVWaves * 128 * kVtStride;
constexpr size_t kOBytes = sizeof(float) * kVWaves * 32 * 129;
constexpr size_t kVLds = kRowBytes + kVtBytes > kOBytes ? kRowBytes + kVtBytes : kOBytes;

__global__ __launch_bounds__(kVThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void verify_kernel(VerifyArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int G = a.group, R = a.m * G;

  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kVLds];
  __shared__ float s_m[kVWaves][32], s_l[kVWaves][32];
  uint32_t *s_prow = reinterpret_cast<uint32_t *>(s_raw);
  uint16_t(*s_vt)[128 * kVtStride] = reinterpret_cast<uint16_t(*)[128 * kVtStride]>(s_raw + kRowBytes);
  float(*s_o)[32][129] = reinterpret_cast<float(*)[32][129]>(s_raw);

  // ---- rows: kept (segment-relative idx), before the segment, after it ----
  const int cap = a.max_blocks * kBlk;
  const int n = clampi(a.seq_len[b], 0, cap);
  const int lim = max(n - a.m, 0);   // the segment ends before the drafts: they are always attended
  const int s0 = clampi(a.seg_begin[b], 0, lim);
  const int s1 = clampi(a.seg_end[b], s0, lim);
  const int cnt = min(a.k + s0 + (n - s1), kVerifyMaxRows);
  const int32_t *tab = a.block_table + (size_t)b * a.max_blocks;
  const int32_t *ib = a.k > 0 ? a.idx + ((size_t)b * a.hkv + g) * a.k : nullptr;
  for (int j = tid; j < cnt; j += kVThreads) {
    int row;
    if (j < a.k) {
      const int r = ib[j];
      row = (r >= 0 && r < s1 - s0) ? s0 + r : -1;
    } else if (j < a.k + s0) {
      row = j - a.k;
    } else {
      row = s1 + (j - a.k - s0);
    }
    uint32_t pr = kNoRow;
    if (row >= 0) {
      const int blk = tab[row >> 4];
      if (blk >= 0 && (int64_t)blk < a.num_blocks)
        pr = ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
    }
    s_prow[j] = pr;
  }

  // ---- this lane's query column (B operand of k-step kk: dims kk*16 + hf*8 .. +8,
  // so the two lane halves of a key read adjacent 16-byte pieces) ----
  bf16x8 qop[8];
  const int qr = col / max(G, 1), qh = col % max(G, 1);
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
  uint16_t *vt = s_vt[wave];
  const int last_vis = cnt - a.m + qr;  // virtual index of this column's draft: the last it sees

  // K and V of key t0 + col, this lane's half of the dims (invalid: the query row, masked).
  // Software pipelined: the next tile's loads are issued once this tile's
  // K has gone into S and its V into LDS, and land during softmax and P V.
  bf16x8 kop[8];
  uint4 vv[8];
  uint32_t tile_mask = 0;   // bit i: key t0 + i of the loaded tile is attended
  auto load_tile = [&](int t0) {
    const int key = t0 + col;
    const uint32_t pr = key < cnt ? s_prow[key] : kNoRow;
    tile_mask = (uint32_t)__ballot(pr != kNoRow);   // lanes 0..31 (hf = 0) cover the 32 keys
    const uint16_t *krow = pr != kNoRow ? a.k_pool + (size_t)pr * kD : a.q;
    const uint16_t *vrow = pr != kNoRow ? a.v_pool + (size_t)pr * kD : a.q;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kop[kk] = __builtin_bit_cast(bf16x8, reinterpret_cast<const uint4 *>(krow + hf * 8)[2 * kk]);
      vv[kk] = reinterpret_cast<const uint4 *>(vrow + hf * 8)[2 * kk];
    }
  };
  if (wave * 32 < cnt) load_tile(wave * 32);

  for (int t0 = wave * 32; t0 < cnt; t0 += kVWaves * 32) {
    const uint32_t vmask = tile_mask;
    // V transposed into this wave's LDS: vt[vt_row(d)][key]
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint32_t w4[4] = {vv[kk].x, vv[kk].y, vv[kk].z, vv[kk].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = kk * 16 + hf * 8 + e;
        const uint32_t word = w4[e >> 1];
        vt[vt_row(d) * kVtStride + col] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    }
    // S = K Q^T: d[j] is key t0 + 8*(j/4) + 4*hf + j%4, query column col
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[kk], s, 0, 0, 0);
    if (t0 + kVWaves * 32 < cnt) load_tile(t0 + kVWaves * 32);
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
    tm = fmaxf(tm, __shfl_xor(tm, 32));   // the column's other 16 keys
    const float mnew = fmaxf(mrun, tm);
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mrun - mnew);
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = x[j] == -INFINITY ? 0.f : fast_exp2(x[j] - mnew);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ps += p[j];
    lsum = lsum * alpha + ps;
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[dt][j] *= alpha;
    // P as the B operand: keys hf*8 .. +8 (first product), 16 + hf*8 .. +8 (second)
    float send[8], recv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      send[i] = hf ? p[i] : p[4 + i];
      send[4 + i] = hf ? p[8 + i] : p[12 + i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) recv[i] = __shfl_xor(send[i], 32);
    float b1[8], b2[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b1[i] = hf ? recv[i] : p[i];
      b1[4 + i] = hf ? p[4 + i] : recv[i];
      b2[i] = hf ? recv[4 + i] : p[8 + i];
      b2[4 + i] = hf ? p[12 + i] : recv[4 + i];
    }
    bf16x8 b1h, b1l, b2h, b2l;
    split8(b1, b1h, b1l);
    split8(b2, b2h, b2l);
    __builtin_amdgcn_wave_barrier();   // this wave's V^T writes before its reads
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = dt * 32 + col;
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(vt + vt_row(d) * kVtStride + hf * 8);
      const bf16x8 a2 = *reinterpret_cast<const bf16x8 *>(vt + vt_row(d) * kVtStride + 16 + hf * 8);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1h, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1l, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2h, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2l, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();   // reads done before the next tile's writes
  }

  // ---- merge: the column's two half-sums, then the waves ----
  const float lcol = lsum + __shfl_xor(lsum, 32);
  __syncthreads();   // every wave is done with the rows and V^T before s_o overwrites them
  if (hf == 0) {
    s_m[wave][col] = mrun;
    s_l[wave][col] = lcol;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) s_o[wave][col][dt * 32 + 8 * (j >> 2) + 4 * hf + (j & 3)] = acc[dt][j];
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
      A += s_o[w][c][d] * f;
    }
    const int r = c / G, h = c % G;
    const size_t ob = ((size_t)b * a.m + r) * a.hq + g * G + h;
    a.out[ob * kD + d] = L > 0.f ? A / L : 0.f;
    if (d == 0 && a.lse != nullptr) a.lse[ob] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs &a, int batch, hipStream_t s) {
  if (a.m < 1 || a.group < 1 || a.m * a.group > 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_kernel, dim3(a.hkv, batch), dim3(kVThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
