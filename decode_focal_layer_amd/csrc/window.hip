// FastKV window saliency on MFMA (FastKV section 2A, Token-Selective
// Propagation: the attention weights from a recent window of queries to all
// context tokens, averaged, rank the tokens).
//
// For one (sequence, kv head) the window rows x group heads form R query
// rows (row index qr = r * G + h; window row r is the query of position
// n - W + r and, when causal, sees keys <= that position), taken 32 at a time:
// each pass below covers rows [qr0, qr0 + 32), and a pass after the first adds
// its scores to the partial row the earlier ones wrote.  The
// logits Q K^T are a dense (R x 128) * (128 x keys) contraction in bf16 with
// fp32 accumulation, computed with v_mfma_f32_32x32x16_bf16.
//
// Two passes over K:
//   pass 1 (stats): grid (key tiles, kv heads, sequences).  MFMA with the keys
//     as the A rows and the query rows as the B columns, so each lane holds one
//     query row and 16 keys of every 32-key block: the per-row reference
//     mc = max(dot) * c (fp32, c = scale * log2 e) and the sum of
//     2^(dot * c - mc) stay lane-local.  Each exponent is one fused multiply-add
//     rounded once (relative error of the term about 2^-24 |exponent| ln 2);
//     the 16 terms of a block are added in fp32, the blocks in fp64.  Each tile
//     writes (reference, sum) per query row.
//   merge: one small kernel combines the tiles' statistics per query row in
//     fp64 into (reference, 1 / sum);
//   pass 2 (scores): MFMA with the query rows as A and the keys as B, so each
//     lane holds one key and 16 query rows: the probabilities
//     2^(dot * c - mc) / sum, the same exponent as in pass 1, are summed over
//     the rows lane-locally in fp64, then across the two half-waves.
//   The fp64 per-(kv head) scores feed the group-sum / pool post-pass.
//
// The head dimension is permuted identically in both operands (lane half hf
// holds dims [hf*64, hf*64+64), 8 per MFMA step); the dot product is
// independent of the order of its terms.  K reaches the MFMA operands
// through LDS: each wave streams its 32-key blocks into slices of its own by
// direct non-temporal loads of whole rows (K is read once per pass, so it
// need not displace anything cached), one block ahead of the one it uses.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWinThreads = 256;

struct WinView {
  int n, s0, s1;
};
__device__ __forceinline__ WinView win_view(const WinArgs &a, int b) {
  WinView v;
  v.n = clampi(a.seq_len[b], 0, a.max_blocks * kBlk);
  v.s0 = clampi(a.seg_begin[b], 0, v.n);
  v.s1 = clampi(a.seg_end[b], v.s0, v.n);
  return v;
}

// lane's query operand: row qr = lane % 32, dims [hf*64, hf*64+64)
__device__ __forceinline__ void load_q(const WinArgs &a, int b, int g, int lane, bf16x8 (&qop)[8]) {
  const int qr = a.qr0 + (lane & 31), hf = lane >> 5;   // this pass's block of 32 query rows
  const int R = a.n_rows * a.group;
  if (qr < R) {
    const int r = qr / a.group, h = qr % a.group;
    const uint4 *p = reinterpret_cast<const uint4 *>(a.q + (((size_t)b * a.n_rows + r) * a.hq + g * a.group + h) * kD + hf * 64);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, p[kk]);
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qop[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
}

// The block ids of one tile's keys, staged in LDS once (invalid -> -1).
constexpr int kWinMaxTileBlocks = 2048 / kBlk;

__device__ __forceinline__ void stage_tile_blocks(const WinArgs &a, int b, int kb0, int kend, int *s_blk) {
  const int nblk = (kend - kb0 + kBlk - 1) / kBlk;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) {
    const int blk = a.block_table[(size_t)b * a.max_blocks + kb0 / kBlk + i];
    s_blk[i] = (blk >= 0 && (int64_t)blk < a.num_blocks) ? blk : -1;
  }
}

// ---- K through LDS by direct, non-temporal loads ----
// Each wave streams its own 32-key blocks through two 8 KiB LDS slices of its
// own (static arrays, one per slice parity: the compiler then knows a load
// into one slice leaves the other alone and waits only for the loads of the
// slice it reads).  A K row is read once, by whole 256-byte rows per load
// instruction, so it can bypass the caches.

typedef __attribute__((address_space(1))) void gmem_t;
typedef __attribute__((address_space(3))) void lmem_t;
constexpr int kWinWaves = kWinThreads / 64;
constexpr int kSliceBytes = 32 * 256;   // one wave's 32-key block of K
constexpr int kNonTemporal = 2;         // cache-policy bits of the direct loads: nt

// The K rows of keys [kb, kb + 32) -- two whole cache blocks, kb a multiple of
// 16 -- into this wave's slice: load u of half h fills keys kb + 16h + 4u ..
// +3 (64 lanes x 16 bytes, lane L's at byte 16L of that stretch), lane L
// taking chunk (L%16) ^ (key%16) of key kb + 16h + 4u + L/16, so that the
// slice holds chunk c of key r at byte 256r + 16 (c ^ r%16).  Chunk (L%16) ^
// (4u + L/16) is c0 ^ 4u, c0 = (L%16) ^ (L/16): lane L's byte offset in the
// block's 4 KiB run is 1024u + (lo ^ 64u), lo = 256 (L/16) + 16 c0.  A block
// that is invalid, or starts at or past t1, reads the pool's first block of
// this kv head instead (its keys are masked by the caller), so every call
// issues the same eight loads.
__device__ __forceinline__ void dma_block(const WinArgs &a, int g, const int *s_blk, int kb0, int kb, int t1,
                                          uint8_t *slice, uint32_t lo) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key0 = kb + 16 * h;
    const int bi = min(max((key0 - kb0) >> 4, 0), kWinMaxTileBlocks - 1);
    const int sb = s_blk[bi];   // read unbranched (a read under a branch is waited for at once)
    const int blk = __builtin_amdgcn_readfirstlane(key0 < t1 ? sb : -1);
    KVSEL_CHECK((int64_t)blk < a.num_blocks, kDbgKvRow, blk);
    const uint8_t *run = reinterpret_cast<const uint8_t *>(a.k_pool) +
                         ((size_t)((uint32_t)max(blk, 0) * (uint32_t)a.hkv + (uint32_t)g) << 12);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_global_load_lds((gmem_t *)(run + 1024 * u + (lo ^ (64u * u))),
                                       (lmem_t *)(slice + (16 * h + 4 * u) * 256), 16, 0, kNonTemporal);
  }
}

// lane's key operand from a slice: key kl = lane % 32, dims [hf*64, hf*64+64)
// (chunk hf*8 + kk at 16 * ((hf*8 + kk) ^ kl%16) in row kl: rb ^ 16kk)
__device__ __forceinline__ void slice_k(const uint8_t *slice, uint32_t rb, bf16x8 (&kop)[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kop[kk] = *reinterpret_cast<const bf16x8 *>(slice + (rb ^ (16u * kk)));
}

// The queries are in registers before the first direct load: the compiler
// counts direct loads and ordinary loads as completing out of order, so an
// ordinary load still in flight would turn every wait in the loop into a wait
// for all loads.
__device__ __forceinline__ void have_q(const bf16x8 (&qop)[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(qop[kk]));
}

// Walk a wave's 32-key blocks k0 = first, first + 128, ... < end through its
// two slices: the next block's loads are in flight while one block is used
// (past the end they read the dummy block).
template <typename DmaF, typename UseF>
__device__ __forceinline__ void walk_slices(int first, int end, uint8_t *sl0, uint8_t *sl1, DmaF dma, UseF use) {
  dma(first, sl0);
  for (int k0 = first; k0 < end; k0 += 256) {
    dma(k0 + 128, sl1);
    use(k0, sl0);
    if (k0 + 128 >= end) break;
    dma(k0 + 256, sl0);
    use(k0 + 128, sl1);
  }
}

__global__ __launch_bounds__(kWinThreads) void window_stats_kernel(WinArgs a) {
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const WinView v = win_view(a, b);
  const int t0 = tile * a.tile_rows;
  if (t0 >= v.n) return;   // tiles past the last are never read (the merge stops at ceil(n / tile))
  const int t1 = min(t0 + a.tile_rows, v.n);
  __shared__ float s_m[8][32];
  __shared__ double s_z[8][32];

  __shared__ int s_blk[kWinMaxTileBlocks + 1];
  __shared__ __attribute__((aligned(16))) uint8_t s_sl0[kWinWaves][kSliceBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_sl1[kWinWaves][kSliceBytes];
  stage_tile_blocks(a, b, t0, t1, s_blk);
  bf16x8 qop[8];
  load_q(a, b, g, lane, qop);
  const int qr = lane & 31, hf = lane >> 5;   // this lane's query row in the block
  const int qg = a.qr0 + qr;                   // and among all of them
  // keys [t0, kend) are visible to this lane's query row
  int kend = t0;
  if (qg < a.n_rows * a.group) kend = a.causal ? min(t1, v.n - a.n_rows + qg / a.group + 1) : t1;
  const float cf = (float)(a.scale * 1.4426950408889634);
  float mc = -INFINITY;   // reference: the largest dot * cf so far (fp32)
  double z = 0.0;         // sum of 2^(dot * cf - mc), per element in fp32
  __syncthreads();
  const uint32_t lo = (uint32_t)(lane >> 4) * 256u + (uint32_t)(((lane & 15) ^ (lane >> 4)) << 4);
  const uint32_t rb = (uint32_t)qr * 256u + (uint32_t)(((hf * 8) ^ (qr & 15)) << 4);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto dma = [&](int kb, uint8_t *sl) { dma_block(a, g, s_blk, t0, kb, t1, sl, lo); };
  auto use = [&](int kb, const uint8_t *sl) {
    bf16x8 kop[8];
    slice_k(sl, rb, kop);
    f32x16 d = {};   // A rows: keys kb .. kb+31
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[kk], d, 0, 0, 0);
    // d[j]: key kb + 8*(j/4) + 4*hf + j%4 (j < 8: the block of kb, else the
    // next one), query row qr.  Keys this row does not see, or in an invalid
    // block, -> -inf.
    const int bi = (kb - t0) >> 4;
    const bool ok0 = s_blk[bi] >= 0, ok1 = kb + 16 >= t1 || s_blk[bi + 1] >= 0;
    if (kb + 32 > kend || !ok0 || !ok1) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kb + 8 * (j >> 2) + 4 * hf + (j & 3) >= kend || !(j < 8 ? ok0 : ok1)) d[j] = -INFINITY;
    }
    float bm = d[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) bm = fmaxf(bm, d[j]);
    const float bmc = bm * cf;
    if (bmc > mc) {
      if (mc != -INFINITY) z *= exp2_acc((double)mc - (double)bmc);
      mc = bmc;
    }
    if (mc != -INFINITY) {
      float zs = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) zs += fast_exp2(fmaf(d[j], cf, -mc));
      z += (double)zs;
    }
  };
  have_q(qop);
  walk_slices(t0 + wave * 32, t1, s_sl0[wv], s_sl1[wv], dma, use);
  s_m[wave * 2 + hf][qr] = mc;
  s_z[wave * 2 + hf][qr] = z;
  __syncthreads();
  if (tid < 32) {
    float M = -INFINITY;
    for (int i = 0; i < 8; ++i) M = fmaxf(M, s_m[i][tid]);
    double Z = 0.0;
    if (M != -INFINITY)
      for (int i = 0; i < 8; ++i)
        if (s_m[i][tid] != -INFINITY) Z += s_z[i][tid] * exp2_acc((double)s_m[i][tid] - (double)M);
    float *st = a.stat + ((((size_t)b * a.hkv + g) * a.ntiles + tile) * 32 + tid) * 4;
    st[0] = M;
    *reinterpret_cast<double *>(st + 2) = Z;
  }
}

// per query row: merge the key tiles' (reference, sum) into (reference, 1 / sum);
// grid (kv heads, sequences), 1024 threads = 32 query rows x 32 tile strides
__global__ __launch_bounds__(1024) void window_merge_kernel(WinArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int qr = tid & 31, part = tid >> 5;
  __shared__ float s_m[32][32];
  __shared__ double s_z[32][32];
  const WinView v = win_view(a, b);
  const int nt = min((v.n + a.tile_rows - 1) / a.tile_rows, a.ntiles);
  const float *st0 = a.stat + (((size_t)b * a.hkv + g) * a.ntiles * 32 + qr) * 4;
  float m = -INFINITY;
  for (int t = part; t < nt; t += 32) m = fmaxf(m, st0[(size_t)t * 32 * 4]);
  s_m[part][qr] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int p = 0; p < 32; ++p) M = fmaxf(M, s_m[p][qr]);
  double z = 0.0;
  if (M != -INFINITY)
    for (int t = part; t < nt; t += 32) {
      const float mt = st0[(size_t)t * 32 * 4];
      if (mt != -INFINITY)
        z += *reinterpret_cast<const double *>(st0 + (size_t)t * 32 * 4 + 2) * exp2_acc((double)mt - (double)M);
    }
  s_z[part][qr] = z;
  __syncthreads();
  if (part == 0) {
    double Z = 0.0;
    for (int p = 0; p < 32; ++p) Z += s_z[p][qr];
    double *rs = a.rowstat + (((size_t)b * a.hkv + g) * 32 + qr) * 2;
    // a row that sees no key: a reference no dot reaches and 1 / sum = 0
    rs[0] = M != -INFINITY && Z > 0.0 ? (double)M : 3.0e38;
    rs[1] = M != -INFINITY && Z > 0.0 ? 1.0 / Z : 0.0;
  }
}

__global__ __launch_bounds__(kWinThreads) void window_scores_kernel(WinArgs a) {
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const WinView v = win_view(a, b);
  const int t0 = max(tile * a.tile_rows, v.s0);
  const int t1 = min(tile * a.tile_rows + a.tile_rows, v.s1);
  if (t0 >= t1) return;
  __shared__ float s_M[32], s_iZ[32];
  if (tid < 32) {
    const double *rs = a.rowstat + (((size_t)b * a.hkv + g) * 32 + tid) * 2;
    s_M[tid] = (float)rs[0];
    s_iZ[tid] = (float)rs[1];
  }
  __syncthreads();

  const int tb0 = tile * a.tile_rows;   // block-aligned base of the tile's block ids
  __shared__ int s_blk[kWinMaxTileBlocks + 1];
  __shared__ __attribute__((aligned(16))) uint8_t s_sl0[kWinWaves][kSliceBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_sl1[kWinWaves][kSliceBytes];
  stage_tile_blocks(a, b, tb0, t1, s_blk);
  bf16x8 qop[8];
  load_q(a, b, g, lane, qop);
  const int kl = lane & 31, hf = lane >> 5;
  const float cf = (float)(a.scale * 1.4426950408889634);
  // this lane's 16 query rows: qr(j) = 8*(j/4) + 4*hf + j%4
  float rmc[16], riz[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    rmc[j] = s_M[8 * (j >> 2) + 4 * hf + (j & 3)];
    riz[j] = s_iZ[8 * (j >> 2) + 4 * hf + (j & 3)];
  }
  // keys <= all_vis are visible to every query row (rows past n_rows * group
  // have 1 / sum = 0)
  const int all_vis = a.causal ? v.n - a.n_rows : v.n - 1;
  const int R = a.n_rows * a.group;
  double *dst = a.part + ((size_t)b * a.hkv + g) * a.ld64;
  __syncthreads();
  const uint32_t lo = (uint32_t)(lane >> 4) * 256u + (uint32_t)(((lane & 15) ^ (lane >> 4)) << 4);
  const uint32_t rb = (uint32_t)kl * 256u + (uint32_t)(((hf * 8) ^ (kl & 15)) << 4);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto dma = [&](int kb, uint8_t *sl) { dma_block(a, g, s_blk, tb0, kb, t1, sl, lo); };
  // A block's scores leave one block later, after the next block's loads went
  // out: the wait at a block's start then covers that store too without
  // holding the block up.  Keys of the segment only; invalid blocks score 0.
  int pkey = -1;       // this lane's key of the previous block (-1: none)
  double pval = 0.0;
  auto flush = [&] {
    if (hf == 0 && pkey >= t0 && pkey < t1 && pkey - v.s0 < a.ld64)
      dst[pkey - v.s0] = a.accumulate ? dst[pkey - v.s0] + pval : pval;
  };
  auto use = [&](int kb, const uint8_t *sl) {
    bf16x8 kop[8];
    slice_k(sl, rb, kop);
    // the previous block's store, after this block's operands are read
    asm volatile("" ::"v"(kop[7]) : "memory");
    flush();
    f32x16 d = {};   // B columns: keys kb .. kb+31
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[kk], kop[kk], d, 0, 0, 0);
    // d[j]: query row qr(j), key kb + kl
    const int key = kb + kl;
    double acc = 0.0;
    if (kb + 31 <= all_vis) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc += (double)(fast_exp2(fmaf(d[j], cf, -rmc[j])) * riz[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qr = a.qr0 + 8 * (j >> 2) + 4 * hf + (j & 3);
        const bool vis = qr < R && key < v.n && (!a.causal || key <= v.n - a.n_rows + qr / a.group);
        if (vis) acc += (double)(fast_exp2(fmaf(d[j], cf, -rmc[j])) * riz[j]);
      }
    }
    acc += __shfl_xor(acc, 32);
    const int bi = min(max((key - tb0) >> 4, 0), kWinMaxTileBlocks - 1);
    pval = s_blk[bi] >= 0 ? acc : 0.0;
    pkey = key;
  };
  // blocks aligned to the tile's block-aligned base (each load covers whole
  // cache blocks); keys before t0 (before the segment) are not stored
  have_q(qop);
  walk_slices(tb0 + wave * 32, t1, s_sl0[wv], s_sl1[wv], dma, use);
  flush();
}

}  // namespace

// Work-groups aimed at per pass.  Measured at C2 (one 32768-token prompt,
// 8 kv heads): 128 -> 10.4k, 256 -> 11.8k, 512 -> 10.5k, 1024 -> 10.2k
// selections/s; each work-group's fixed costs (block ids, queries, the fp64
// merge of its waves' statistics) are spread over more keys, one per CU.
#ifndef KVSEL_WIN_WGS
#define KVSEL_WIN_WGS 256
#endif

WinPlan win_plan(int batch, int hkv, int group, int n_rows, int max_seq_len, int max_seg_len) {
  WinPlan p;
  const int64_t pairs = (int64_t)batch * hkv;
  // about one work-group per CU (KVSEL_WIN_WGS), at least 128 keys each
  int64_t t = ((int64_t)max_seq_len * pairs + KVSEL_WIN_WGS - 1) / KVSEL_WIN_WGS;
  t = (t + 127) / 128 * 128;
  if (t < 128) t = 128;
  if (t > kWinMaxTileBlocks * kBlk) t = kWinMaxTileBlocks * kBlk;
  p.tile_rows = (int)t;
  p.ntiles = (int)((max_seq_len + t - 1) / t);
  if (p.ntiles < 1) p.ntiles = 1;
  p.rows_q = n_rows * group;
  p.ld64 = max_seg_len > 0 ? max_seg_len : 1;
  size_t off = kCounterBytes;
  p.off_stat = off;
  off = align_up(off + (size_t)pairs * p.ntiles * 32 * 4 * sizeof(float));
  p.off_rowstat = off;
  off = align_up(off + (size_t)pairs * 32 * 2 * sizeof(double));
  p.off_part = off;
  off = align_up(off + (size_t)pairs * p.ld64 * sizeof(double));
  p.total = off;
  return p;
}

// The query rows of a kv head (window rows x group heads) in blocks of 32, one
// MFMA tile each: every block has its own statistics (its rows' normalisers)
// and adds its probabilities to the same fp64 partial scores.
hipError_t launch_window(const WinArgs &a0, const WinPlan &p, int batch, hipStream_t s) {
  dim3 grid(p.ntiles, a0.hkv, batch), block(kWinThreads);
  const int R = a0.n_rows * a0.group;
  for (int qr0 = 0; qr0 < (R > 0 ? R : 1); qr0 += 32) {
    WinArgs a = a0;
    a.qr0 = qr0;
    a.accumulate = qr0 > 0 ? 1 : 0;
    hipLaunchKernelGGL(window_stats_kernel, grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(window_merge_kernel, dim3(a.hkv, batch), dim3(1024), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(window_scores_kernel, grid, block, 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvsel
