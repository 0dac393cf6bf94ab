// FastKV window saliency on MFMA (FastKV section 2A, Token-Selective
// Propagation: the attention weights from a recent window of queries to all
// context tokens, averaged, rank the tokens).
//
// For one (sequence, kv head) the window rows x group heads form R <= 32
// query rows (row index qr = r * G + h; window row r is the query of
// position n - W + r and, when causal, sees keys <= that position).  The
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
// holds dims [hf*64, hf*64+64), 8 per MFMA step), so each lane reads one
// whole 128-byte half of a key row; the dot product is independent of the
// order of its terms.
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
  const int qr = lane & 31, hf = lane >> 5;
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

// lane's key operand for key row `key` of the tile whose block ids start at
// kb0.  Keys past kend or in an invalid block read `dummy` (any 256 valid
// bytes) instead; the caller masks them.  No branch: every call issues the
// same eight loads, so the compiler's wait counts stay exact.
__device__ __forceinline__ bool load_k(const WinArgs &a, int g, const int *s_blk, int kb0, int key, int kend,
                                       const uint16_t *dummy, int lane, bf16x8 (&kop)[8]) {
  const int hf = lane >> 5;
  const int bi = min(max((key - kb0) >> 4, 0), kWinMaxTileBlocks - 1);
  const int blk = key < kend ? s_blk[bi] : -1;
  const uint16_t *row = blk >= 0
      ? a.k_pool + ((size_t)((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * kBlk + (key & 15)) * kD
      : dummy;
  const uint4 *p = reinterpret_cast<const uint4 *>(row + hf * 64);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kop[kk] = __builtin_bit_cast(bf16x8, p[kk]);
  return blk >= 0;
}

// Walk a wave's 32-key blocks k0 = first, first + 128, ... < end with two
// operand buffers: the next block's loads are in flight while one block is
// used (loads past the end read the dummy row), and no register copy forces
// an early wait.
template <typename LoadF, typename UseF>
__device__ __forceinline__ void walk_blocks(int first, int end, LoadF load, UseF use) {
  bf16x8 ka[8], kb[8];
  load(first, ka);
  for (int k0 = first; k0 < end; k0 += 256) {
    load(k0 + 128, kb);
    use(k0, ka);
    if (k0 + 128 >= end) break;
    load(k0 + 256, ka);
    use(k0 + 128, kb);
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
  stage_tile_blocks(a, b, t0, t1, s_blk);
  bf16x8 qop[8];
  load_q(a, b, g, lane, qop);
  const int qr = lane & 31, hf = lane >> 5;
  // keys [t0, kend) are visible to this lane's query row
  int kend = t0;
  if (qr < a.n_rows * a.group) kend = a.causal ? min(t1, v.n - a.n_rows + qr / a.group + 1) : t1;
  const float cf = (float)(a.scale * 1.4426950408889634);
  float mc = -INFINITY;   // reference: the largest dot * cf so far (fp32)
  double z = 0.0;         // sum of 2^(dot * cf - mc), per element in fp32
  __syncthreads();
  const uint16_t *dummy = a.q;
  auto load = [&](int kb, bf16x8 (&kop)[8]) { load_k(a, g, s_blk, t0, kb + qr, t1, dummy, lane, kop); };
  auto use = [&](int kb, const bf16x8 (&kop)[8]) {
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
  walk_blocks(t0 + wave * 32, t1, load, use);
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
  __shared__ double s_out[kWinMaxTileBlocks * kBlk];
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
  const uint16_t *dummy = a.q;
  auto load = [&](int kb, bf16x8 (&kop)[8]) { load_k(a, g, s_blk, tb0, kb + kl, t1, dummy, lane, kop); };
  auto use = [&](int kb, const bf16x8 (&kop)[8]) {
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
        const int qr = 8 * (j >> 2) + 4 * hf + (j & 3);
        const bool vis = qr < R && key < v.n && (!a.causal || key <= v.n - a.n_rows + qr / a.group);
        if (vis) acc += (double)(fast_exp2(fmaf(d[j], cf, -rmc[j])) * riz[j]);
      }
    }
    acc += __shfl_xor(acc, 32);
    // keys in an invalid block score 0; the tile's scores leave through LDS
    if (hf == 0 && key < t1) s_out[key - tb0] = s_blk[(key - tb0) >> 4] >= 0 ? acc : 0.0;
  };
  // blocks aligned to the tile start so that each wave's keys are contiguous
  walk_blocks(t0 + wave * 32, t1, load, use);
  __syncthreads();
  for (int key = t0 + tid; key < t1; key += kWinThreads)
    if (key - v.s0 < a.ld64) dst[key - v.s0] = s_out[key - tb0];
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

hipError_t launch_window(const WinArgs &a, const WinPlan &p, int batch, hipStream_t s) {
  dim3 grid(p.ntiles, a.hkv, batch), block(kWinThreads);
  hipLaunchKernelGGL(window_stats_kernel, grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(window_merge_kernel, dim3(a.hkv, batch), dim3(1024), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(window_scores_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kvsel
