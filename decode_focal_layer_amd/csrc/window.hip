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
//     query row and 16 keys of every 32-key block: the per-row running max and
//     sum of 2^((dot - max) * scale * log2 e) stay lane-local (sum in fp64).
//     Each tile writes (max, sum) per query row.
//   merge: one small kernel combines the tiles' statistics per query row in
//     fp64 into (max, 1 / sum);
//   pass 2 (scores): MFMA with the query rows as A and the keys as B, so each lane holds one
//     key and 16 query rows: the normalised probabilities are summed over the
//     rows lane-locally in fp64, then across the two half-waves.
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

__device__ __forceinline__ uint32_t win_phys(const WinArgs &a, int b, int g, int row) {
  const int blk = a.block_table[(size_t)b * a.max_blocks + (row >> 4)];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return kNoRow;
  return ((uint32_t)blk * (uint32_t)a.hkv + (uint32_t)g) * (uint32_t)kBlk + (uint32_t)(row & 15);
}

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

// lane's key operand for key row `key` (invalid -> zeros)
__device__ __forceinline__ void load_k(const WinArgs &a, int b, int g, int key, int n, int lane, bf16x8 (&kop)[8]) {
  const int hf = lane >> 5;
  const uint32_t pr = key < n ? win_phys(a, b, g, key) : kNoRow;
  if (pr != kNoRow) {
    const uint4 *p = reinterpret_cast<const uint4 *>(a.k_pool + (size_t)pr * kD + hf * 64);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = __builtin_bit_cast(bf16x8, p[kk]);
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
}

// key visible to query row qr
__device__ __forceinline__ bool visible(const WinArgs &a, int n, int key, int qr) {
  if (key >= n || qr >= a.n_rows * a.group) return false;
  if (!a.causal) return true;
  const int r = qr / a.group;
  return key <= n - a.n_rows + r;
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

  bf16x8 qop[8];
  load_q(a, b, g, lane, qop);
  const int qr = lane & 31, hf = lane >> 5;
  const double c = a.scale * 1.4426950408889634;
  float m = -INFINITY;
  double z = 0.0;
  bf16x8 knext[8];
  if (t0 + wave * 32 < t1) load_k(a, b, g, t0 + wave * 32 + qr, t1, lane, knext);
  for (int kb = t0 + wave * 32; kb < t1; kb += 128) {
    bf16x8 kop[8];   // A rows: keys kb .. kb+31; the next block's rows are loaded meanwhile
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = knext[kk];
    if (kb + 128 < t1) load_k(a, b, g, kb + 128 + qr, t1, lane, knext);
    f32x16 d = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[kk], d, 0, 0, 0);
    // d[j]: key kb + 8*(j/4) + 4*hf + j%4, query row qr
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kb + 8 * (j >> 2) + 4 * hf + (j & 3);
      if (key < t1 && visible(a, v.n, key, qr)) bm = fmaxf(bm, d[j]);
    }
    if (bm > m) {
      if (m != -INFINITY) z *= exp2_acc(((double)m - (double)bm) * c);
      m = bm;
    }
    if (m != -INFINITY) {
      double zs = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kb + 8 * (j >> 2) + 4 * hf + (j & 3);
        if (key < t1 && visible(a, v.n, key, qr)) zs += exp2_acc(((double)d[j] - (double)m) * c);
      }
      z += zs;
    }
  }
  s_m[wave * 2 + hf][qr] = m;
  s_z[wave * 2 + hf][qr] = z;
  __syncthreads();
  if (tid < 32) {
    float M = -INFINITY;
    for (int i = 0; i < 8; ++i) M = fmaxf(M, s_m[i][tid]);
    double Z = 0.0;
    if (M != -INFINITY)
      for (int i = 0; i < 8; ++i)
        if (s_m[i][tid] != -INFINITY) Z += s_z[i][tid] * exp2_acc(((double)s_m[i][tid] - (double)M) * c);
    float *st = a.stat + ((((size_t)b * a.hkv + g) * a.ntiles + tile) * 32 + tid) * 4;
    st[0] = M;
    *reinterpret_cast<double *>(st + 2) = Z;
  }
}

// per query row: merge the key tiles' (max, sum) into (max, 1 / sum);
// grid (kv heads, sequences), 1024 threads = 32 query rows x 32 tile strides
__global__ __launch_bounds__(1024) void window_merge_kernel(WinArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int qr = tid & 31, part = tid >> 5;
  __shared__ float s_m[32][32];
  __shared__ double s_z[32][32];
  const WinView v = win_view(a, b);
  const int nt = min((v.n + a.tile_rows - 1) / a.tile_rows, a.ntiles);
  const double c = a.scale * 1.4426950408889634;
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
        z += *reinterpret_cast<const double *>(st0 + (size_t)t * 32 * 4 + 2) * exp2_acc(((double)mt - (double)M) * c);
    }
  s_z[part][qr] = z;
  __syncthreads();
  if (part == 0) {
    double Z = 0.0;
    for (int p = 0; p < 32; ++p) Z += s_z[p][qr];
    double *rs = a.rowstat + (((size_t)b * a.hkv + g) * 32 + qr) * 2;
    rs[0] = (double)M;
    rs[1] = Z > 0.0 ? 1.0 / Z : 0.0;
  }
}

__global__ __launch_bounds__(kWinThreads) void window_scores_kernel(WinArgs a) {
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const WinView v = win_view(a, b);
  const int t0 = max(tile * a.tile_rows, v.s0);
  const int t1 = min(tile * a.tile_rows + a.tile_rows, v.s1);
  if (t0 >= t1) return;
  __shared__ double s_M[32], s_iZ[32];
  const double c = a.scale * 1.4426950408889634;
  if (tid < 32) {
    const double *rs = a.rowstat + (((size_t)b * a.hkv + g) * 32 + tid) * 2;
    s_M[tid] = rs[0];
    s_iZ[tid] = rs[1];
  }
  __syncthreads();

  bf16x8 qop[8];
  load_q(a, b, g, lane, qop);
  const int kl = lane & 31, hf = lane >> 5;
  double *dst = a.part + ((size_t)b * a.hkv + g) * a.ld64;
  // blocks aligned to the tile start so that each wave's keys are contiguous
  bf16x8 knext[8];
  if (t0 + wave * 32 < t1) load_k(a, b, g, t0 + wave * 32 + kl, t1, lane, knext);
  for (int kb = t0 + wave * 32; kb < t1; kb += 128) {
    bf16x8 kop[8];   // B columns: keys kb .. kb+31; the next block's rows are loaded meanwhile
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = knext[kk];
    if (kb + 128 < t1) load_k(a, b, g, kb + 128 + kl, t1, lane, knext);
    f32x16 d = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[kk], kop[kk], d, 0, 0, 0);
    // d[j]: query row 8*(j/4) + 4*hf + j%4, key kb + kl
    const int key = kb + kl;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qr = 8 * (j >> 2) + 4 * hf + (j & 3);
      if (visible(a, v.n, key, qr)) acc += exp2_acc(((double)d[j] - s_M[qr]) * c) * s_iZ[qr];
    }
    acc += __shfl_xor(acc, 32);
    if (hf == 0 && key < t1 && key - v.s0 < a.ld64) dst[key - v.s0] = acc;
  }
}

}  // namespace

WinPlan win_plan(int batch, int hkv, int group, int n_rows, int max_seq_len, int max_seg_len) {
  WinPlan p;
  const int64_t pairs = (int64_t)batch * hkv;
  // about two work-groups per CU (512), at least 128 keys each
  int64_t t = ((int64_t)max_seq_len * pairs + 511) / 512;
  t = (t + 127) / 128 * 128;
  if (t < 128) t = 128;
  if (t > 2048) t = 2048;
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
