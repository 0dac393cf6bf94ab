// Internal launch plans and launcher entry points of libkvsel (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvsel.h"

namespace kvsel {

constexpr size_t kAlign = 256;
// Every workspace starts with this many bytes of split counters, one per
// (sequence, kv head) pair, used by the attention kernels to find the last
// work-group of a pair and always left at zero when they finish: pairs per
// call are limited to kCounterBytes / 4.
constexpr size_t kCounterBytes = 65536;
constexpr int kMaxPairs = (int)(kCounterBytes / 4);
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// split-KV decode attention
// ---------------------------------------------------------------------------
constexpr int kAttnThreads = 256;
constexpr int kAttnRowsPerIter = 64;   // 16 lane groups x 4 rows
constexpr int kAttnMaxRps = 8192;   // rows resolved into LDS per work-group (32 KiB)
constexpr int kRec = 160;              // floats per partial record: acc[128], m, l, pad (640 B)

struct AttnPlan {
  int rps = 0;          // virtual rows per split (multiple of 64)
  int nsplit = 0;       // splits per (sequence, kv head)
  int ld_logits = 0;    // row stride of the logit scratch (0: none)
  size_t off_counters = 0, off_rec = 0, off_logits = 0, off_extra = 0, total = 0;
};

// mode: 0 = no logits, 1 = segment rows, 2 = every row
AttnPlan attn_plan(int batch, int hkv, int hq, int max_rows, int logit_mode, int max_seg_len,
                   int max_seq_len);

struct AttnArgs {
  const uint16_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *seg_begin, *seg_end;
  int64_t num_blocks;
  int32_t max_blocks, hkv, hq, k;
  int32_t shared_rows;  // > 0: rows are shared across sequences, load them through the caches
  int32_t det;          // 1: each wave takes a fixed share of the rows (bitwise reproducible)
  const uint16_t *q;
  const int32_t *idx;   // [batch][hkv][k] kept indices (gather)
  int32_t dense;        // 1: every row [0, seq_len); 0: gather
  float scale_log2;     // softmax scale * log2(e)
  int32_t rps, nsplit;
  uint32_t *counters;   // per-pair arrival counters at the start of the workspace (zero between calls)
  float *rec;           // [batch][hq][nsplit][kRec]
  float *out, *lse;
  float *mass;          // non-null: the segment's attention share per head instead of out
  float *logits;        // [batch][hq][ld_logits] raw q.k dots, or null
  int64_t ld_logits;
  int32_t logit_mode;
  // fused focal selection (one work-group per (sequence, kv head)): the
  // segment logits stay in LDS (seg_cap per head) and the work-group
  // normalises them and selects sel_k indices itself
  int32_t *sel_idx;     // [batch][hkv][sel_k], or null (no fused selection)
  const int32_t *sel_warm;
  int32_t sel_k;
  float *sel_scores;    // [batch][hkv][sel_ld] or null
  int64_t sel_ld;
  int32_t seg_cap;
  double scale;
};

// dynamic LDS the fused focal kernel may take for the segment logits
constexpr size_t kFusedLdsBytes = 80 * 1024;
inline bool fused_focal_fits(int group, int max_seg_len) {
  const size_t cap = (size_t)((max_seg_len + 3) / 4 * 4);
  // the selection runs on eight waves: work-groups of 512 or more threads (G <= 4)
  return group <= 4 && cap > 0 && (size_t)group * cap * sizeof(float) <= kFusedLdsBytes;
}

hipError_t launch_attn(const AttnArgs &a, int batch, int group, hipStream_t s);

// Allows kernel `fn` up to `bytes` of dynamic LDS on the current device: set
// once per (device, kernel, size), thread-safe (launch_util.hip).
hipError_t allow_dynamic_lds(const void *fn, int bytes);

// focal-layer choice: one work-group
constexpr int kMaxLayers = 1024;
hipError_t launch_pick_layers(const float *ratios, int64_t ld, int n_layers, int n, int n_pick, int32_t *layers,
                              hipStream_t s);

// logits only (no V): rows [lo, hi) per mode into the logit scratch
hipError_t launch_logits(const AttnArgs &a, int batch, int group, int max_rows, hipStream_t s);

// ---------------------------------------------------------------------------
// focal score normalisation (logits -> head-summed probabilities), alone or
// fused with the top-k of each (sequence, kv head)
// ---------------------------------------------------------------------------
constexpr int kSelMaxSeg = 12288;   // fused selection: candidate segment held in LDS

struct SelArgs {
  const float *logits;   // [batch][hq][ld_logits] raw q.k dots
  int64_t ld_logits;
  const int32_t *seq_len, *seg_begin, *seg_end;
  int32_t cap_rows;      // max_blocks * block (clamp for seq_len)
  int32_t hq, heads_per_out, n_out;   // output rows per sequence = n_out
  int32_t norm;          // KVSEL_NORM_*
  double scale;
  float *scores;         // fp32 [batch][n_out][ld], or null
  int64_t ld;
  double *scores64;      // fp64 [batch][n_out][ld64] (norm kernel, when scores is null)
  int64_t ld64;
  int32_t k;             // fused selection: budget, warm start, output
  const int32_t *warm;
  int32_t *idx;          // [batch][n_out][k]
};
hipError_t launch_focal_norm(const SelArgs &a, int batch, hipStream_t s);
hipError_t launch_focal_select(const SelArgs &a, int batch, hipStream_t s);

// ---------------------------------------------------------------------------
// group sum + average pool over fp64 partial scores
// ---------------------------------------------------------------------------
struct PoolArgs {
  const double *part;    // [batch][n_in][ld64]
  int64_t ld64;
  int32_t n_in, n_out;   // n_in partial rows fold into n_out output rows
  const int32_t *seq_len, *seg_begin, *seg_end;
  int32_t cap_rows;
  int32_t width;         // odd
  float *scores;         // [batch][n_out][ld]
  int64_t ld;
};
hipError_t launch_pool(const PoolArgs &a, int batch, int max_seg_len, hipStream_t s);

// ---------------------------------------------------------------------------
// FastKV window scoring on MFMA
// ---------------------------------------------------------------------------
struct WinArgs {
  const uint16_t *k_pool;
  const int32_t *block_table, *seq_len, *seg_begin, *seg_end;
  int64_t num_blocks;
  int32_t max_blocks, hkv, hq, group, n_rows, causal;
  const uint16_t *q;     // [batch][n_rows][hq][128]
  float scale_log2;
  double scale;
  int32_t tile_rows, ntiles;   // keys per work-group tile, tiles per sequence
  int32_t qr0;           // first query row (window row x group head) of this pass's block of 32
  int32_t accumulate;    // 1: add this block's scores to the partial row (a later block)
  float *stat;           // [batch][hkv][ntiles][32] x {max dot (f32), pad, sum (f64)}
  double *rowstat;       // [batch][hkv][32] x {max dot, 1 / sum}, merged over tiles
  double *part;          // [batch][hkv][ld64] fp64 group scores
  int64_t ld64;
};
struct WinPlan {
  int tile_rows = 0, ntiles = 0, rows_q = 0;
  size_t off_stat = 0, off_rowstat = 0, off_part = 0, total = 0;
  int64_t ld64 = 0;
};
WinPlan win_plan(int batch, int hkv, int group, int n_rows, int max_seq_len, int max_seg_len);
hipError_t launch_window(const WinArgs &a, const WinPlan &p, int batch, hipStream_t s);

// ---------------------------------------------------------------------------
// exact top-k
// ---------------------------------------------------------------------------
struct TopkArgs {
  const float *scores;
  int64_t ld;
  int32_t rows, n, k;
  const int32_t *warm;
  int32_t *idx;
  const int32_t *n_row;   // or null: row r ranks its first min(n_row[r], n) scores
};
// workspace of kvsel_topk: coarse-bin counts of the long-row path (0: none)
size_t topk_workspace_bytes(int rows, int n);
hipError_t launch_topk(const TopkArgs &a, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// row gather
// ---------------------------------------------------------------------------
hipError_t launch_gather_rows(const void *src, int64_t row_bytes, int64_t n_src_rows,
                              const int32_t *idx, int32_t n_idx, int64_t tail_begin,
                              int32_t n_tail, void *dst, hipStream_t s);

}  // namespace kvsel
