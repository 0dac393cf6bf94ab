// Launchers of the MFMA attention kernels (draft verification, causal
// prefill over a compacted sequence); host side.
#pragma once

#include "kvsel_internal.h"

namespace kvsel {

// draft verification attention (MFMA): one work-group per (sequence, kv head)
constexpr int kVerifyMaxRows = 8192;   // attended rows per (sequence, kv head), resolved into LDS
struct VerifyArgs {
  const uint16_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *seg_begin, *seg_end;
  int64_t num_blocks;
  int32_t max_blocks, hkv, hq, group, m, k;
  const uint16_t *q;     // [batch][m][hq][128]
  const int32_t *idx;    // [batch][hkv][k]
  float scale_log2;
  float *out, *lse;      // [batch][m][hq][128], [batch][m][hq]
  int32_t rows_cap;      // attended rows per (sequence, kv head), at most kVerifyMaxRows
  int32_t col0;          // first query column (draft x group head) of this launch's block of 32
};
hipError_t launch_verify(const VerifyArgs &a, int batch, hipStream_t s);

// causal prefill over a compacted sequence (MFMA): one work-group per
// (128 query rows, kv head, sequence)
struct PrefillArgs {
  const uint16_t *q, *k, *v;     // [total][hq][128], [total][hkv][128] x2
  const int32_t *cu_seqlens;     // [batch + 1]
  float *out, *lse;              // [total][hq][128], [total][hq]
  int32_t max_seqlen, hq, hkv, group;
  float scale_log2;
  int32_t nblk, items;           // set by launch_prefill
};
hipError_t launch_prefill(const PrefillArgs &a, int batch, hipStream_t s);

// every sequence's queries over one row range that all sequences share,
// read through one block table (MFMA): one work-group per (128 query rows,
// kv head)
constexpr int kSharedMaxBlocks = 1024;   // cache blocks the range may touch (their ids go to LDS)
struct SharedArgs {
  const uint16_t *k_pool, *v_pool;
  const int32_t *table;          // the block table the rows are read through
  int64_t num_blocks;
  int32_t hkv, hq, group, batch;
  int32_t row_begin, row_end;
  int32_t splits, chunk;         // the range in `splits` parts of `chunk` rows (a multiple of 64)
  int32_t accumulate;            // splits = 1: out/lse hold another part on entry; the range is folded in
  const uint16_t *q;             // [batch][hq][128]
  float scale_log2;
  float *out, *lse;              // [splits][batch][hq][128], [splits][batch][hq]
  float *logits;                 // or null: raw dots [batch][hq][ld_logits] of each sequence's segment rows
  int64_t ld_logits;
  const int32_t *seg_begin, *seg_end;
  int32_t nblk, items;           // set by launch_shared
};
hipError_t launch_shared(const SharedArgs &a, hipStream_t s);

// out = attention over the union of `parts` disjoint row sets from the parts
constexpr int kMaxMergeParts = 64;
hipError_t launch_merge(const float *o, const float *lse, int parts, int64_t rows, float *out, float *lse_out,
                        hipStream_t s);

}  // namespace kvsel
