/*
 * kvsel.h -- libkvsel: attention-score-guided KV token selection followed by
 * sparse decode attention, for AMD Instinct MI355X (gfx950).
 *
 * The path this library runs, per decode step:
 *   1. a focal layer scores the query against the cached keys of a candidate
 *      segment (visual tokens in FastOCR; the long prompt in FastKV) and sums
 *      the softmax probabilities over the query heads that share a kv head;
 *   2. the k highest-scoring tokens are kept (ties to the lower index);
 *   3. the other layers attend only over the kept tokens plus every token
 *      outside the candidate segment (text, layout, recent or suffix rows);
 *      the full cache stays in memory and only the attended subset changes.
 *
 * Sources:
 *   FastOCR: Dynamic Visual Fixation via KV Cache Pruning -- technical
 *     summary, Methodology: Focal-Guided Pruning (focal-layer scoring over
 *     the full cache, top image tokens at kept ratio tau, propagation to
 *     non-focal layers) and Cross-Step Fixation Reuse (warm start from the
 *     previous step's set); Significance (the full cache is retained).
 *   FastKV: Decoupling of Context Reduction and KV Cache Compression --
 *     section 2A Token-Selective Propagation (saliency from a recent window
 *     of queries, averaged; top tokens plus the window tokens propagate)
 *     and section 2B Decoupled KV Retention (a per-layer decode budget).
 *   HPD-Parsing wiki -- method item 2, shared-prefix KV reuse and context
 *     isolation (branches read one prefix zero-copy; each attends to the
 *     shared context, its own prefix and its own history).
 *
 * Conventions (every entry point):
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains device memory; scratch comes from a
 *     caller workspace sized by the matching kvsel_*_workspace() call.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns.  Ordering is the stream's.
 *   - Argument errors are found on the host before any HIP call and return
 *     KVSEL_EINVAL / KVSEL_ENOSPC / KVSEL_EUNSUPPORTED with nothing enqueued;
 *     the text is in kvsel_last_error() (thread-local).  A failed launch
 *     returns KVSEL_EHIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation.
 *   - Device-resident integers (seq_len, segment bounds, block ids, kept
 *     indices) are clamped or skipped by the kernels when out of range, so a
 *     bad value gives a wrong result, never an out-of-bounds access.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Workspace: the byte count from kvsel_*_workspace(); the buffer must be
 *     256-byte aligned and ZERO-FILLED ONCE before its first use.  Its first
 *     64 KiB hold split counters that only the attention calls touch and
 *     that every call leaves at zero when its kernels finish, so a workspace
 *     can be reused by any later call on the same stream.  Two calls that may
 *     run at the same time need separate workspaces.
 *   - batch * num_kv_heads <= 16384 (KVSEL_EUNSUPPORTED otherwise).
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define KVSEL_API __attribute__((visibility("default")))
#else
#define KVSEL_API
#endif

typedef int32_t kvsel_status;
#define KVSEL_OK            0
#define KVSEL_EINVAL       (-1)  /* bad argument                                  */
#define KVSEL_ENOSPC       (-2)  /* workspace too small                           */
#define KVSEL_EUNSUPPORTED (-3)  /* head_dim != 128, block_size != 16, group > 8  */
#define KVSEL_EHIP         (-4)  /* a HIP launch failed                           */
#define KVSEL_EDEBUG       (-5)  /* debug build: a device-side check failed       */

#define KVSEL_VERSION 3

#define KVSEL_REDUCE_GROUP 0     /* one score per (sequence, kv head)            */
#define KVSEL_REDUCE_ALL   1     /* one score per (sequence): summed over heads  */

#define KVSEL_NORM_SEGMENT 0     /* softmax over the candidate segment only      */
#define KVSEL_NORM_CONTEXT 1     /* softmax over every row the query can see     */

/* kvsel_kv_desc.flags */
#define KVSEL_FLAG_DETERMINISTIC 1   /* attention sums its rows in a fixed order  */

typedef void *kvsel_stream;      /* hipStream_t */

/*
 * Paged KV cache descriptor (non-owning).
 *
 * K and V pools are bf16 [num_blocks][num_kv_heads][block_size][head_dim]:
 * one (block, kv head) is a contiguous block_size*head_dim*2 = 4 KiB run.
 * Logical row j of sequence b is row j % block_size of physical block
 * block_table[b * max_blocks_per_seq + j / block_size].  Rows [0, seq_len[b])
 * are present.  Sequences that share a prefix list the same physical block
 * ids (zero-copy; HPD wiki, method item 2).  A contiguous cache is the
 * identity table.
 *
 * Candidate segment: rows [seg_begin[b], seg_end[b]) are scored and
 * selectable; every row outside it is always attended by gather attention.
 *
 * shared_rows is a cache hint for a shared prefix: rows [0, shared_rows) of
 * every sequence are read by many sequences (their blocks appear in many
 * tables).  With shared_rows == 0 every K/V row is read by one sequence, and
 * the attention kernels stream rows with non-temporal loads so that they do
 * not evict what is reused from call to call (block tables, indices,
 * queries); with shared_rows > 0 they load every row through the caches so
 * that the prefix stays there.  Results do not depend on it.
 *
 * flags: 0 or KVSEL_FLAG_DETERMINISTIC.  By default the attention calls
 * (kvsel_gather_attn, kvsel_dense_attn, kvsel_focal_attn,
 * kvsel_visual_mass) hand rows to waves on demand, so which wave adds which
 * row, and with it the rounding of the output (not the row set, the scores
 * or the kept indices), can vary from run to run.  With
 * KVSEL_FLAG_DETERMINISTIC every wave takes a fixed share of the rows and the
 * focal selection runs as its own kernel after the attention, so every
 * output is bitwise reproducible, at some cost in speed.  Every other call is
 * bitwise reproducible either way.  Other bits: KVSEL_EINVAL.
 */
typedef struct {
  int32_t batch;               /* sequences (or branches)                        */
  int32_t num_kv_heads;        /* H_kv                                           */
  int32_t head_dim;            /* must be 128                                    */
  int32_t block_size;          /* must be 16                                     */
  int32_t max_blocks_per_seq;  /* row stride of block_table                      */
  int32_t max_seq_len;         /* host upper bound of seq_len[] (grid sizing);   */
                               /* <= max_blocks_per_seq * block_size             */
  int32_t max_seg_len;         /* host upper bound of seg_end[] - seg_begin[]     */
  int32_t min_seg_len;         /* host lower bound of seg_end[] - seg_begin[]     */
                               /* (0 if unknown); sizes the gather launch        */
  int64_t num_blocks;          /* physical blocks in each pool                   */
  const uint16_t *k_pool;      /* bf16, device                                   */
  const uint16_t *v_pool;      /* bf16, device (may be NULL for kvsel_score)     */
  const int32_t *block_table;  /* [batch][max_blocks_per_seq], device            */
  const int32_t *seq_len;      /* [batch], device                                */
  const int32_t *seg_begin;    /* [batch], device                                */
  const int32_t *seg_end;      /* [batch], device                                */
  int32_t shared_rows;         /* >= 0: leading rows shared across sequences      */
  int32_t flags;               /* KVSEL_FLAG_* (0: default)                      */
} kvsel_kv_desc;

/* Version of this header's ABI (KVSEL_VERSION). */
KVSEL_API int32_t kvsel_version(void);
/* Static text for a status code. */
KVSEL_API const char *kvsel_status_string(kvsel_status s);
/* Text of the last error on the calling thread ("" if none). */
KVSEL_API const char *kvsel_last_error(void);

/*
 * kvsel_debug_status -- the device-side checks of a debug build.
 *
 * A library built with KVSEL_DEBUG=1 (libkvsel_debug.so beside the release
 * build) checks inside its kernels the facts they rely on: every K/V row
 * read lies inside its pool, LDS indices inside their arrays, every output
 * slot inside its row (a top-k position below k), every split arrival
 * counter started at zero (a workspace shared by overlapping calls, or not
 * zeroed, breaks that), counts within their bounds.  A failed check does not
 * trap; it is counted in device memory, with the code (KVSEL_DBG_* below) and
 * a detail value of the first one.  This call reads and clears the counts;
 * synchronise the device first.  violations, first_code and first_detail may
 * each be NULL.  Returns KVSEL_OK if no check failed, KVSEL_EDEBUG if one
 * did, KVSEL_EHIP if the counts could not be read, and KVSEL_EUNSUPPORTED
 * (outputs 0) from a release build, whose kernels hold no checks.
 */
#define KVSEL_DBG_KV_ROW    1   /* detail: the physical row                       */
#define KVSEL_DBG_LDS       2   /* detail: the index                              */
#define KVSEL_DBG_OUT_SLOT  3   /* detail: the slot                               */
#define KVSEL_DBG_COUNTER   4   /* detail: the counter value found                */
#define KVSEL_DBG_SRC_ROW   5   /* detail: the row                                */
#define KVSEL_DBG_COUNT     6   /* detail: the count                              */
KVSEL_API kvsel_status kvsel_debug_status(uint32_t *violations, uint32_t *first_code, uint32_t *first_detail);

/*
 * kvsel_score -- token saliency over the candidate segment.
 * (FastOCR Focal-Guided Pruning: focal-layer attention over the full cache;
 *  FastKV 2A: attention weights from a recent window of queries, averaged.)
 *
 * q: bf16 [batch][n_rows][num_q_heads][128].  n_rows == 1 is a decode query
 * at position seq_len[b]-1 (it sees every present row).  n_rows > 1 is a
 * window: row r is the query of position seq_len[b] - n_rows + r and, when
 * `causal`, sees rows <= its position.  Query head h reads kv head
 * h / (num_q_heads / num_kv_heads).
 *
 * Each (row, head) takes a softmax of its logits (q . k) * scale over the
 * segment (NORM_SEGMENT) or over every row it sees (NORM_CONTEXT); the
 * probabilities of the segment tokens are summed over the rows and the heads
 * of a kv head's group (REDUCE_GROUP) or over all heads (REDUCE_ALL).  If
 * pool_width > 1 (odd), the sums are then averaged over a centred window of
 * pool_width tokens, zero-padded at the segment ends, always divided by
 * pool_width.
 *
 * scores: fp32 [batch][num_kv_heads or 1][ld], entry i is segment token
 * seg_begin[b] + i; entries past the segment length are not written.
 * Requires ld >= max_seg_len.  n_rows in [1, 64].  NORM_SEGMENT requires
 * n_rows == 1 (a window is always context-normalised).  n_rows > 1 uses
 * MFMA on the (n_rows x group) query rows of a kv head, 32 at a time: each
 * further block of 32 rows reads the keys twice more.  Workspace:
 * kvsel_score_workspace(kv, n_rows, num_q_heads, reduce, norm).
 */
KVSEL_API kvsel_status kvsel_score(const kvsel_kv_desc *kv, const uint16_t *q, int32_t n_rows,
                         int32_t num_q_heads, float scale, int32_t reduce, int32_t norm,
                         int32_t causal, int32_t pool_width, float *scores, int64_t ld,
                         void *ws, size_t ws_bytes, kvsel_stream stream);
KVSEL_API size_t kvsel_score_workspace(const kvsel_kv_desc *kv, int32_t n_rows, int32_t num_q_heads,
                             int32_t reduce, int32_t norm);

/*
 * kvsel_topk -- exact top-k per row.
 * (FastOCR Focal-Guided Pruning: keep the top tau of image tokens; FastKV 2A:
 *  keep the top-ranked tokens; Cross-Step Fixation Reuse: warm start.)
 *
 * scores: fp32 [rows][ld], the first n entries of each row are candidates.
 * idx: int32 [rows][k], the k indices (in [0, n)) of the largest scores,
 * ascending.  Among exactly equal scores the lower index is kept.  Scores
 * must not be NaN.
 *
 * n_per_row: NULL, or device int32 [rows]: row r's candidates are its first
 * min(n_per_row[r], n) entries (a negative count is 0).  A row with at most k
 * candidates gets all of them, ascending, and -1 in the remaining slots.
 *
 * warm_idx: NULL, or int32 [rows][k], a previous selection (strictly
 * ascending, in [0, n)).  Then theta = the lowest current score among the
 * warm indices and only tokens scoring >= theta are ranked; at least k of
 * them do, so the result is identical to the cold call.  A row whose warm
 * indices are not strictly ascending and in range is ranked cold.
 * Requires 1 <= k <= n <= ld, rows >= 1.
 */
KVSEL_API kvsel_status kvsel_topk(const float *scores, int64_t ld, int32_t rows, const int32_t *n_per_row,
                        int32_t n, int32_t k, const int32_t *warm_idx, int32_t *idx, void *ws,
                        size_t ws_bytes, kvsel_stream stream);
KVSEL_API size_t kvsel_topk_workspace(int32_t rows, int32_t n, int32_t k);

/*
 * kvsel_gather_attn -- decode attention over the kept rows.
 * (FastOCR Cross-Layer Propagation: non-focal layers attend only to the
 *  pruned set; FastKV 2B: decode over the retained KV.)
 *
 * q: bf16 [batch][num_q_heads][128], the decode query of position
 * seq_len[b]-1.  idx: int32 [batch][num_kv_heads][k], segment-relative
 * indices (row = seg_begin[b] + idx); an index outside the segment is
 * skipped.  For every q head, attention over R = {kept rows} U [0, seg_begin)
 * U [seg_end, seq_len): out = sum_R softmax((q . k_i) * scale) v_i.
 * Duplicate indices are attended once per occurrence: pass distinct indices.
 *
 * out: fp32 [batch][num_q_heads][128].  lse: NULL or fp32
 * [batch][num_q_heads], natural-log softmax normaliser (-inf if R is empty,
 * with out = 0).  k may be 0 (only the always-kept rows).
 */
KVSEL_API kvsel_status kvsel_gather_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads,
                               float scale, const int32_t *idx, int32_t k, float *out, float *lse,
                               void *ws, size_t ws_bytes, kvsel_stream stream);
/*
 * kvsel_gather_attn_noalloc -- kvsel_gather_attn without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * minus ws / ws_bytes, same result (up to summation order, as any two calls
 * of kvsel_gather_attn).  Scratch (the split records of pairs whose rows are
 * split over several work-groups) lives in a fixed 4 MiB device array of the
 * library, one per GPU, held until the process ends; its address is looked
 * up on the first call on each device.  A call that would need more scratch
 * than that returns KVSEL_ENOSPC before anything is enqueued (use
 * kvsel_gather_attn).  Every call on one GPU shares its array: calls that may
 * run at the same time on one GPU (other streams, other threads) race on it
 * and must not overlap.  The array needs no clearing: every record a call
 * reads it has written itself, and its per-pair arrival counters start at
 * zero (the array is zero when the library loads) and are left at zero by
 * every call.  Makes no allocation of any kind.
 */
KVSEL_API kvsel_status kvsel_gather_attn_noalloc(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads,
                                                 float scale, const int32_t *idx, int32_t k, float *out, float *lse,
                                                 kvsel_stream stream);

/* Workspace bytes for kvsel_gather_attn with budget k (k >= 0), or for
 * kvsel_dense_attn when k < 0 (with_scores: seg_scores will be passed; norm:
 * its normalisation).  0 if the descriptor or head count is invalid. */
KVSEL_API size_t kvsel_attn_workspace(const kvsel_kv_desc *kv, int32_t num_q_heads, int32_t k,
                            int32_t with_scores, int32_t norm);

/*
 * kvsel_dense_attn -- decode attention over every present row, optionally
 * fused with the focal score of the candidate segment.
 * (FastOCR Focal-Guided Pruning: only focal layers attend over the full KV
 *  cache, and select from that attention.)
 *
 * q, out, lse: as kvsel_gather_attn, with R = [0, seq_len).
 * seg_scores: NULL, or fp32 [batch][num_kv_heads][ld]: the same scores as
 * kvsel_score(n_rows = 1, REDUCE_GROUP, norm, pool_width = 1), taken from the
 * same pass over K.  Requires ld >= max_seg_len when seg_scores is set.
 * Workspace: kvsel_attn_workspace(kv, num_q_heads, -1, seg_scores != NULL,
 * norm).
 */
KVSEL_API kvsel_status kvsel_dense_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads,
                              float scale, float *out, float *lse, float *seg_scores, int64_t ld,
                              int32_t norm, void *ws, size_t ws_bytes, kvsel_stream stream);

/*
 * kvsel_focal_attn -- the fused focal pass: dense attention over every present
 * row, the focal score of the candidate segment from the same pass over K,
 * and the top-k of each (sequence, kv head).
 * (FastOCR Focal-Guided Pruning: a focal layer attends over the full cache
 *  and selects the top-attended image tokens; Cross-Step Fixation Reuse: the
 *  previous step's set warm-starts the selection.)
 *
 * Equal to kvsel_dense_attn(..., seg_scores, ld, norm) followed by
 * kvsel_topk(seg_scores, ld, batch * num_kv_heads, segment length, k,
 * warm_idx, idx): the same scores bit for bit and the same idx; out and lse
 * equal up to summation order (rows are handed to waves on demand).  q, out,
 * lse as kvsel_dense_attn; idx, warm_idx: int32 [batch][num_kv_heads][k]
 * (warm_idx NULL or a previous selection, see kvsel_topk).  seg_scores: NULL
 * or fp32 [batch][num_kv_heads][ld].  A sequence whose segment is shorter
 * than k keeps all of it and pads idx with -1 (skipped by gather attention).
 * Requires 1 <= k, max_seg_len <= 12288 (KVSEL_EUNSUPPORTED otherwise).
 * Workspace: kvsel_attn_workspace(kv, num_q_heads, -1, 1, norm).
 */
KVSEL_API kvsel_status kvsel_focal_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads,
                                        float scale, float *out, float *lse, int32_t norm, int32_t k,
                                        const int32_t *warm_idx, int32_t *idx, float *seg_scores, int64_t ld,
                                        void *ws, size_t ws_bytes, kvsel_stream stream);

/*
 * kvsel_gather_rows -- dst[j] = src[idx[j]] for j < n_idx, then
 * dst[n_idx + t] = src[tail_begin + t] for t < n_tail; rows of row_bytes
 * bytes, copied bit-exactly.
 * (FastKV 2A: the top-ranked tokens plus the window tokens are propagated.)
 *
 * row_bytes must be a positive multiple of 16; src, dst 16-byte aligned.
 * Indices outside [0, n_src_rows) produce a zero row.
 */
KVSEL_API kvsel_status kvsel_gather_rows(const void *src, int64_t row_bytes, int64_t n_src_rows,
                               const int32_t *idx, int32_t n_idx, int64_t tail_begin,
                               int32_t n_tail, void *dst, kvsel_stream stream);

/*
 * kvsel_visual_mass -- the image-attention ratio of each query head: the
 * share of its attention on the candidate segment.
 * (FastOCR Focal-Guided Pruning, Focal Layer Selection: a short warm-up
 *  profiles this ratio for every layer.)
 *
 * mass[b][h] = sum over i in [seg_begin[b], seg_end[b]) of softmax_i(scale *
 * q[b][h] . K[b][g(h)][i]), the softmax over every present row [0,
 * seq_len[b]); 0 for an empty segment.  q: bf16 [batch][num_q_heads][128];
 * mass: fp32 [batch][num_q_heads].  K is read once and V is not read
 * (v_pool may be NULL).  Workspace: kvsel_mass_workspace(kv, num_q_heads).
 */
KVSEL_API kvsel_status kvsel_visual_mass(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads,
                                         float scale, float *mass, void *ws, size_t ws_bytes, kvsel_stream stream);
KVSEL_API size_t kvsel_mass_workspace(const kvsel_kv_desc *kv, int32_t num_q_heads);

/*
 * kvsel_pick_layers -- the focal layers: the n_pick layers with the highest
 * mean image-attention ratio.
 * (FastOCR Focal-Guided Pruning, Focal Layer Selection: a small fixed set of
 *  layers with high concentration on image tokens.)
 *
 * ratios: fp32, device, layer l's n values at ratios[l * ld + j], j < n (for
 * instance the kvsel_visual_mass outputs of every warm-up step).  The means
 * are compared exactly (the sums are formed in integer arithmetic, so the
 * result does not depend on the order of the terms; a non-finite ratio
 * counts as 0); layers ranked by mean descending, equal means to the lower
 * layer; layers: int32 [n_pick], the chosen layers ascending.  Requires
 * 1 <= n_pick <= n_layers <= 1024, n >= 1, ld >= n.
 */
KVSEL_API kvsel_status kvsel_pick_layers(const float *ratios, int64_t ld, int32_t n_layers, int32_t n,
                                         int32_t n_pick, int32_t *layers, kvsel_stream stream);

/*
 * kvsel_verify_attn -- attention of m drafted tokens, verified in parallel.
 * (HPD-Parsing wiki, P-MTP: each branch drafts several tokens and verifies
 *  them in one step.)
 *
 * The drafts' own K/V rows are the last m rows of each sequence (positions
 * seq_len[b]-m .. seq_len[b]-1); a segment reaching into them is taken as
 * ending at seq_len[b]-m, so the drafts are always attended.  Draft r's
 * query, q[b][r][h], attends over the rows kvsel_gather_attn would attend
 * (kept rows seg_begin + idx, every row outside the segment) whose position
 * is <= seq_len[b]-m+r: everything before the drafts, and the drafts up to
 * its own.  q: bf16 [batch][m][num_q_heads][128]; idx: as kvsel_gather_attn
 * (NULL when k = 0); out: fp32 [batch][m][num_q_heads][128]; lse: NULL or
 * fp32 [batch][m][num_q_heads].  Requires m <= 64 and at most 8192
 * attended rows per (sequence, kv head), drafts included: k + max_seq_len -
 * min_seg_len + m <= 8192 (KVSEL_EUNSUPPORTED otherwise).  The query columns
 * (m x num_q_heads / num_kv_heads per kv head) run 32 at a time, each block
 * reading the rows once more.  No workspace.
 */
KVSEL_API kvsel_status kvsel_verify_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t m,
                                         int32_t num_q_heads, float scale, const int32_t *idx, int32_t k,
                                         float *out, float *lse, kvsel_stream stream);

/*
 * kvsel_prefill_attn -- causal prefill attention over the propagated tokens.
 * (FastKV, section 2A, Token-Selective Propagation: the layers after the
 *  TSP layer process only the top-ranked tokens and the window tokens.)
 *
 * Sequences are packed: sequence b holds rows cu_seqlens[b] ..
 * cu_seqlens[b+1]-1 (device array of batch + 1 non-decreasing int32; every
 * length <= max_seqlen, rows past max_seqlen are not computed).  The rows
 * keep their order of position, so row i of a sequence sees rows 0..i of
 * it.  q: bf16 [total][num_q_heads][128]; k, v: bf16
 * [total][num_kv_heads][128]; query head h reads kv head
 * h / (num_q_heads / num_kv_heads); scale > 0; out: fp32 [total][num_q_heads][128];
 * lse: NULL or fp32 [total][num_q_heads] (natural log).  q, k, v and out
 * 16-byte aligned.  P V runs in fp16 with V scaled by a power of two that
 * grows with the largest V magnitude each work-group has read: V of any
 * magnitude, each V value exact or off by less than 2^-20 of that largest
 * magnitude.  No workspace.
 */
KVSEL_API kvsel_status kvsel_prefill_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                          const int32_t *cu_seqlens, int32_t batch, int32_t max_seqlen,
                                          int32_t num_q_heads, int32_t num_kv_heads, float scale, float *out,
                                          float *lse, kvsel_stream stream);

/*
 * kvsel_shared_attn -- every sequence's queries over one shared row range.
 * (HPD-Parsing wiki, method item 2: the branches reuse the shared context's
 *  KV zero-copy.)  The part of each branch's attention that all branches
 * have in common, computed once per kv head for all of them.
 *
 * Rows [row_begin, row_end) must lie inside the shared rows
 * (kv->shared_rows) and be the same cache blocks in every sequence's block
 * table; they are read through sequence 0's.  The range is cut into
 * `splits` parts of whole 64-row tiles (1 .. 64; more parts, more
 * work-groups), each attended apart: part s writes out[s] and lse[s], to be
 * combined by kvsel_merge_attn.  q: bf16 [batch][q_per_seq][num_q_heads][128]
 * (q_per_seq queries per sequence: 1 for a decode step, m for m drafts);
 * out: fp32 [splits][batch][q_per_seq][num_q_heads][128], each part
 * normalised over its rows; lse: fp32 [splits][batch][q_per_seq][num_q_heads]
 * (natural log; -inf and out =
 * 0 for an empty part), NULL allowed when splits = 1.  accumulate = 1
 * (splits = 1, lse required): out and lse hold on entry the attention of
 * each query over other rows (normalised, with its lse, e.g. from
 * kvsel_gather_attn or kvsel_verify_attn), and the call replaces them with
 * the exact merge of that and this range (kvsel_merge_attn of the two, in
 * place; -inf lse for both gives out = 0).  q and out 16-byte
 * aligned; scale > 0; the range may touch at most 1024 cache blocks
 * (KVSEL_EUNSUPPORTED otherwise).  P V runs in fp16 with V scaled by a power
 * of two, as in kvsel_prefill_attn (V of any magnitude).  logits: NULL, or fp32 [batch][num_q_heads][ld_logits]
 * (q_per_seq = 1, ld_logits >= max_seg_len): the raw dots q.k of each
 * sequence's segment rows that lie inside the range, entry i for segment
 * row seg_begin + i (the input of kvsel_select_logits; rows outside the
 * range are not written).  A table entry of the range that is not a pool
 * block (< 0 or >= num_blocks) is skipped: its rows are not attended and
 * their logits are -inf.  No workspace.
 */
KVSEL_API kvsel_status kvsel_shared_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t q_per_seq,
                                         int32_t num_q_heads, float scale, int32_t row_begin, int32_t row_end,
                                         int32_t splits, int32_t accumulate, float *out, float *lse, float *logits,
                                         int64_t ld_logits, kvsel_stream stream);

/*
 * kvsel_select_logits -- the focal selection from segment logits: per
 * (sequence, kv head) the softmax over the candidate segment of each query
 * head of the group, summed over the group, and the exact top-k (ties to the
 * lower index, ascending, warm start as kvsel_focal_attn).  (FastOCR,
 * Focal-Guided Pruning: the focal layers select the top-attended image
 * tokens.)  logits: fp32 [batch][num_q_heads][ld_logits], the raw dots q.k
 * of segment row seg_begin + i at entry i (as kvsel_shared_attn writes them);
 * norm: KVSEL_NORM_SEGMENT; idx: [batch][num_kv_heads][k]; seg_scores: NULL
 * or fp32 [batch][num_kv_heads][ld].  max_seg_len <= 12288.
 */
KVSEL_API kvsel_status kvsel_select_logits(const kvsel_kv_desc *kv, const float *logits, int64_t ld_logits,
                                           int32_t num_q_heads, float scale, int32_t norm, int32_t k,
                                           const int32_t *warm_idx, int32_t *idx, float *seg_scores, int64_t ld,
                                           kvsel_stream stream);

/*
 * kvsel_merge_attn -- attention over the union of `parts` disjoint row sets
 * from the attention over each: out = sum_p o[p] e^lse[p] / sum_p e^lse[p],
 * lse_out = log sum_p e^lse[p] (a part with lse = -inf counts for nothing;
 * all empty gives out = 0, lse_out = -inf).  o: fp32 [parts][rows][128] and
 * out: fp32 [rows][128], 16-byte aligned; lse: fp32 [parts][rows]; lse_out:
 * fp32 [rows]; 1 <= parts <= 64.  out may be one of the parts of o and
 * lse_out one of the parts of lse (in place).
 */
KVSEL_API kvsel_status kvsel_merge_attn(const float *o, const float *lse, int32_t parts, int64_t rows, float *out,
                                        float *lse_out, kvsel_stream stream);

/*
 * Branch lifecycle: a reference-counted block pool (host side) and the fork
 * of a branch.
 * (HPD-Parsing wiki, inference scheduling: a content branch spawned at a
 *  fork token shares the parent's KV through a fork pointer, zero copy; the
 *  shared blocks are released by reference count once every branch holding
 *  them is done.)
 *
 * The pool hands out the physical block ids of one paged cache (as used in
 * block tables); each id has a reference count, and an id is free when its
 * count is 0.  A pool is not thread-safe.  kvsel_pool_create returns NULL
 * for num_blocks outside [1, 2^31).  kvsel_pool_refcount returns -1 for an
 * id out of range; kvsel_pool_free_count -1 for a NULL pool.
 */
typedef struct kvsel_block_pool kvsel_block_pool;
KVSEL_API kvsel_block_pool *kvsel_pool_create(int64_t num_blocks);
KVSEL_API void kvsel_pool_destroy(kvsel_block_pool *pool);
KVSEL_API int64_t kvsel_pool_free_count(const kvsel_block_pool *pool);
KVSEL_API int32_t kvsel_pool_refcount(const kvsel_block_pool *pool, int32_t block);
/* n free ids into ids, each with count 1 (KVSEL_ENOSPC if fewer are free). */
KVSEL_API kvsel_status kvsel_pool_alloc(kvsel_block_pool *pool, int32_t n, int32_t *ids);
/* Count + 1 for each allocated id (KVSEL_EINVAL for a free or bad id). */
KVSEL_API kvsel_status kvsel_pool_retain(kvsel_block_pool *pool, const int32_t *ids, int32_t n);
/* Count - 1 for each id; an id reaching 0 is free again.  Rejects (EINVAL,
 * nothing changed) a list holding an id more often than its count. */
KVSEL_API kvsel_status kvsel_pool_release(kvsel_block_pool *pool, const int32_t *ids, int32_t n);

/*
 * kvsel_fork -- the child's block table at a fork.  parent_table and
 * child_table are HOST int32 [max_blocks]; the parent holds parent_len rows.
 * Every block holding only rows below parent_len is shared (count + 1).  If
 * parent_len ends inside a block, a newly allocated block receives a copy of
 * it (every kv head's 16 rows of K and V, bit for bit; copy on write, since
 * both branches append after the fork point): one kernel enqueued on stream
 * (k_pool, v_pool: the cache's device pools [num_blocks][num_kv_heads][16][128]
 * bf16, and the pool's ids must all be below num_blocks; not needed when
 * parent_len is a multiple of 16).  child_table entries past the fork point
 * are -1.  KVSEL_ENOSPC if no block is free for the copy; nothing changes on
 * an error.
 */
KVSEL_API kvsel_status kvsel_fork(kvsel_block_pool *pool, const int32_t *parent_table, int32_t parent_len,
                                  int32_t max_blocks, int32_t *child_table, uint16_t *k_pool, uint16_t *v_pool,
                                  int64_t num_blocks, int32_t num_kv_heads, kvsel_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
