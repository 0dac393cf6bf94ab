// libkvsel C-ABI: argument validation (pure host code, before any HIP call),
// workspace layout and launch of the kernels on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.h"
#include "kvsel_internal.h"
#include "mfma_kernels.h"

using namespace kvsel;

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace kvsel {
// sets the calling thread's error text (also used by the block pool)
kvsel_status pool_fail(kvsel_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}
void clear_error() { g_err[0] = 0; }
}  // namespace kvsel

namespace {

kvsel_status fail(kvsel_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

kvsel_status ok() {
  g_err[0] = 0;
  return KVSEL_OK;
}

kvsel_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(KVSEL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

kvsel_status check_desc(const kvsel_kv_desc *kv, bool need_v) {
  if (kv == nullptr) return fail(KVSEL_EINVAL, "kv descriptor is NULL");
  if (kv->head_dim != kD) return fail(KVSEL_EUNSUPPORTED, "head_dim %d unsupported (128 only)", kv->head_dim);
  if (kv->block_size != kBlk) return fail(KVSEL_EUNSUPPORTED, "block_size %d unsupported (16 only)", kv->block_size);
  if (kv->batch < 1) return fail(KVSEL_EINVAL, "batch must be >= 1");
  if (kv->num_kv_heads < 1) return fail(KVSEL_EINVAL, "num_kv_heads must be >= 1");
  if ((int64_t)kv->batch * kv->num_kv_heads > kMaxPairs)
    return fail(KVSEL_EUNSUPPORTED, "batch * num_kv_heads > %d", kMaxPairs);
  if (kv->max_blocks_per_seq < 1) return fail(KVSEL_EINVAL, "max_blocks_per_seq must be >= 1");
  if ((int64_t)kv->max_blocks_per_seq * kBlk > 0x7fffffff) return fail(KVSEL_EUNSUPPORTED, "sequence too long");
  if (kv->max_seq_len < 0 || (int64_t)kv->max_seq_len > (int64_t)kv->max_blocks_per_seq * kBlk)
    return fail(KVSEL_EINVAL, "max_seq_len must be in [0, max_blocks_per_seq*16]");
  if (kv->max_seg_len < 0 || kv->max_seg_len > kv->max_seq_len)
    return fail(KVSEL_EINVAL, "max_seg_len must be in [0, max_seq_len]");
  if (kv->min_seg_len < 0 || kv->min_seg_len > kv->max_seg_len)
    return fail(KVSEL_EINVAL, "min_seg_len must be in [0, max_seg_len]");
  if (kv->num_blocks < 1) return fail(KVSEL_EINVAL, "num_blocks must be >= 1");
  if ((uint64_t)kv->num_blocks * (uint64_t)kv->num_kv_heads * kBlk >= 0xffffffffull)
    return fail(KVSEL_EUNSUPPORTED, "pool has 2^32 or more rows");
  if (kv->shared_rows < 0) return fail(KVSEL_EINVAL, "shared_rows must be >= 0");
  if ((kv->flags & ~KVSEL_FLAG_DETERMINISTIC) != 0) return fail(KVSEL_EINVAL, "unknown flags 0x%x", kv->flags);
  if (!kv->k_pool || !kv->block_table || !kv->seq_len || !kv->seg_begin || !kv->seg_end)
    return fail(KVSEL_EINVAL, "k_pool, block_table, seq_len, seg_begin and seg_end are required");
  if (need_v && !kv->v_pool) return fail(KVSEL_EINVAL, "v_pool is required");
  if (!aligned(kv->k_pool, 16) || (kv->v_pool && !aligned(kv->v_pool, 16)))
    return fail(KVSEL_EINVAL, "k_pool and v_pool must be 16-byte aligned");
  return KVSEL_OK;
}

kvsel_status check_heads(const kvsel_kv_desc *kv, int32_t hq, int *group) {
  if (hq < 1 || hq % kv->num_kv_heads != 0)
    return fail(KVSEL_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", hq,
                kv->num_kv_heads);
  const int G = hq / kv->num_kv_heads;
  if (G < 1 || G > 8) return fail(KVSEL_EUNSUPPORTED, "group size %d unsupported (1 .. 8)", G);
  *group = G;
  return KVSEL_OK;
}

kvsel_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return KVSEL_OK;
  if (ws == nullptr) return fail(KVSEL_EINVAL, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, kAlign)) return fail(KVSEL_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(KVSEL_ENOSPC, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return KVSEL_OK;
}

int gather_rows_bound(const kvsel_kv_desc *kv, int32_t k) {
  const int64_t r = (int64_t)k + kv->max_seq_len - kv->min_seg_len;
  return (int)(r < 1 ? 1 : (r > 0x7fffffff ? 0x7fffffff : r));
}

int logit_mode_of(bool with_scores, int32_t norm) {
  return with_scores ? (norm == KVSEL_NORM_SEGMENT ? 1 : 2) : 0;
}

AttnArgs attn_args(const kvsel_kv_desc *kv, const uint16_t *q, int32_t hq, float scale, const int32_t *idx,
                   int32_t k, const AttnPlan &p, char *ws, float *out, float *lse, int logit_mode) {
  AttnArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = kv->block_table;
  a.seq_len = kv->seq_len;
  a.seg_begin = kv->seg_begin;
  a.seg_end = kv->seg_end;
  a.num_blocks = kv->num_blocks;
  a.max_blocks = kv->max_blocks_per_seq;
  a.shared_rows = kv->shared_rows;
  a.det = (kv->flags & KVSEL_FLAG_DETERMINISTIC) != 0 ? 1 : 0;
  a.hkv = kv->num_kv_heads;
  a.hq = hq;
  a.k = k;
  a.q = q;
  a.idx = idx;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rps = p.rps;
  a.nsplit = p.nsplit;
  a.counters = reinterpret_cast<uint32_t *>(ws + p.off_counters);
  a.rec = reinterpret_cast<float *>(ws + p.off_rec);
  a.out = out;
  a.lse = lse;
  a.logits = logit_mode ? reinterpret_cast<float *>(ws + p.off_logits) : nullptr;
  a.ld_logits = p.ld_logits;
  a.logit_mode = logit_mode;
  a.scale = (double)scale;
  return a;
}

SelArgs sel_args(const kvsel_kv_desc *kv, int32_t hq, int heads_per_out, int n_out, int32_t norm, float scale,
                 const float *logits, int64_t ld_logits) {
  SelArgs n{};
  n.logits = logits;
  n.ld_logits = ld_logits;
  n.seq_len = kv->seq_len;
  n.seg_begin = kv->seg_begin;
  n.seg_end = kv->seg_end;
  n.cap_rows = kv->max_blocks_per_seq * kBlk;
  n.hq = hq;
  n.heads_per_out = heads_per_out;
  n.n_out = n_out;
  n.norm = norm;
  n.scale = (double)scale;
  return n;
}

// kvsel_score scratch layout
struct ScorePlan {
  bool window = false;
  AttnPlan lp;      // decode: logits plan (rps, ld_logits, offsets)
  WinPlan wp;       // window
  size_t off_part = 0, total = 0;
  int64_t ld64 = 0;
};

ScorePlan score_plan(const kvsel_kv_desc *kv, int32_t n_rows, int32_t hq, int32_t reduce, int32_t norm,
                     int32_t pool_width) {
  ScorePlan sp;
  const int G = hq / kv->num_kv_heads;
  if (n_rows > 1) {
    sp.window = true;
    sp.wp = win_plan(kv->batch, kv->num_kv_heads, G, n_rows, kv->max_seq_len, kv->max_seg_len);
    sp.total = sp.wp.total;
    return sp;
  }
  const int mode = logit_mode_of(true, norm);
  const int rows = mode == 1 ? kv->max_seg_len : kv->max_seq_len;
  sp.lp = attn_plan(kv->batch, kv->num_kv_heads, hq, rows > 0 ? rows : 1, mode, kv->max_seg_len, kv->max_seq_len);
  // the logits kernel needs only the logit scratch; reuse the plan's layout from off_logits
  size_t off = sp.lp.off_extra;
  const bool need_part = pool_width > 1;
  sp.ld64 = kv->max_seg_len > 0 ? kv->max_seg_len : 1;
  if (need_part) {
    const int n_out = reduce == KVSEL_REDUCE_GROUP ? kv->num_kv_heads : 1;
    sp.off_part = off;
    off = align_up(off + (size_t)kv->batch * n_out * sp.ld64 * sizeof(double));
  }
  sp.total = off;
  return sp;
}

}  // namespace

// the debug words of every source file (debug builds register one reader per file)
namespace {
constexpr int kMaxDbgFiles = 64;
kvsel::DbgTakeFn g_dbg_fns[kMaxDbgFiles];   // zero before any dynamic initialisation runs
int g_dbg_n = 0;
}  // namespace

bool kvsel::dbg_register(DbgTakeFn f) {
  if (g_dbg_n >= kMaxDbgFiles) return false;
  g_dbg_fns[g_dbg_n++] = f;
  return true;
}

extern "C" {

int32_t kvsel_version(void) { return KVSEL_VERSION; }

kvsel_status kvsel_debug_status(uint32_t *violations, uint32_t *first_code, uint32_t *first_detail) {
  uint32_t total = 0, code = 0, detail = 0;
  if (violations != nullptr) *violations = 0;
  if (first_code != nullptr) *first_code = 0;
  if (first_detail != nullptr) *first_detail = 0;
#if KVSEL_DEBUG
  for (int i = 0; i < g_dbg_n; ++i) {
    uint32_t w[3];
    if (!g_dbg_fns[i](w)) return fail(KVSEL_EHIP, "reading the debug words failed");
    if (w[0] != 0u && total == 0u) {
      code = w[1];
      detail = w[2];
    }
    total += w[0];
  }
  if (violations != nullptr) *violations = total;
  if (first_code != nullptr) *first_code = code;
  if (first_detail != nullptr) *first_detail = detail;
  if (total != 0u) return fail(KVSEL_EDEBUG, "%u device check(s) failed; first: code %u, detail %u", total, code, detail);
  return ok();
#else
  (void)total;
  (void)code;
  (void)detail;
  return fail(KVSEL_EUNSUPPORTED, "not a debug build (compile with KVSEL_DEBUG=1)");
#endif
}

const char *kvsel_status_string(kvsel_status s) {
  switch (s) {
    case KVSEL_OK: return "ok";
    case KVSEL_EINVAL: return "invalid argument";
    case KVSEL_ENOSPC: return "workspace too small";
    case KVSEL_EUNSUPPORTED: return "unsupported shape";
    case KVSEL_EHIP: return "HIP error";
    case KVSEL_EDEBUG: return "device check failed";
    default: return "unknown status";
  }
}

const char *kvsel_last_error(void) { return g_err; }

// ------------------------------------------------------------------------
size_t kvsel_attn_workspace(const kvsel_kv_desc *kv, int32_t num_q_heads, int32_t k, int32_t with_scores,
                            int32_t norm) {
  int G;
  if (check_desc(kv, false) != KVSEL_OK || check_heads(kv, num_q_heads, &G) != KVSEL_OK) return 0;
  const int rows = k < 0 ? (kv->max_seq_len > 0 ? kv->max_seq_len : 1) : gather_rows_bound(kv, k);
  const int mode = k < 0 ? logit_mode_of(with_scores != 0, norm) : 0;
  return attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, rows, mode, kv->max_seg_len, kv->max_seq_len).total;
}

kvsel_status kvsel_gather_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads, float scale,
                               const int32_t *idx, int32_t k, float *out, float *lse, void *ws, size_t ws_bytes,
                               kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr) return fail(KVSEL_EINVAL, "out is NULL");
  if (k < 0) return fail(KVSEL_EINVAL, "k must be >= 0");
  if (k > 0 && idx == nullptr) return fail(KVSEL_EINVAL, "idx is NULL with k > 0");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  const AttnPlan p = attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, gather_rows_bound(kv, k), 0,
                               kv->max_seg_len, kv->max_seq_len);
  if ((st = check_ws(ws, ws_bytes, p.total)) != KVSEL_OK) return st;
  AttnArgs a = attn_args(kv, q, num_q_heads, scale, idx, k, p, (char *)ws, out, lse, 0);
  a.dense = 0;   // k == 0: only the always-attended rows
  return hip_status(launch_attn(a, kv->batch, G, (hipStream_t)stream), "gather_attn launch");
}

}  // extern "C"

// ------------------------------------------------------------------------
// Gathered attention without a caller workspace: the split records live in a
// fixed device array of this library, one per GPU (each device holds its own
// copy of a __device__ variable).  Its address is looked up once per device,
// with that device current, by hipGetSymbolAddress; host code only ever uses
// that address, never the array's name (which on the host is a stand-in, not
// a device address).
namespace {

constexpr size_t kNoAllocScratchBytes = 4u << 20;
constexpr int kNoAllocMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kNoAllocMaxDevices];   // per device, null until looked up

// this device's copy of `scratch`, looked up on the first call on the device
kvsel_status scratch_of_current_device(char **ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVSEL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(KVSEL_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || p == nullptr)
      return fail(KVSEL_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g));
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<char *>(g_scratch_ptr[dev]);
  return KVSEL_OK;
}

}  // namespace

extern "C" {

kvsel_status kvsel_gather_attn_noalloc(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads, float scale,
                                       const int32_t *idx, int32_t k, float *out, float *lse, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr) return fail(KVSEL_EINVAL, "out is NULL");
  if (k < 0) return fail(KVSEL_EINVAL, "k must be >= 0");
  if (k > 0 && idx == nullptr) return fail(KVSEL_EINVAL, "idx is NULL with k > 0");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  const AttnPlan p = attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, gather_rows_bound(kv, k), 0,
                               kv->max_seg_len, kv->max_seq_len);
  if (p.total > kNoAllocScratchBytes)
    return fail(KVSEL_ENOSPC, "the call needs %zu bytes of scratch; the fixed buffer holds %zu (use kvsel_gather_attn)",
                p.total, kNoAllocScratchBytes);
  char *ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != KVSEL_OK) return st;
  // the split records are written before they are read; the arrival
  // counters at the head of the layout start at zero (device memory of a
  // loaded module is zero-filled) and every call leaves them at zero
  AttnArgs a = attn_args(kv, q, num_q_heads, scale, idx, k, p, ws, out, lse, 0);
  a.dense = 0;
  return hip_status(launch_attn(a, kv->batch, G, (hipStream_t)stream), "gather_attn_noalloc launch");
}

kvsel_status kvsel_dense_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads, float scale, float *out,
                              float *lse, float *seg_scores, int64_t ld, int32_t norm, void *ws, size_t ws_bytes,
                              kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr) return fail(KVSEL_EINVAL, "out is NULL");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  if (seg_scores != nullptr) {
    if (norm != KVSEL_NORM_SEGMENT && norm != KVSEL_NORM_CONTEXT) return fail(KVSEL_EINVAL, "bad norm %d", norm);
    if (ld < kv->max_seg_len || ld < 1) return fail(KVSEL_EINVAL, "ld must be >= max_seg_len");
  }
  const int mode = logit_mode_of(seg_scores != nullptr, norm);
  const AttnPlan p = attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, kv->max_seq_len > 0 ? kv->max_seq_len : 1,
                               mode, kv->max_seg_len, kv->max_seq_len);
  if ((st = check_ws(ws, ws_bytes, p.total)) != KVSEL_OK) return st;
  AttnArgs a = attn_args(kv, q, num_q_heads, scale, nullptr, 0, p, (char *)ws, out, lse, mode);
  a.dense = 1;
  hipError_t e = launch_attn(a, kv->batch, G, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "dense_attn launch");
  if (seg_scores == nullptr) return ok();
  SelArgs n = sel_args(kv, num_q_heads, G, kv->num_kv_heads, norm, scale, a.logits, p.ld_logits);
  n.scores = seg_scores;
  n.ld = ld;
  return hip_status(launch_focal_norm(n, kv->batch, (hipStream_t)stream), "focal score launch");
}

kvsel_status kvsel_verify_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t m, int32_t num_q_heads,
                               float scale, const int32_t *idx, int32_t k, float *out, float *lse,
                               kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (m < 1) return fail(KVSEL_EINVAL, "m must be >= 1");
  if (m > 64) return fail(KVSEL_EUNSUPPORTED, "m = %d drafts (1 .. 64)", m);
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr) return fail(KVSEL_EINVAL, "out is NULL");
  if (k < 0) return fail(KVSEL_EINVAL, "k must be >= 0");
  if (k > 0 && idx == nullptr) return fail(KVSEL_EINVAL, "idx is NULL with k > 0");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  // a segment reaching into the drafts is cut before them: up to m more rows
  const int64_t rows_cap = (int64_t)gather_rows_bound(kv, k) + m;
  if (rows_cap > kVerifyMaxRows)
    return fail(KVSEL_EUNSUPPORTED, "more than %d attended rows per (sequence, kv head)", kVerifyMaxRows);
  VerifyArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = kv->block_table;
  a.seq_len = kv->seq_len;
  a.seg_begin = kv->seg_begin;
  a.seg_end = kv->seg_end;
  a.num_blocks = kv->num_blocks;
  a.max_blocks = kv->max_blocks_per_seq;
  a.hkv = kv->num_kv_heads;
  a.hq = num_q_heads;
  a.group = G;
  a.m = m;
  a.k = k;
  a.q = q;
  a.idx = idx;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.rows_cap = (int32_t)rows_cap;
  return hip_status(launch_verify(a, kv->batch, (hipStream_t)stream), "verify_attn launch");
}

kvsel_status kvsel_prefill_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu_seqlens,
                                int32_t batch, int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                                float scale, float *out, float *lse, kvsel_stream stream) {
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens == nullptr || out == nullptr)
    return fail(KVSEL_EINVAL, "q, k, v, cu_seqlens and out are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(KVSEL_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (batch < 1 || batch > 65535) return fail(KVSEL_EINVAL, "batch must be in [1, 65535]");
  if (num_kv_heads < 1 || num_kv_heads > 65535 || num_q_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(KVSEL_EINVAL, "num_q_heads must be a positive multiple of num_kv_heads (1 .. 65535)");
  if (max_seqlen < 0) return fail(KVSEL_EINVAL, "max_seqlen must be >= 0");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(KVSEL_EINVAL, "scale must be finite and positive");
  const int G = num_q_heads / num_kv_heads;
  if ((int64_t)num_kv_heads * kD * 2 * 64 >= 0xffffffffll) return fail(KVSEL_EUNSUPPORTED, "num_kv_heads too large");
  if ((int64_t)max_seqlen * G > 0x7fffff00ll) return fail(KVSEL_EUNSUPPORTED, "max_seqlen * group >= 2^31");
  if (((int64_t)max_seqlen * G + 127) / 128 * num_kv_heads * batch >= 0x7ffffff0ll)
    return fail(KVSEL_EUNSUPPORTED, "too many 128-row blocks");
  if (max_seqlen == 0) {
    clear_error();
    return KVSEL_OK;
  }
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seqlens;
  a.out = out;
  a.lse = lse;
  a.max_seqlen = max_seqlen;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = G;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(launch_prefill(a, batch, (hipStream_t)stream), "prefill_attn launch");
}

kvsel_status kvsel_shared_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t q_per_seq, int32_t num_q_heads,
                               float scale, int32_t row_begin, int32_t row_end, int32_t splits, int32_t accumulate,
                               float *out, float *lse, float *logits, int64_t ld_logits, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr || !aligned(out, 16)) return fail(KVSEL_EINVAL, "out must be a 16-byte aligned pointer");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(KVSEL_EINVAL, "scale must be finite and positive");
  if (row_begin < 0 || row_end < row_begin || row_end > kv->shared_rows ||
      (int64_t)row_end > (int64_t)kv->max_blocks_per_seq * kBlk)
    return fail(KVSEL_EINVAL, "rows [%d, %d) must lie inside the shared rows [0, %d)", row_begin, row_end,
                kv->shared_rows);
  if (row_end > row_begin && ((row_end - 1) >> 4) - (row_begin >> 4) + 1 > kSharedMaxBlocks)
    return fail(KVSEL_EUNSUPPORTED, "the range touches more than %d cache blocks", kSharedMaxBlocks);
  if (splits < 1 || splits > kMaxMergeParts) return fail(KVSEL_EINVAL, "splits must be in [1, %d]", kMaxMergeParts);
  if (splits > 1 && lse == nullptr) return fail(KVSEL_EINVAL, "lse is required with splits > 1");
  if (accumulate != 0 && accumulate != 1) return fail(KVSEL_EINVAL, "accumulate must be 0 or 1");
  if (accumulate && (splits != 1 || lse == nullptr))
    return fail(KVSEL_EINVAL, "accumulate needs splits = 1 and lse");
  if (q_per_seq < 1 || (int64_t)kv->batch * q_per_seq * G > 0x7fffff00ll)
    return fail(KVSEL_EINVAL, "q_per_seq must be >= 1 (and batch * q_per_seq * group < 2^31)");
  if (logits != nullptr && (q_per_seq != 1 || ld_logits < kv->max_seg_len || ld_logits < 1))
    return fail(KVSEL_EINVAL, "logits need q_per_seq = 1 and ld_logits >= max_seg_len");
  SharedArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.table = kv->block_table;   // sequence 0's row: the shared rows are the same blocks in every table
  a.num_blocks = kv->num_blocks;
  a.hkv = kv->num_kv_heads;
  a.hq = num_q_heads;
  a.group = G;
  a.batch = kv->batch * q_per_seq;   // every query of every sequence sees the same shared rows
  a.row_begin = row_begin;
  a.row_end = row_end;
  a.splits = splits;
  a.accumulate = accumulate;
  a.q = q;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  a.logits = logits;
  a.ld_logits = ld_logits;
  a.seg_begin = kv->seg_begin;
  a.seg_end = kv->seg_end;
  return hip_status(launch_shared(a, (hipStream_t)stream), "shared_attn launch");
}

kvsel_status kvsel_select_logits(const kvsel_kv_desc *kv, const float *logits, int64_t ld_logits,
                                 int32_t num_q_heads, float scale, int32_t norm, int32_t k, const int32_t *warm_idx,
                                 int32_t *idx, float *seg_scores, int64_t ld, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, false)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (logits == nullptr || idx == nullptr) return fail(KVSEL_EINVAL, "logits and idx are required");
  if (ld_logits < kv->max_seg_len || ld_logits < 1) return fail(KVSEL_EINVAL, "ld_logits must be >= max_seg_len");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  if (norm != KVSEL_NORM_SEGMENT) return fail(KVSEL_EINVAL, "only the segment normalisation is selected from logits");
  if (k < 1) return fail(KVSEL_EINVAL, "k must be >= 1");
  if (kv->max_seg_len > kSelMaxSeg)
    return fail(KVSEL_EUNSUPPORTED, "max_seg_len %d > %d", kv->max_seg_len, kSelMaxSeg);
  if (seg_scores != nullptr && (ld < kv->max_seg_len || ld < 1)) return fail(KVSEL_EINVAL, "ld must be >= max_seg_len");
  SelArgs n = sel_args(kv, num_q_heads, G, kv->num_kv_heads, norm, scale, logits, ld_logits);
  n.scores = seg_scores;
  n.ld = seg_scores != nullptr ? ld : 0;
  n.k = k;
  n.warm = warm_idx;
  n.idx = idx;
  return hip_status(launch_focal_select(n, kv->batch, (hipStream_t)stream), "select from logits launch");
}

kvsel_status kvsel_merge_attn(const float *o, const float *lse, int32_t parts, int64_t rows, float *out,
                              float *lse_out, kvsel_stream stream) {
  if (o == nullptr || lse == nullptr || out == nullptr || lse_out == nullptr)
    return fail(KVSEL_EINVAL, "o, lse, out and lse_out are required");
  if (!aligned(o, 16) || !aligned(out, 16)) return fail(KVSEL_EINVAL, "o and out must be 16-byte aligned");
  if (parts < 1 || parts > kMaxMergeParts) return fail(KVSEL_EINVAL, "parts must be in [1, %d]", kMaxMergeParts);
  if (rows < 0) return fail(KVSEL_EINVAL, "rows must be >= 0");
  return hip_status(launch_merge(o, lse, parts, rows, out, lse_out, (hipStream_t)stream), "merge_attn launch");
}

size_t kvsel_mass_workspace(const kvsel_kv_desc *kv, int32_t num_q_heads) {
  int G;
  if (check_desc(kv, false) != KVSEL_OK || check_heads(kv, num_q_heads, &G) != KVSEL_OK) return 0;
  return attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, kv->max_seq_len > 0 ? kv->max_seq_len : 1, 0,
                   kv->max_seg_len, kv->max_seq_len)
      .total;
}

kvsel_status kvsel_visual_mass(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads, float scale,
                               float *mass, void *ws, size_t ws_bytes, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, false)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (mass == nullptr) return fail(KVSEL_EINVAL, "mass is NULL");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  const AttnPlan p = attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, kv->max_seq_len > 0 ? kv->max_seq_len : 1, 0,
                               kv->max_seg_len, kv->max_seq_len);
  if ((st = check_ws(ws, ws_bytes, p.total)) != KVSEL_OK) return st;
  AttnArgs a = attn_args(kv, q, num_q_heads, scale, nullptr, 0, p, (char *)ws, nullptr, nullptr, 0);
  a.dense = 1;
  a.mass = mass;
  return hip_status(launch_attn(a, kv->batch, G, (hipStream_t)stream), "visual_mass launch");
}

kvsel_status kvsel_pick_layers(const float *ratios, int64_t ld, int32_t n_layers, int32_t n, int32_t n_pick,
                               int32_t *layers, kvsel_stream stream) {
  if (ratios == nullptr || layers == nullptr) return fail(KVSEL_EINVAL, "ratios and layers are required");
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(KVSEL_EINVAL, "n_layers must be in [1, %d]", kMaxLayers);
  if (n < 1) return fail(KVSEL_EINVAL, "n must be >= 1");
  if (ld < n) return fail(KVSEL_EINVAL, "ld must be >= n");
  if (n_pick < 1 || n_pick > n_layers) return fail(KVSEL_EINVAL, "n_pick must be in [1, n_layers]");
  return hip_status(launch_pick_layers(ratios, ld, n_layers, n, n_pick, layers, (hipStream_t)stream),
                    "pick_layers launch");
}

kvsel_status kvsel_focal_attn(const kvsel_kv_desc *kv, const uint16_t *q, int32_t num_q_heads, float scale, float *out,
                              float *lse, int32_t norm, int32_t k, const int32_t *warm_idx, int32_t *idx,
                              float *seg_scores, int64_t ld, void *ws, size_t ws_bytes, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, true)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (out == nullptr || idx == nullptr) return fail(KVSEL_EINVAL, "out and idx are required");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  if (norm != KVSEL_NORM_SEGMENT && norm != KVSEL_NORM_CONTEXT) return fail(KVSEL_EINVAL, "bad norm %d", norm);
  if (k < 1) return fail(KVSEL_EINVAL, "k must be >= 1");
  if (kv->max_seg_len > kSelMaxSeg)
    return fail(KVSEL_EUNSUPPORTED, "max_seg_len %d > %d: use kvsel_dense_attn + kvsel_topk", kv->max_seg_len,
                kSelMaxSeg);
  if (seg_scores != nullptr && (ld < kv->max_seg_len || ld < 1)) return fail(KVSEL_EINVAL, "ld must be >= max_seg_len");
  const int mode = logit_mode_of(true, norm);
  const AttnPlan p = attn_plan(kv->batch, kv->num_kv_heads, num_q_heads, kv->max_seq_len > 0 ? kv->max_seq_len : 1,
                               mode, kv->max_seg_len, kv->max_seq_len);
  if ((st = check_ws(ws, ws_bytes, p.total)) != KVSEL_OK) return st;
  AttnArgs a = attn_args(kv, q, num_q_heads, scale, nullptr, 0, p, (char *)ws, out, lse, mode);
  a.dense = 1;
  // the fused form's selecting waves leave the streaming part way: it is taken
  // only when the rows may be summed in any order
  if (p.nsplit == 1 && norm == KVSEL_NORM_SEGMENT && fused_focal_fits(G, kv->max_seg_len) && a.det == 0) {
    // one kernel: attention, segment logits kept in LDS, selection per (sequence, kv head)
    a.logits = nullptr;
    a.sel_idx = idx;
    a.sel_warm = warm_idx;
    a.sel_k = k;
    a.sel_scores = seg_scores;
    a.sel_ld = seg_scores != nullptr ? ld : 0;
    a.seg_cap = (kv->max_seg_len + 3) / 4 * 4;
    return hip_status(launch_attn(a, kv->batch, G, (hipStream_t)stream), "focal attention launch");
  }
  hipError_t e = launch_attn(a, kv->batch, G, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "focal attention launch");
  SelArgs n = sel_args(kv, num_q_heads, G, kv->num_kv_heads, norm, scale, a.logits, p.ld_logits);
  n.scores = seg_scores;
  n.ld = seg_scores != nullptr ? ld : 0;
  n.k = k;
  n.warm = warm_idx;
  n.idx = idx;
  return hip_status(launch_focal_select(n, kv->batch, (hipStream_t)stream), "focal select launch");
}

// ------------------------------------------------------------------------
size_t kvsel_score_workspace(const kvsel_kv_desc *kv, int32_t n_rows, int32_t num_q_heads, int32_t reduce,
                             int32_t norm) {
  int G;
  if (check_desc(kv, false) != KVSEL_OK || check_heads(kv, num_q_heads, &G) != KVSEL_OK) return 0;
  if (n_rows < 1) return 0;
  // the pool post-pass scratch is sized for any pool width
  return score_plan(kv, n_rows, num_q_heads, reduce, norm, 3).total;
}

kvsel_status kvsel_score(const kvsel_kv_desc *kv, const uint16_t *q, int32_t n_rows, int32_t num_q_heads, float scale,
                         int32_t reduce, int32_t norm, int32_t causal, int32_t pool_width, float *scores, int64_t ld,
                         void *ws, size_t ws_bytes, kvsel_stream stream) {
  kvsel_status st;
  int G;
  if ((st = check_desc(kv, false)) != KVSEL_OK) return st;
  if ((st = check_heads(kv, num_q_heads, &G)) != KVSEL_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return fail(KVSEL_EINVAL, "q must be a 16-byte aligned pointer");
  if (scores == nullptr) return fail(KVSEL_EINVAL, "scores is NULL");
  if (n_rows < 1 || n_rows > 64) return fail(KVSEL_EINVAL, "n_rows must be in [1, 64]");
  if (reduce != KVSEL_REDUCE_GROUP && reduce != KVSEL_REDUCE_ALL) return fail(KVSEL_EINVAL, "bad reduce %d", reduce);
  if (norm != KVSEL_NORM_SEGMENT && norm != KVSEL_NORM_CONTEXT) return fail(KVSEL_EINVAL, "bad norm %d", norm);
  if (n_rows > 1 && norm != KVSEL_NORM_CONTEXT)
    return fail(KVSEL_EINVAL, "a query window (n_rows > 1) is context-normalised");
  if (pool_width < 1 || pool_width % 2 == 0) return fail(KVSEL_EINVAL, "pool_width must be odd and >= 1");
  if (ld < kv->max_seg_len || ld < 1) return fail(KVSEL_EINVAL, "ld must be >= max_seg_len");
  if (!isfinite(scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  const ScorePlan sp = score_plan(kv, n_rows, num_q_heads, reduce, norm, pool_width);
  if ((st = check_ws(ws, ws_bytes, sp.total)) != KVSEL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char *w = (char *)ws;
  const int n_out = reduce == KVSEL_REDUCE_GROUP ? kv->num_kv_heads : 1;

  if (sp.window) {
    WinArgs a{};
    a.k_pool = kv->k_pool;
    a.block_table = kv->block_table;
    a.seq_len = kv->seq_len;
    a.seg_begin = kv->seg_begin;
    a.seg_end = kv->seg_end;
    a.num_blocks = kv->num_blocks;
    a.max_blocks = kv->max_blocks_per_seq;
    a.hkv = kv->num_kv_heads;
    a.hq = num_q_heads;
    a.group = G;
    a.n_rows = n_rows;
    a.causal = causal ? 1 : 0;
    a.q = q;
    a.scale = (double)scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.tile_rows = sp.wp.tile_rows;
    a.ntiles = sp.wp.ntiles;
    a.stat = reinterpret_cast<float *>(w + sp.wp.off_stat);
    a.rowstat = reinterpret_cast<double *>(w + sp.wp.off_rowstat);
    a.part = reinterpret_cast<double *>(w + sp.wp.off_part);
    a.ld64 = sp.wp.ld64;
    hipError_t e = launch_window(a, sp.wp, kv->batch, s);
    if (e != hipSuccess) return hip_status(e, "window score launch");
    PoolArgs pa{};
    pa.part = a.part;
    pa.ld64 = a.ld64;
    pa.n_in = kv->num_kv_heads;
    pa.n_out = n_out;
    pa.seq_len = kv->seq_len;
    pa.seg_begin = kv->seg_begin;
    pa.seg_end = kv->seg_end;
    pa.cap_rows = kv->max_blocks_per_seq * kBlk;
    pa.width = pool_width;
    pa.scores = scores;
    pa.ld = ld;
    return hip_status(launch_pool(pa, kv->batch, kv->max_seg_len, s), "pool launch");
  }

  const int mode = logit_mode_of(true, norm);
  const int rows = mode == 1 ? kv->max_seg_len : kv->max_seq_len;
  const AttnArgs a = attn_args(kv, q, num_q_heads, scale, nullptr, 0, sp.lp, w, nullptr, nullptr, mode);
  hipError_t e = launch_logits(a, kv->batch, G, rows, s);
  if (e != hipSuccess) return hip_status(e, "score logits launch");
  SelArgs n = sel_args(kv, num_q_heads, reduce == KVSEL_REDUCE_GROUP ? G : num_q_heads, n_out, norm, scale, a.logits,
                       sp.lp.ld_logits);
  if (pool_width == 1) {
    n.scores = scores;
    n.ld = ld;
    return hip_status(launch_focal_norm(n, kv->batch, s), "score launch");
  }
  n.scores64 = reinterpret_cast<double *>(w + sp.off_part);
  n.ld64 = sp.ld64;
  e = launch_focal_norm(n, kv->batch, s);
  if (e != hipSuccess) return hip_status(e, "score launch");
  PoolArgs pa{};
  pa.part = n.scores64;
  pa.ld64 = sp.ld64;
  pa.n_in = n_out;
  pa.n_out = n_out;
  pa.seq_len = kv->seq_len;
  pa.seg_begin = kv->seg_begin;
  pa.seg_end = kv->seg_end;
  pa.cap_rows = kv->max_blocks_per_seq * kBlk;
  pa.width = pool_width;
  pa.scores = scores;
  pa.ld = ld;
  return hip_status(launch_pool(pa, kv->batch, kv->max_seg_len, s), "pool launch");
}

// ------------------------------------------------------------------------
size_t kvsel_topk_workspace(int32_t rows, int32_t n, int32_t k) {
  if (rows < 1 || k < 1 || k > n) return 0;
  return topk_workspace_bytes(rows, n);
}

kvsel_status kvsel_topk(const float *scores, int64_t ld, int32_t rows, const int32_t *n_per_row, int32_t n, int32_t k,
                        const int32_t *warm_idx, int32_t *idx, void *ws, size_t ws_bytes, kvsel_stream stream) {
  kvsel_status st;
  if (scores == nullptr || idx == nullptr) return fail(KVSEL_EINVAL, "scores and idx are required");
  if (rows < 1) return fail(KVSEL_EINVAL, "rows must be >= 1");
  if (k < 1 || k > n) return fail(KVSEL_EINVAL, "need 1 <= k <= n (k=%d, n=%d)", k, n);
  if ((int64_t)n > ld) return fail(KVSEL_EINVAL, "need n <= ld");
  if (rows > 65535) return fail(KVSEL_EINVAL, "rows must be <= 65535");
  if ((st = check_ws(ws, ws_bytes, topk_workspace_bytes(rows, n))) != KVSEL_OK) return st;
  TopkArgs a{scores, ld, rows, n, k, warm_idx, idx, n_per_row};
  return hip_status(launch_topk(a, ws, (hipStream_t)stream), "topk launch");
}

// ------------------------------------------------------------------------
kvsel_status kvsel_gather_rows(const void *src, int64_t row_bytes, int64_t n_src_rows, const int32_t *idx,
                               int32_t n_idx, int64_t tail_begin, int32_t n_tail, void *dst, kvsel_stream stream) {
  if (src == nullptr || dst == nullptr) return fail(KVSEL_EINVAL, "src and dst are required");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(KVSEL_EINVAL, "src and dst must be 16-byte aligned");
  if (row_bytes <= 0 || row_bytes % 16 != 0) return fail(KVSEL_EINVAL, "row_bytes must be a positive multiple of 16");
  if (n_idx < 0 || n_tail < 0 || n_src_rows < 0) return fail(KVSEL_EINVAL, "negative count");
  if (n_idx > 0 && idx == nullptr) return fail(KVSEL_EINVAL, "idx is NULL with n_idx > 0");
  if ((int64_t)n_idx + n_tail > 0x7fffffff) return fail(KVSEL_EINVAL, "too many rows");
  return hip_status(launch_gather_rows(src, row_bytes, n_src_rows, idx, n_idx, tail_begin, n_tail, dst,
                                       (hipStream_t)stream),
                    "gather_rows launch");
}

}  // extern "C"
