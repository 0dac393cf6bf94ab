// Branch lifecycle of a paged cache: a reference-counted block pool and the
// fork of a branch.
//
// HPD-Parsing wiki (inference scheduling): when the layout branch emits a
// fork token, the scheduler spawns a content branch that shares the
// parent's KV through a fork pointer, zero copy; the shared blocks are
// released by reference count once every branch holding them is done.
//
// Host side: per block a reference count, and a LIFO free list.  A fork
// shares every block that holds only rows before the fork point (count + 1)
// and gives the child a private copy of a block the parent has only partly
// filled (copy on write: both branches append after the fork point).  The
// copy is one small kernel on the caller's stream: every kv head's 16 rows
// of K and of V, bit for bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "kvsel_internal.h"

struct kvsel_block_pool {
  std::vector<int32_t> ref;         // reference count per block (0: free)
  std::vector<int32_t> free_list;   // free block ids; the back is handed out next
};

namespace kvsel {

kvsel_status pool_fail(kvsel_status s, const char *fmt, ...);   // api.hip: the thread's error text
void clear_error();

namespace {

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// one work-group per (kv head, pool): 4 KiB = 256 x 16 B
__global__ __launch_bounds__(256) void copy_block_kernel(uint4 *k_pool, uint4 *v_pool, int64_t src, int64_t dst,
                                                         int hkv) {
  const int h = blockIdx.x % hkv;
  uint4 *pool = blockIdx.x < hkv ? k_pool : v_pool;
  const size_t run = 4096 / sizeof(uint4);   // one (block, kv head) run of 16 rows x 128 bf16
  pool[((size_t)dst * hkv + h) * run + threadIdx.x] = pool[((size_t)src * hkv + h) * run + threadIdx.x];
}

// every id in range and, counting repeats, holding at least that many references
bool refs_ok(const kvsel_block_pool *p, const int32_t *ids, int32_t n) {
  std::unordered_map<int32_t, int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || (size_t)b >= p->ref.size()) return false;
    if (++need[b] > p->ref[b]) return false;
  }
  return true;
}

}  // namespace
}  // namespace kvsel

using namespace kvsel;

extern "C" {

kvsel_block_pool *kvsel_pool_create(int64_t num_blocks) {
  if (num_blocks < 1 || num_blocks > 0x7fffffff) return nullptr;
  kvsel_block_pool *p = new (std::nothrow) kvsel_block_pool;
  if (p == nullptr) return nullptr;
  p->ref.assign((size_t)num_blocks, 0);
  p->free_list.resize((size_t)num_blocks);
  for (int64_t i = 0; i < num_blocks; ++i) p->free_list[(size_t)i] = (int32_t)(num_blocks - 1 - i);   // 0 first
  return p;
}

void kvsel_pool_destroy(kvsel_block_pool *p) { delete p; }

int64_t kvsel_pool_free_count(const kvsel_block_pool *p) { return p ? (int64_t)p->free_list.size() : -1; }

int32_t kvsel_pool_refcount(const kvsel_block_pool *p, int32_t block) {
  if (p == nullptr || block < 0 || (size_t)block >= p->ref.size()) return -1;
  return p->ref[block];
}

kvsel_status kvsel_pool_alloc(kvsel_block_pool *p, int32_t n, int32_t *ids) {
  if (p == nullptr || (n > 0 && ids == nullptr) || n < 0) return pool_fail(KVSEL_EINVAL, "bad pool, n or ids");
  if ((size_t)n > p->free_list.size())
    return pool_fail(KVSEL_ENOSPC, "%d blocks requested, %zu free", n, p->free_list.size());
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = p->free_list.back();
    p->free_list.pop_back();
    p->ref[ids[i]] = 1;
  }
  clear_error();
  return KVSEL_OK;
}

kvsel_status kvsel_pool_retain(kvsel_block_pool *p, const int32_t *ids, int32_t n) {
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return pool_fail(KVSEL_EINVAL, "bad pool, n or ids");
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || (size_t)ids[i] >= p->ref.size() || p->ref[ids[i]] == 0)
      return pool_fail(KVSEL_EINVAL, "block %d is not allocated", ids[i]);
  for (int32_t i = 0; i < n; ++i) ++p->ref[ids[i]];
  clear_error();
  return KVSEL_OK;
}

kvsel_status kvsel_pool_release(kvsel_block_pool *p, const int32_t *ids, int32_t n) {
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return pool_fail(KVSEL_EINVAL, "bad pool, n or ids");
  if (!refs_ok(p, ids, n)) return pool_fail(KVSEL_EINVAL, "release of a block with no reference left");
  for (int32_t i = 0; i < n; ++i)
    if (--p->ref[ids[i]] == 0) p->free_list.push_back(ids[i]);
  clear_error();
  return KVSEL_OK;
}

kvsel_status kvsel_fork(kvsel_block_pool *p, const int32_t *parent_table, int32_t parent_len, int32_t max_blocks,
                        int32_t *child_table, uint16_t *k_pool, uint16_t *v_pool, int64_t num_blocks,
                        int32_t num_kv_heads, kvsel_stream stream) {
  if (p == nullptr || parent_table == nullptr || child_table == nullptr)
    return pool_fail(KVSEL_EINVAL, "pool, parent_table and child_table are required");
  if (max_blocks < 1 || parent_len < 0 || (int64_t)parent_len > (int64_t)max_blocks * kBlk)
    return pool_fail(KVSEL_EINVAL, "parent_len must be in [0, max_blocks*16]");
  const int32_t nfull = parent_len / kBlk;
  const bool partial = parent_len % kBlk != 0;
  const int32_t nused = nfull + (partial ? 1 : 0);
  if (!refs_ok(p, parent_table, nused)) return pool_fail(KVSEL_EINVAL, "the parent's blocks are not allocated");
  if (partial) {
    if (k_pool == nullptr || v_pool == nullptr || num_kv_heads < 1)
      return pool_fail(KVSEL_EINVAL, "k_pool, v_pool and num_kv_heads are needed to copy the partly filled block");
    if (!aligned16(k_pool) || !aligned16(v_pool)) return pool_fail(KVSEL_EINVAL, "pools must be 16-byte aligned");
    // every id the pool hands out must be a block of the device pools
    if ((int64_t)p->ref.size() > num_blocks)
      return pool_fail(KVSEL_EINVAL, "the block pool (%zu ids) is larger than the cache (%lld blocks)", p->ref.size(),
                       (long long)num_blocks);
    if ((uint64_t)num_blocks * (uint64_t)num_kv_heads * kBlk >= 0xffffffffull)
      return pool_fail(KVSEL_EUNSUPPORTED, "pool has 2^32 or more rows");
    if (p->free_list.empty()) return pool_fail(KVSEL_ENOSPC, "no free block for the copy of the partly filled block");
  }
  int32_t fresh = -1;
  if (partial) {
    fresh = p->free_list.back();
    hipLaunchKernelGGL(copy_block_kernel, dim3(2 * num_kv_heads), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint4 *>(k_pool), reinterpret_cast<uint4 *>(v_pool),
                       (int64_t)parent_table[nfull], (int64_t)fresh, num_kv_heads);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pool_fail(KVSEL_EHIP, "fork copy launch: %s", hipGetErrorString(e));
    p->free_list.pop_back();
    p->ref[fresh] = 1;
  }
  for (int32_t i = 0; i < nfull; ++i) ++p->ref[parent_table[i]];
  for (int32_t i = 0; i < max_blocks; ++i) child_table[i] = i < nfull ? parent_table[i] : -1;
  if (partial) child_table[nfull] = fresh;
  clear_error();
  return KVSEL_OK;
}

}  // extern "C"
