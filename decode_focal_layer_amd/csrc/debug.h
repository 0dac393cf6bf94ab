// Debug builds (compiled with -DKVSEL_DEBUG=1): device-side invariant checks.
//
// KVSEL_CHECK(cond, code, detail) states a fact the kernel relies on -- an
// address inside its pool, an LDS index inside its array, an output slot
// below k, a split counter that started at zero.  In a debug build a check
// that fails does not trap (a trap would take the whole device down): it
// counts the violation in a word of device memory and keeps the code and a
// detail of the first one.  kvsel_debug_status() reads and clears those words.
// Every source file has its own words (device globals are per translation
// unit here), registered with the host side when the library loads.  In a
// release build the checks compile to nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

// what a failed check was about (the first violation's code)
enum DbgCode : uint32_t {
  kDbgKvRow = 1,      // a K/V row outside its pool
  kDbgLds = 2,        // an LDS index outside its array
  kDbgOutSlot = 3,    // an output slot outside its row (top-k position >= k, ...)
  kDbgCounter = 4,    // a split arrival counter that did not start at zero
  kDbgSrcRow = 5,     // a source row outside its buffer (gather, pool copy)
  kDbgCount = 6,      // a count that breaks its bound (records, candidates)
};

// host side: reads this file's words (violations, first code, first detail)
// and clears them; returns false if the copy failed
typedef bool (*DbgTakeFn)(uint32_t out[3]);
bool dbg_register(DbgTakeFn f);

#if KVSEL_DEBUG
namespace {
__device__ uint32_t g_dbg_words[3];

__device__ __attribute__((noinline)) void dbg_fail(uint32_t code, uint32_t detail) {
  if (atomicAdd(&g_dbg_words[0], 1u) == 0u) {
    atomicExch(&g_dbg_words[1], code);
    atomicExch(&g_dbg_words[2], detail);
  }
}

bool dbg_take_this_file(uint32_t out[3]) {
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_dbg_words), sizeof(uint32_t) * 3) != hipSuccess) return false;
  const uint32_t zero[3] = {0u, 0u, 0u};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_words), zero, sizeof(zero)) == hipSuccess;
}

[[maybe_unused]] const bool g_dbg_registered = dbg_register(&dbg_take_this_file);
}  // namespace
#define KVSEL_CHECK(cond, code, detail)                                               \
  do {                                                                                \
    if (__builtin_expect(!(cond), 0)) ::kvsel::dbg_fail((code), (uint32_t)(detail)); \
  } while (0)
#else
#define KVSEL_CHECK(cond, code, detail) ((void)0)
#endif

}  // namespace kvsel
