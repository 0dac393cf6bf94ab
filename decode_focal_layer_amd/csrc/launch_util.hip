// Host-side launch helpers.
#include <mutex>
#include <set>
#include <tuple>

#include "kvsel_internal.h"

namespace kvsel {

hipError_t allow_dynamic_lds(const void *fn, int bytes) {
  static std::mutex mu;
  static std::set<std::tuple<int, const void *, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, fn, bytes);
  if (done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert(key);
  return e;
}

}  // namespace kvsel
