// Bit-exact row gather: the selected tokens' hidden states, then the window
// tokens (FastKV section 2A: the top-ranked tokens plus the window tokens are
// propagated to the later layers).
//
// One work-group per output row; 16-byte loads and stores.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ src, int64_t row_vec,
                                                          int64_t n_src_rows, const int32_t *__restrict__ idx,
                                                          int32_t n_idx, int64_t tail_begin,
                                                          uint4 *__restrict__ dst) {
  const int j = blockIdx.x;
  const int64_t r = j < n_idx ? (int64_t)idx[j] : tail_begin + (j - n_idx);
  uint4 *d = dst + (size_t)j * row_vec;
  if (r < 0 || r >= n_src_rows) {
    for (int64_t t = threadIdx.x; t < row_vec; t += 256) d[t] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint4 *s = src + (size_t)r * row_vec;
  for (int64_t t = threadIdx.x; t < row_vec; t += 256) d[t] = s[t];
}

}  // namespace

hipError_t launch_gather_rows(const void *src, int64_t row_bytes, int64_t n_src_rows,
                              const int32_t *idx, int32_t n_idx, int64_t tail_begin, int32_t n_tail,
                              void *dst, hipStream_t s) {
  const int rows = n_idx + n_tail;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows), dim3(256), 0, s, (const uint4 *)src, row_bytes / 16,
                     n_src_rows, idx, n_idx, tail_begin, (uint4 *)dst);
  return hipGetLastError();
}

}  // namespace kvsel
