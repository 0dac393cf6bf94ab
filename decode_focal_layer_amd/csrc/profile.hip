// Focal-layer choice from the warm-up's image-attention ratios.
//
// FastOCR (technical summary, Focal-Guided Pruning, "Focal Layer
// Selection"): a short warm-up profiles each layer's image-attention ratio
// and fixes a small set of focal layers with high concentration on image
// tokens.  The ratios themselves come from the attention kernel's
// visual-mass mode (kvsel_visual_mass).
//
// Layers are ranked by the mean of their n ratios.  Every layer has the same
// n, so the ranking is that of the sums, and the sums are taken EXACTLY: each
// fp32 ratio is m * 2^e with an integer m < 2^24 and e in [-149, 104], i.e.
// the integer m << (e + 149) of at most 277 bits.  These integers are added
// in radix-2^32 digits held in int64 limbs (a limb absorbs 2^31 digits
// without overflow), so the sum does not depend on the order of the
// additions, and two layers tie only when their exact sums are equal; then
// the lower layer ranks first.  A non-finite ratio counts as 0.
//
// One work-group of 1024 threads, one wave per layer at a time (wave w takes
// layers w, w + 16, ...): each lane adds its ratios j = lane, lane + 64, ...
// (16 loads in flight) into its own limbs; the limbs are summed over the
// wave's lanes; lane 0 propagates the carries into normalised digits (digit
// j in [0, 2^32), the remaining carry kept as a signed top word).
// Then layer l's rank is the number of layers with a larger sum, or an equal
// sum and a lower index; the layers ranked below n_pick are written in
// ascending order.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

constexpr int kPickThreads = 1024;
constexpr int kLimbs = 10;   // 320 bits: 277 for any finite fp32, the rest for carries

// add (sign) m << s into limbs
__device__ __forceinline__ void limbs_add(int64_t (&acc)[kLimbs], float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t be = (u >> 23) & 0xffu;
  if (be == 0xffu) return;   // inf or NaN: counts as 0
  const uint32_t m = be == 0 ? (u & 0x7fffffu) : ((u & 0x7fffffu) | 0x800000u);
  const int s = be == 0 ? 0 : (int)be - 1;   // e + 149: bit offset of m's lowest bit
  const uint64_t v = (uint64_t)m << (s & 31);
  const int li = s >> 5;
  const int64_t lo = (int64_t)(v & 0xffffffffu), hi = (int64_t)(v >> 32);
  const bool neg = (u >> 31) != 0u;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    const int64_t d = (j == li ? lo : 0) + (j == li + 1 ? hi : 0);
    acc[j] += neg ? -d : d;
  }
}

// a > b for normalised sums (signed top word, then digits from the most significant)
__device__ __forceinline__ bool sum_greater(const int32_t *top, const uint32_t (*dig)[kLimbs], int a, int b) {
  if (top[a] != top[b]) return top[a] > top[b];
  for (int j = kLimbs - 1; j >= 0; --j)
    if (dig[a][j] != dig[b][j]) return dig[a][j] > dig[b][j];
  return false;
}

__global__ __launch_bounds__(kPickThreads) void pick_layers_kernel(const float *ratios, int64_t ld, int n_layers,
                                                                   int n, int n_pick, int32_t *layers) {
  __shared__ uint32_t s_dig[kMaxLayers][kLimbs];
  __shared__ int32_t s_top[kMaxLayers];
  __shared__ uint8_t s_take[kMaxLayers];
  constexpr int NW = kPickThreads / 64, B = 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int l = w; l < n_layers; l += NW) {
    const float *r = ratios + (size_t)l * ld;
    int64_t acc[kLimbs];
#pragma unroll
    for (int j = 0; j < kLimbs; ++j) acc[j] = 0;
    for (int i0 = 0; i0 < n; i0 += B * 64) {
      float x[B];
#pragma unroll
      for (int u = 0; u < B; ++u) x[u] = r[min(i0 + u * 64 + lane, n - 1)];   // unbranched reads
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (i0 + u * 64 + lane < n) limbs_add(acc, x[u]);
    }
    // integer sums over the wave's lanes: exact in any order
#pragma unroll
    for (int j = 0; j < kLimbs; ++j)
      for (int off = 32; off >= 1; off >>= 1) acc[j] += __shfl_xor(acc[j], off);
    if (lane == 0) {
      int64_t carry = 0;
#pragma unroll
      for (int j = 0; j < kLimbs; ++j) {
        const int64_t v = acc[j] + carry;
        carry = v >> 32;   // arithmetic shift: v = carry * 2^32 + digit, digit in [0, 2^32)
        s_dig[l][j] = (uint32_t)(v - (carry << 32));
      }
      s_top[l] = (int32_t)carry;
    }
  }
  __syncthreads();
  for (int l = tid; l < n_layers; l += kPickThreads) {
    int rank = 0;
    for (int m = 0; m < n_layers; ++m)
      rank += (sum_greater(s_top, s_dig, m, l) || (m < l && !sum_greater(s_top, s_dig, l, m))) ? 1 : 0;
    s_take[l] = rank < n_pick ? 1 : 0;
  }
  __syncthreads();
  if (tid == 0) {
    int pos = 0;
    for (int l = 0; l < n_layers && pos < n_pick; ++l)
      if (s_take[l]) layers[pos++] = l;
  }
}

}  // namespace

hipError_t launch_pick_layers(const float *ratios, int64_t ld, int n_layers, int n, int n_pick, int32_t *layers,
                              hipStream_t s) {
  if (n_layers < 1 || n_layers > kMaxLayers || n < 1 || n_pick < 1 || n_pick > n_layers) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pick_layers_kernel, dim3(1), dim3(kPickThreads), 0, s, ratios, ld, n_layers, n, n_pick, layers);
  return hipGetLastError();
}

}  // namespace kvsel
