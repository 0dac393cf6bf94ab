// Focal-layer choice from the warm-up's image-attention ratios.
//
// FastOCR (technical summary, Focal-Guided Pruning, "Focal Layer
// Selection"): a short warm-up profiles each layer's image-attention ratio
// and fixes a small set of focal layers with high concentration on image
// tokens.  The ratios themselves come from the attention kernel's
// visual-mass mode (kvsel_visual_mass).
//
// One work-group of 256 threads.  Per layer, the mean of its n ratios in
// fp64 in a fixed order: thread t adds j = t, t + 256, ... in order, each
// wave's partials are reduced by wave_sum_d, the four wave sums are added in
// order.  Then layer l's rank is the number of layers with a larger mean, or
// an equal mean and a lower index; the layers ranked below n_pick are
// written in ascending order.
#include "common.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {

constexpr int kPickThreads = 256;

__global__ __launch_bounds__(kPickThreads) void pick_layers_kernel(const float *ratios, int64_t ld, int n_layers,
                                                                   int n, int n_pick, int32_t *layers) {
  __shared__ double s_mean[kMaxLayers];
  __shared__ double s_w[kPickThreads / 64];
  __shared__ uint8_t s_take[kMaxLayers];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int l = 0; l < n_layers; ++l) {
    const float *r = ratios + (size_t)l * ld;
    double part = 0.0;
    for (int j = tid; j < n; j += kPickThreads) part += (double)r[j];
    part = wave_sum_d(part);
    if (lane == 0) s_w[w] = part;
    __syncthreads();
    if (tid == 0) {
      double sum = 0.0;
      for (int i = 0; i < kPickThreads / 64; ++i) sum += s_w[i];
      s_mean[l] = sum / (double)n;
    }
    __syncthreads();
  }
  for (int l = tid; l < n_layers; l += kPickThreads) {
    const double ml = s_mean[l];
    int rank = 0;
    for (int m = 0; m < n_layers; ++m) {
      const double mm = s_mean[m];
      rank += (mm > ml || (mm == ml && m < l)) ? 1 : 0;
    }
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
