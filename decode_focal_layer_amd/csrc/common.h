// Device helpers shared by the libkvsel kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace kvsel {

constexpr int kD = 128;        // head_dim
constexpr int kBlk = 16;       // rows per cache block
constexpr uint32_t kNoRow = 0xffffffffu;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 in a uint4 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4 &v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the
// same bits (each step adds a value and its mirror, and fp add commutes).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^(m - mnew) with an empty side (m == -inf) contributing nothing.
__device__ __forceinline__ float rescale(float m, float mnew) {
  return m == -INFINITY ? 0.f : fast_exp2(m - mnew);
}

// 2^x to about one fp32 ulp of relative error for x in the fp32 exponent
// range: the fp32 part of x goes through the hardware exp2 and the remainder
// through the first-order term 2^xl ~ 1 + xl ln 2 (|xl| < 2^-24 |x|).
__device__ __forceinline__ double exp2_acc(double x) {
  const float xh = (float)x;
  const double xl = x - (double)xh;
  return (double)__builtin_amdgcn_exp2f(xh) * (1.0 + xl * 0.6931471805599453);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---- block reductions (blockDim.x a multiple of 64, <= 1024) ----
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// scratch must hold blockDim.x/64 entries; result valid in every thread
__device__ __forceinline__ float block_max(float v, float *scratch) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, double *scratch) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < nw; ++i) r += scratch[i];
  return r;
}

// Sum of val(i) over i in [0, n) with the reduction order of a 1024-thread
// block: virtual thread v (= tid + r * NT) takes i = v, v + 1024, ... in
// order, each virtual wave reduces with xor shuffles (32, 16, ..., 1), and the
// 16 virtual-wave sums are added in order.  The result is bit-identical for
// any NT dividing 1024.  scratch holds 16 doubles; result in every thread.
template <int NT, typename F>
__device__ __forceinline__ double vsum1024(F val, int n, double *scratch) {
  constexpr int R = 1024 / NT;
  const int tid = threadIdx.x;
  double part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    part[r] = 0.0;
    for (int i = tid + r * NT; i < n; i += 1024) part[r] += val(i);
    part[r] = wave_sum_d(part[r]);
  }
  __syncthreads();
  if ((tid & 63) == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) scratch[(tid >> 6) + r * (NT / 64)] = part[r];
  }
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < 16; ++w) s += scratch[w];
  __syncthreads();
  return s;
}

// max of val(i) over i in [0, n); scratch holds NT/64 floats
template <int NT, typename F>
__device__ __forceinline__ float vmax(F val, int n, float *scratch) {
  float m = -INFINITY;
  for (int i = threadIdx.x; i < n; i += NT) m = fmaxf(m, val(i));
  m = wave_max(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, scratch[w]);
  __syncthreads();
  return r;
}

}  // namespace kvsel
