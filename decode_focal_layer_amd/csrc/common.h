// Device helpers shared by the libkvsel kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "debug.h"

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

// ---- wave64 reductions on DPP row operations and lane reads (no LDS) ----
// Within a 16-lane row every step combines a value with a mirrored partner,
// so all lanes of the row end with the same bits; the four row results are
// then read as scalars and combined in a fixed order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_u(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_u<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_u<0x141>(v));   // row_half_mirror
  v = op(v, dpp_u<0x140>(v));   // row_mirror
  return op(op(lane_u(v, 0), lane_u(v, 16)), op(lane_u(v, 32), lane_u(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u<CTRL>((uint32_t)u), hi = dpp_u<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double lane_d(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = lane_u((uint32_t)u, l), hi = lane_u((uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// sum over the wave in a fixed order, the same bits in every lane
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// inclusive prefix sum over the lanes of the wave
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u<0x111>(v);   // row_shr:1 (lanes without a source add 0)
  v += dpp_u<0x112>(v);   // row_shr:2
  v += dpp_u<0x114>(v);   // row_shr:4
  v += dpp_u<0x118>(v);   // row_shr:8
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t t0 = lane_u(v, 15), t1 = lane_u(v, 31), t2 = lane_u(v, 47);
  return v + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

}  // namespace kvsel
