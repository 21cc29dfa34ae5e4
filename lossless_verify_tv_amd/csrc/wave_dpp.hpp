// Wavefront (64-lane) reductions built from DPP row moves, one swizzle and
// two lane reads (gfx950). Unlike shuffles through ds_bpermute they need no
// per-lane address registers, which matters in kernels that keep whole
// slices of a row in registers. Every lane gets the same result.
//
// Order of the steps: within quads (lane ^ 1, lane ^ 2), then mirrored
// half-rows and rows (8 and 16 lanes), then lane ^ 16 inside each half of the
// wave, then the two halves read from lanes 0 and 32. The order is fixed,
// so a reduction of the same values always gives the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace lvtv {

namespace dpp {
constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror
constexpr int kRowMirror = 0x140;   // row_mirror
constexpr int kSwizzleXor16 = 0x401F;  // ds_swizzle bit mode: and 0x1f, xor 0x10
}  // namespace dpp

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), kCtrl, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t swz16_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), dpp::kSwizzleXor16));
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return uint32_t(__builtin_amdgcn_readlane(int(v), lane));
}

// The value of lane (this lane's partner) for each step, as a float or
// double.
template <int kStep>
__device__ __forceinline__ float partner(float v) {
  const uint32_t b = __float_as_uint(v);
  if constexpr (kStep == 0) return __uint_as_float(dpp_u32<dpp::kQuadSwap1>(b));
  if constexpr (kStep == 1) return __uint_as_float(dpp_u32<dpp::kQuadSwap2>(b));
  if constexpr (kStep == 2) return __uint_as_float(dpp_u32<dpp::kHalfMirror>(b));
  if constexpr (kStep == 3) return __uint_as_float(dpp_u32<dpp::kRowMirror>(b));
  return __uint_as_float(swz16_u32(b));
}

template <int kStep>
__device__ __forceinline__ double partner(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  uint32_t lo = uint32_t(b), hi = uint32_t(b >> 32);
  if constexpr (kStep == 0) {
    lo = dpp_u32<dpp::kQuadSwap1>(lo);
    hi = dpp_u32<dpp::kQuadSwap1>(hi);
  } else if constexpr (kStep == 1) {
    lo = dpp_u32<dpp::kQuadSwap2>(lo);
    hi = dpp_u32<dpp::kQuadSwap2>(hi);
  } else if constexpr (kStep == 2) {
    lo = dpp_u32<dpp::kHalfMirror>(lo);
    hi = dpp_u32<dpp::kHalfMirror>(hi);
  } else if constexpr (kStep == 3) {
    lo = dpp_u32<dpp::kRowMirror>(lo);
    hi = dpp_u32<dpp::kRowMirror>(hi);
  } else {
    lo = swz16_u32(lo);
    hi = swz16_u32(hi);
  }
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __uint_as_float(lane_u32(__float_as_uint(v), lane));
}

__device__ __forceinline__ double lane_value(double v, int lane) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint64_t r = (uint64_t(lane_u32(uint32_t(b >> 32), lane)) << 32) |
                     lane_u32(uint32_t(b), lane);
  return __longlong_as_double((long long)r);
}

template <class T>
__device__ __forceinline__ T wsum(T v) {
  v += partner<0>(v);
  v += partner<1>(v);
  v += partner<2>(v);
  v += partner<3>(v);
  v += partner<4>(v);
  return lane_value(v, 0) + lane_value(v, 32);
}

__device__ __forceinline__ float wmax(float v) {
  v = fmaxf(v, partner<0>(v));
  v = fmaxf(v, partner<1>(v));
  v = fmaxf(v, partner<2>(v));
  v = fmaxf(v, partner<3>(v));
  v = fmaxf(v, partner<4>(v));
  return fmaxf(lane_value(v, 0), lane_value(v, 32));
}

template <int kStep>
__device__ __forceinline__ int partner(int v) {
  const uint32_t b = uint32_t(v);
  if constexpr (kStep == 0) return int(dpp_u32<dpp::kQuadSwap1>(b));
  if constexpr (kStep == 1) return int(dpp_u32<dpp::kQuadSwap2>(b));
  if constexpr (kStep == 2) return int(dpp_u32<dpp::kHalfMirror>(b));
  if constexpr (kStep == 3) return int(dpp_u32<dpp::kRowMirror>(b));
  return int(swz16_u32(b));
}

__device__ __forceinline__ int wmin(int v) {
  v = min(v, partner<0>(v));
  v = min(v, partner<1>(v));
  v = min(v, partner<2>(v));
  v = min(v, partner<3>(v));
  v = min(v, partner<4>(v));
  return min(int(lane_u32(uint32_t(v), 0)), int(lane_u32(uint32_t(v), 32)));
}

template <int kStep>
__device__ __forceinline__ ArgMax partner(const ArgMax& a) {
  ArgMax b;
  b.v = partner<kStep>(a.v);
  const uint32_t iu = uint32_t(a.i), nu = uint32_t(a.nan);
  if constexpr (kStep == 0) {
    b.i = int32_t(dpp_u32<dpp::kQuadSwap1>(iu));
    b.nan = int32_t(dpp_u32<dpp::kQuadSwap1>(nu));
  } else if constexpr (kStep == 1) {
    b.i = int32_t(dpp_u32<dpp::kQuadSwap2>(iu));
    b.nan = int32_t(dpp_u32<dpp::kQuadSwap2>(nu));
  } else if constexpr (kStep == 2) {
    b.i = int32_t(dpp_u32<dpp::kHalfMirror>(iu));
    b.nan = int32_t(dpp_u32<dpp::kHalfMirror>(nu));
  } else if constexpr (kStep == 3) {
    b.i = int32_t(dpp_u32<dpp::kRowMirror>(iu));
    b.nan = int32_t(dpp_u32<dpp::kRowMirror>(nu));
  } else {
    b.i = int32_t(swz16_u32(iu));
    b.nan = int32_t(swz16_u32(nu));
  }
  return b;
}

// Argmax over the wave: largest value, lowest index among equal values, NaN
// flag or-ed (argmax_combine is symmetric, so every lane ends equal).
__device__ __forceinline__ ArgMax wargmax(ArgMax a) {
  a = argmax_combine(a, partner<0>(a));
  a = argmax_combine(a, partner<1>(a));
  a = argmax_combine(a, partner<2>(a));
  a = argmax_combine(a, partner<3>(a));
  a = argmax_combine(a, partner<4>(a));
  ArgMax lo, hi;
  lo.v = lane_value(a.v, 0);
  lo.i = int32_t(lane_u32(uint32_t(a.i), 0));
  lo.nan = int32_t(lane_u32(uint32_t(a.nan), 0));
  hi.v = lane_value(a.v, 32);
  hi.i = int32_t(lane_u32(uint32_t(a.i), 32));
  hi.nan = int32_t(lane_u32(uint32_t(a.nan), 32));
  return argmax_combine(lo, hi);
}

}  // namespace lvtv
