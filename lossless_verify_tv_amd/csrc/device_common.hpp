// Device helpers shared by the verify and loss kernels (gfx950, wave64).
//
// Reductions are fixed-order trees (butterfly inside a wave, then LDS in
// wave order), never atomics, so every result is bit-reproducible run to
// run. Per-thread runs are summed in fp32 over at most eight terms and then
// carried in fp64, so sums over 1.5e5 terms keep ~1e-9 relative error.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace lvtv {

constexpr int kBlock = 256;            // threads per workgroup (4 waves)
constexpr int kWave = 64;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kVec = 8;                // elements per thread per step
constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- loads

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Eight consecutive elements [e, e+8) of one row, as fp32. Elements at or
// beyond V read as -inf (they then carry zero probability and never win an
// argmax over a real element, which has a lower index). `vec_ok` says the
// row base is 16-byte aligned and V is a multiple of 8, so the whole group
// can be fetched with 16-byte loads.
template <int kDtype>
__device__ __forceinline__ void load8(const void* row, int64_t e, int64_t V,
                                      bool vec_ok, float (&x)[kVec]) {
  if (vec_ok && e + kVec <= V) {
    if constexpr (kDtype == 1) {
      const uint4 w = *reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(row) + e);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(u[i] << 16);
        x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + e);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + e + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int64_t idx = e + i;
      if (idx < V) {
        if constexpr (kDtype == 1)
          x[i] = bf16_bits_to_f32(static_cast<const uint16_t*>(row)[idx]);
        else
          x[i] = static_cast<const float*>(row)[idx];
      } else {
        x[i] = -INFINITY;
      }
    }
  }
}

// One element of a row as fp32.
template <int kDtype>
__device__ __forceinline__ float load1(const void* row, int64_t idx) {
  if constexpr (kDtype == 1)
    return bf16_bits_to_f32(static_cast<const uint16_t*>(row)[idx]);
  else
    return static_cast<const float*>(row)[idx];
}

// Canonical scaled logit fl32(x * inv_t): a correctly rounded binary32
// product that the compiler may not fuse into a later operation.
__device__ __forceinline__ float scale_logit(float x, float inv_t, bool unit) {
  return unit ? x : __fmul_rn(x, inv_t);
}

// exp(s - m) for fp32 s, m, with the m * log2(e) product hoisted per row:
// v_exp_f32(fma(s, log2e, -m*log2e)). The rounding of m*log2(e) is a common
// factor of the whole row and cancels when the row is normalised.
__device__ __forceinline__ float exp_shifted(float s, float neg_m_log2e) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(s, kLog2e, neg_m_log2e));
}

// ---------------------------------------------------------------- reductions

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide sum in fixed order; every thread gets the result. `scratch`
// holds kWavesPerBlock entries.
template <class T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[wave] = v;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) r += scratch[w];
  return r;
}

__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) r = fmaxf(r, scratch[w]);
  return r;
}

// Argmax with the lowest index among equal values; NaN values are left out
// of the comparison and reported through `nan`.
struct ArgMax {
  float v;
  int32_t i;
  int32_t nan;
};

__device__ __forceinline__ ArgMax argmax_combine(ArgMax a, ArgMax b) {
  ArgMax r;
  r.nan = a.nan | b.nan;
  const bool take_b = (b.v > a.v) || (b.v == a.v && b.i < a.i);
  r.v = take_b ? b.v : a.v;
  r.i = take_b ? b.i : a.i;
  return r;
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    ArgMax b;
    b.v = __shfl_xor(a.v, o, kWave);
    b.i = __shfl_xor(a.i, o, kWave);
    b.nan = __shfl_xor(a.nan, o, kWave);
    a = argmax_combine(a, b);
  }
  return a;
}

__device__ __forceinline__ ArgMax block_argmax(ArgMax a, ArgMax* scratch) {
  a = wave_argmax(a);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[wave] = a;
  __syncthreads();
  ArgMax r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) r = argmax_combine(r, scratch[w]);
  return r;
}

// Row statistics of one slice for the softmax: max m and sum of exp(s - m).
// A slice that is entirely -inf keeps m = -inf and a sum of 0 (or NaN if it
// held a NaN), so that combining slices stays exact.
struct SliceStat {
  double m;
  double l;
};

// Combine per-slice (m, l) into the row's (M, L): M = max m_s,
// L = sum_s l_s exp((m_s - M) scale), in fp64, in slice order (scale is the
// natural-log factor of the exponent: 1 for exp(x - m)). Every thread of the
// block gets the same values.
__device__ __forceinline__ void combine_row_stats(const SliceStat* parts, int n,
                                                  double* scratch_d,
                                                  float* scratch_f, double& M,
                                                  double& L, double scale) {
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < n; s += kBlock) mloc = fmaxf(mloc, (float)parts[s].m);
  const float mf = block_max(mloc, scratch_f);
  M = (double)mf;
  double lloc = 0.0;
  for (int s = threadIdx.x; s < n; s += kBlock) {
    const double ms = parts[s].m;
    // slices that are entirely -inf weigh 0 (their l is 0, or NaN if a NaN
    // was present, which must propagate)
    const double wgt = (ms == -INFINITY) ? 0.0 : exp((ms - M) * scale);
    lloc += (ms == -INFINITY) ? parts[s].l * 0.0 : parts[s].l * wgt;
  }
  L = block_sum(lloc, scratch_d);
}

}  // namespace lvtv
