// dspark_schedule: confidence-scheduled verify lengths on gfx950, one
// workgroup.
//
// Definition (page title, section): "Reading Qwen Bebop and DeepSeek
// DSpark", "DSpark's second piece: confidence-scheduled verify length".
// Request r has per-position confidences c_{r,j} (the chance that draft token
// j survives once every earlier one did; the pages' soft label is
// 1 - d_TV, the verify step's alpha). Its prefix survivals are
// a_{r,j} = prod_{i<=j} c_{r,i}. Verifying l_r tokens of every request feeds
// B = sum_r (1 + l_r) tokens to the target model and yields
// tau = sum_r (1 + sum_{j<=l_r} a_{r,j}) tokens in expectation; the lengths
// maximise Theta = tau SPS(B), SPS(B) being the engine's decode steps per
// second at batch size B.
//
// a_{r,j} does not grow with j, so for a fixed B the best lengths take the
// B - R largest survivals, which form a prefix of every request. The kernel:
//   1. survivals in binary32, left to right (confidences clamped to [0, 1],
//      NaN read as 0), as 64-bit keys: the complement of the value's bits
//      above the flat index r L + j, so that one ascending sort orders them
//      largest first and equal values by index;
//   2. a bitonic sort of the keys in LDS;
//   3. an fp64 block scan of the sorted survivals; Theta(B) for every B from
//      R to R (1 + L), the largest kept (the smallest B among equals; a NaN
//      Theta never wins);
//   4. l_r = one past the last position of request r among the taken keys.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "../../include/lvtv.h"

namespace lvtv {
namespace sched {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxItems = LVTV_SCHED_MAX_ITEMS;  // R L
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;

struct Shared {
  uint64_t key[kMaxItems];
  int32_t len[kMaxItems];  // per request (R <= R L)
  double wsum[kWaves];
  double wbest[kWaves];
  int32_t wt[kWaves];
  int32_t best_t;
  double best_theta;
};

__device__ __forceinline__ float clamp_conf(float c) {
  // NaN and non-positive values read as +0, values above 1 as 1
  return c > 0.f ? fminf(c, 1.f) : 0.f;
}

__device__ __forceinline__ float key_value(uint64_t key) {
  return __uint_as_float(0xffffffffu - uint32_t(key >> 32));
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(const float* conf, const float* sps,
                                                            int R, int L, int32_t* verify_len,
                                                            double* best) {
  __shared__ Shared sh;
  const int n = R * L;
  int P = 1;
  while (P < n) P <<= 1;
  const int tid = threadIdx.x;

  // 1. survivals as sort keys
  for (int r = tid; r < R; r += kThreads) {
    float run = 1.f;
    for (int j = 0; j < L; ++j) {
      run = __fmul_rn(run, clamp_conf(conf[size_t(r) * L + j]));
      const uint32_t idx = uint32_t(r * L + j);
      sh.key[idx] = (uint64_t(0xffffffffu - __float_as_uint(run)) << 32) | idx;
    }
    sh.len[r] = 0;
  }
  for (int i = n + tid; i < P; i += kThreads) sh.key[i] = ~uint64_t(0);
  __syncthreads();

  // 2. bitonic sort, ascending
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = sh.key[i], b = sh.key[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            sh.key[i] = b;
            sh.key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  // 3. scan of the sorted survivals: thread t owns items [t q, t q + q)
  const int q = (n + kThreads - 1) / kThreads;
  const int i0 = tid * q;
  double local = 0.0;
  for (int i = i0; i < min(i0 + q, n); ++i) local += (double)key_value(sh.key[i]);
  // exclusive prefix of the per-thread totals: within the wave, then waves
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  double inc = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  if (lane == kWave - 1) sh.wsum[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += sh.wsum[w];
  double s = base + inc - local;  // survivals taken before item i0
  // Theta for B = R + t, t = i + 1 over the thread's items (and t = 0)
  double bv = -INFINITY;
  int bt = INT_MAX;
  if (tid == 0) {
    const double th = double(R) * (double)sps[R];
    if (th == th) {
      bv = th;
      bt = 0;
    }
  }
  for (int i = i0; i < min(i0 + q, n); ++i) {
    s += (double)key_value(sh.key[i]);
    const double th = (double(R) + s) * (double)sps[R + i + 1];
    if (th > bv) {  // a NaN never wins; the first (smallest t) among equals stays
      bv = th;
      bt = i + 1;
    }
  }
  // block argmax: largest Theta, smallest t among equals
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double ov = __shfl_xor(bv, o, kWave);
    const int ot = __shfl_xor(bt, o, kWave);
    if (ov > bv || (ov == bv && ot < bt)) {
      bv = ov;
      bt = ot;
    }
  }
  if (lane == 0) {
    sh.wbest[wave] = bv;
    sh.wt[wave] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    double v = sh.wbest[0];
    int t = sh.wt[0];
    for (int w = 1; w < kWaves; ++w)
      if (sh.wbest[w] > v || (sh.wbest[w] == v && sh.wt[w] < t)) {
        v = sh.wbest[w];
        t = sh.wt[w];
      }
    if (t == INT_MAX) t = 0;  // every Theta was NaN: verify nothing
    sh.best_t = t;
    sh.best_theta = v;
  }
  __syncthreads();

  // 4. lengths
  const int t = sh.best_t;
  for (int i = tid; i < t; i += kThreads) {
    const uint32_t idx = uint32_t(sh.key[i]);
    const int r = int(idx) / L, j = int(idx) - r * L;
    atomicMax(&sh.len[r], j + 1);
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) verify_len[r] = sh.len[r];
  if (tid == 0) {
    best[0] = sh.best_theta;
    best[1] = double(R + t);
  }
}

}  // namespace
}  // namespace sched
}  // namespace lvtv

extern "C" int dspark_schedule(const float* confidence, const float* sps, int32_t R, int32_t L,
                               int32_t* verify_len, double* best, void* stream) {
  if (R < 1 || L < 1 || int64_t(R) * L > LVTV_SCHED_MAX_ITEMS) return LVTV_ERR_SHAPE;
  if (!confidence || !sps || !verify_len || !best) return LVTV_ERR_NULL;
  hipLaunchKernelGGL(lvtv::sched::schedule_kernel, dim3(1), dim3(lvtv::sched::kThreads), 0,
                     static_cast<hipStream_t>(stream), confidence, sps, R, L, verify_len, best);
  return hipGetLastError() == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}
