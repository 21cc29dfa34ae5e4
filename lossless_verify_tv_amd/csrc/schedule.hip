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
//      above the flat index r L + j, so that ascending order is largest
//      first and equal values by index; a request's keys, survivals that
//      never grow, form an ascending run already;
//   2. a merge sort that starts from those R runs: ceil(log2 R) rounds
//      between two LDS buffers, each thread placing E consecutive outputs
//      of a round after one binary search for where they start;
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
  uint64_t key[kMaxItems];  // survival keys, then the merge rounds' buffers
  union {
    uint64_t other[kMaxItems];  // the second merge buffer
    struct {
      float conf[kMaxItems];    // confidences (before the sort)
      int32_t len[kMaxItems];   // lengths per request (R <= R L; after the sort)
    } io;
  } u;
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

// Merges the n keys of sh.key, ascending runs of w keys each (the last one
// possibly shorter), pairwise until one run holds them all; keys are
// distinct. Thread t writes outputs [t E, t E + E) of a round: a binary
// search finds how many of the pair's first run precede its first output,
// then it merges on from there (starting again where the next pair begins).
// Returns the buffer holding the result.
template <int E>
__device__ __forceinline__ const uint64_t* merge_runs(Shared& sh, int n, int w) {
  const int o0 = threadIdx.x * E;
  uint64_t* src = sh.key;
  uint64_t* dst = sh.u.other;
  for (; w < n; w *= 2) {
    if (o0 < n) {
      int a0 = o0 - o0 % (2 * w);
      int a1 = min(a0 + w, n), b1 = min(a0 + 2 * w, n);
      const int k = o0 - a0;
      // smallest i with A[i] > B[k - 1 - i]: the first k outputs hold i of A
      int lo = max(0, k - (b1 - a1)), hi = min(k, a1 - a0);
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (src[a0 + mid] < src[a1 + k - 1 - mid])
          lo = mid + 1;
        else
          hi = mid;
      }
      int i = a0 + lo, j = a1 + k - lo;  // next unmerged key of each run
      uint64_t va = i < a1 ? src[i] : ~uint64_t(0);
      uint64_t vb = j < b1 ? src[j] : ~uint64_t(0);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int o = o0 + e;
        if (o >= n) break;
        if (o == b1) {  // the next pair of runs starts here
          a0 = o;
          a1 = min(a0 + w, n);
          b1 = min(a0 + 2 * w, n);
          i = a0;
          j = a1;
          va = src[i];
          vb = j < b1 ? src[j] : ~uint64_t(0);
        }
        const bool ta = va < vb;
        dst[o] = ta ? va : vb;
        i += ta;
        j += !ta;
        const int p = ta ? i : j;
        const uint64_t nv = p < (ta ? a1 : b1) ? src[p] : ~uint64_t(0);
        va = ta ? nv : va;
        vb = ta ? vb : nv;
      }
    }
    __syncthreads();
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  return src;
}

template <int E>
__device__ __forceinline__ void schedule_body(const float* conf, const float* sps, int R, int L,
                                              int32_t* verify_len, double* best, Shared& sh) {
  const int n = R * L;
  const int tid = threadIdx.x;
  // the throughputs this thread's sorted items price (B = R + i + 1), loaded
  // now so their latency hides behind the sort
  float my_sps[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    my_sps[e] = i < n ? sps[R + i + 1] : 0.f;
  }
  const float sps0 = sps[R];

  // 1. confidences into LDS (coalesced), survivals as sort keys: request
  //    r's keys form the ascending run [r L, r L + L)
  for (int i = tid; i < n; i += kThreads) sh.u.io.conf[i] = conf[i];
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) {
    float run = 1.f;
    int j = 0;
    // 8 confidences read ahead of their products, so that a long request
    // waits on LDS once per 8 positions
    for (; j + 8 <= L; j += 8) {
      float c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) c[q] = sh.u.io.conf[r * L + j + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        run = __fmul_rn(run, clamp_conf(c[q]));
        const uint32_t idx = uint32_t(r * L + j + q);
        sh.key[idx] = (uint64_t(0xffffffffu - __float_as_uint(run)) << 32) | idx;
      }
    }
    for (; j < L; ++j) {
      run = __fmul_rn(run, clamp_conf(sh.u.io.conf[r * L + j]));
      const uint32_t idx = uint32_t(r * L + j);
      sh.key[idx] = (uint64_t(0xffffffffu - __float_as_uint(run)) << 32) | idx;
    }
  }
  __syncthreads();

  // 2. sort, ascending: the largest survivals first, equal ones by index;
  //    thread t then takes sorted items [t E, t E + E)
  const uint64_t* sorted = merge_runs<E>(sh, n, L);
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    x[e] = i < n ? sorted[i] : ~uint64_t(0);
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) sh.u.io.len[r] = 0;

  // 3. scan of the sorted survivals: thread t owns items [t E, t E + E)
  double local = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (tid * E + e < n) local += (double)key_value(x[e]);
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
  double s = base + inc - local;  // survivals taken before item t E
  // Theta for B = R + t, t = i + 1 over the thread's items (and t = 0)
  double bv = -INFINITY;
  int bt = INT_MAX;
  if (tid == 0) {
    const double th = double(R) * (double)sps0;
    if (th == th) {
      bv = th;
      bt = 0;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    if (i < n) {
      s += (double)key_value(x[e]);
      const double th = (double(R) + s) * (double)my_sps[e];
      if (th > bv) {  // a NaN never wins; the first (smallest t) among equals stays
        bv = th;
        bt = i + 1;
      }
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

  // 4. lengths: one past the last position of each request among the taken
  const int t = sh.best_t;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    if (i < t) {
      const uint32_t idx = uint32_t(x[e]);
      const int r = int(idx) / L, j = int(idx) - r * L;
      atomicMax(&sh.u.io.len[r], j + 1);
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) verify_len[r] = sh.u.io.len[r];
  if (tid == 0) {
    best[0] = sh.best_theta;
    best[1] = double(R + t);
  }
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(const float* conf, const float* sps,
                                                            int R, int L, int32_t* verify_len,
                                                            double* best) {
  __shared__ Shared sh;
  const int n = R * L;
  if (n <= kThreads)
    schedule_body<1>(conf, sps, R, L, verify_len, best, sh);
  else if (n <= 2 * kThreads)
    schedule_body<2>(conf, sps, R, L, verify_len, best, sh);
  else if (n <= 4 * kThreads)
    schedule_body<4>(conf, sps, R, L, verify_len, best, sh);
  else
    schedule_body<8>(conf, sps, R, L, verify_len, best, sh);
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
