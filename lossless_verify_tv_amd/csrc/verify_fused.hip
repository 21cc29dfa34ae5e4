// spec_verify, single-read kernel (one launch) for gfx950.
//
// Each workgroup owns one slice of 8192 tokens of one (request b, position
// k) pair of rows: target row k and, for k < K_b, draft row k (k = K_b is
// the bonus row, target only). It streams the slice from HBM once into
// registers, then:
//   1. computes the slice's softmax statistics for both rows (max, sum of
//      exp), publishes them as tagged words and collects those of the other
//      slices of the same rows (bounded wait, see fused_common.hpp);
//   2. with the row statistics, turns its register-held exponentials into
//      p and q and accumulates alpha = sum min(p, q) over the slice and, per
//      2048-token chunk (one wave's contiguous span), the residual mass
//      sum max(0, p - q), or for the bonus row the mass of p;
//   3. counts itself in at its request; the last of the request's
//      workgroups finalises it: status checks, alpha_k, the accept scan with
//      Philox uniforms, and the inverse-CDF draw (chunk from the chunk
//      masses, token from an fp64 recomputation inside the chunk).
// Greedy requests (T = 0) take the argmax of the raw logits instead (one
// pass, no exchange).
//
// Cites (page title, section): "Reading Qwen Bebop and DeepSeek DSpark",
// "Formulas" (alpha(y) = min(1, p/q); alpha_RS = sum min(p, q) = 1 - d_TV);
// "Speculative Decoding and MTP" survey, section 2 (ordered acceptance, bonus
// distribution), section 3 (residual max(0, p - q)/Z), section 4 (same
// temperature for p and q; greedy argmax rule), section 21 (acceptance and
// residual sampling fused on the GPU, no per-cycle CPU sync).
//
// Arithmetic: scaled logit s = fl32(x * fl32(1/T)) (x itself at T = 1);
// exponentials are taken base 2 against a per-slice reference
// R = fl32(m * L2E), m the slice max of s, L2E = fl32(log2 e):
// e = 2^fl32(s * L2E - R). A row's statistics are (R_max, L = sum over
// slices l_s 2^(R_s - R_max)) in fp64, so p(v) = 2^(s_v L2E - R_max) / L.
// The finalize step evaluates that formula in fp64 for the accept ratios and
// inside the chosen chunk.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "../../include/lvtv.h"
#include "device_common.hpp"
#include "fused_common.hpp"
#include "philox.hpp"
#include "verify_fused.hpp"

namespace lvtv {
namespace vf {
namespace {

constexpr int kSteps = 4;                          // 16-byte groups per thread per row
constexpr int kSlice = kBlock * kVec * kSteps;     // 8192 tokens per workgroup
constexpr int kSpan = kWave * kVec * kSteps;       // 2048 tokens per wave = one chunk
constexpr int kStepStride = kWave * kVec;          // 512
constexpr int kRowsMax = 2 * LVTV_MAX_K + 1;
constexpr float kL2E = 1.44269504088896340736f;

struct Args {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* kreq;
  const float* temp;
  const uint64_t* seed;
  int B, Kmax, V;
  int spin_limit;
  int32_t* acc_len;
  int32_t* out_tokens;
  float* alpha;
  int32_t* status;
  int S, NC;
  FusedCtl* ctl;
  uint32_t* req;
  uint64_t* stat;    // [B][Kmax+1][S][4]: R_t, l_t, R_d, l_d (greedy: v_t, i_t, v_d, i_d)
  uint64_t* apart;   // [B][Kmax][S]: slice alpha
  uint64_t* chunk;   // [B][Kmax+1][NC]: chunk masses (residual, or p for the bonus row)
};

__device__ __forceinline__ bool temperature_ok(float t) { return (t >= 0.f) && !isinf(t); }

template <int kDtype>
__device__ __forceinline__ const void* row_ptr(const Args& a, int b, bool target, int k) {
  constexpr int kSize = kDtype == 1 ? 2 : 4;
  const int64_t row = target ? (int64_t(b) * (a.Kmax + 1) + k) : (int64_t(b) * a.Kmax + k);
  return static_cast<const char*>(target ? a.target : a.draft) + row * int64_t(a.V) * kSize;
}

__device__ __forceinline__ size_t stat_idx(const Args& a, int b, int k, int s) {
  return ((size_t(b) * (a.Kmax + 1) + k) * a.S + s) * 4;
}
__device__ __forceinline__ size_t apart_idx(const Args& a, int b, int k, int s) {
  return (size_t(b) * a.Kmax + k) * a.S + s;
}
__device__ __forceinline__ size_t chunk_idx(const Args& a, int b, int k, int c) {
  return (size_t(b) * (a.Kmax + 1) + k) * a.NC + c;
}

// ------------------------------------------------------------------ slices

// Token index of thread-element (step i, element j) in slice s.
__device__ __forceinline__ int64_t elem_base(int s) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  return int64_t(s) * kSlice + wave * kSpan + lane * kVec;
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void load_slice(const void* row, int64_t V, int s,
                                           float (&x)[kSteps][kVec]) {
  const int64_t base = elem_base(s);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) load8_nt<kDtype, kVecOk>(row, base + i * kStepStride, V, x[i]);
}

// Block reduction of two floats at once (max or sum), fixed order.
struct Red2 {
  float v[kWavesPerBlock][2];
};

__device__ __forceinline__ void block_max2(float& a, float& b, Red2& sh) {
  a = wave_max(a);
  b = wave_max(b);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.v[threadIdx.x / kWave][0] = a;
    sh.v[threadIdx.x / kWave][1] = b;
  }
  __syncthreads();
  a = sh.v[0][0];
  b = sh.v[0][1];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) {
    a = fmaxf(a, sh.v[w][0]);
    b = fmaxf(b, sh.v[w][1]);
  }
}

__device__ __forceinline__ void block_sum2(float& a, float& b, Red2& sh) {
  a = wave_sum(a);
  b = wave_sum(b);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.v[threadIdx.x / kWave][0] = a;
    sh.v[threadIdx.x / kWave][1] = b;
  }
  __syncthreads();
  a = sh.v[0][0];
  b = sh.v[0][1];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) {
    a += sh.v[w][0];
    b += sh.v[w][1];
  }
}

struct SliceStats {
  float R;     // log2-domain reference fl32(m * L2E) (-inf for an all -inf slice)
  float l;     // sum of 2^(s L2E - R) over the slice
  float wsum;  // this wave's part of l (its chunk)
};

// In place: x <- scaled logits -> exponentials; returns the slice statistics
// of the target row and, with kTwo, of the draft row. Every thread of the
// block must call it.
template <bool kTwo>
__device__ __forceinline__ void slice_stats(float (&xt)[kSteps][kVec], float (&xd)[kSteps][kVec],
                                            float inv_t, bool unit, Red2& sh, SliceStats& st,
                                            SliceStats& sd) {
  float mt = -INFINITY, md = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      xt[i][j] = scale_logit(xt[i][j], inv_t, unit);
      mt = fmaxf(mt, xt[i][j]);
      if constexpr (kTwo) {
        xd[i][j] = scale_logit(xd[i][j], inv_t, unit);
        md = fmaxf(md, xd[i][j]);
      }
    }
  block_max2(mt, md, sh);
  const float rt = (mt == -INFINITY) ? -INFINITY : mt * kL2E;
  const float rd = (md == -INFINITY) ? -INFINITY : md * kL2E;
  const float nt = (mt == -INFINITY) ? 0.f : -rt;
  const float nd = (md == -INFINITY) ? 0.f : -rd;
  float lt = 0.f, ld = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      xt[i][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[i][j], kL2E, nt));
      lt += xt[i][j];
      if constexpr (kTwo) {
        xd[i][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[i][j], kL2E, nd));
        ld += xd[i][j];
      }
    }
  const float wt = wave_sum(lt), wd = wave_sum(ld);
  float bt = lt, bd = ld;
  block_sum2(bt, bd, sh);
  st = SliceStats{rt, bt, wt};
  sd = SliceStats{rd, bd, wd};
}

// Row statistics from the per-slice (R, l) words (4 words per slice, R at
// offset offR, l at offL), computed by one wave with one slice per lane:
// R_max = max R_s and L = sum_s l_s 2^(R_s - R_max) in fp64 (fixed
// butterfly order). Slices that are entirely -inf weigh 0 (their l is 0, or
// NaN when a NaN was present, which must propagate). All lanes of the
// calling wave get the result.
__device__ __forceinline__ void combine_row_wave(const uint32_t* words, int S, int offR, int offL,
                                                 float& Rmax, double& L) {
  const int lane = threadIdx.x & (kWave - 1);
  const float R = lane < S ? __uint_as_float(words[4 * lane + offR]) : -INFINITY;
  const float l = lane < S ? __uint_as_float(words[4 * lane + offL]) : 0.f;
  const float m = wave_max(R);
  const double w = (R == -INFINITY) ? (double)l * 0.0 : (double)l * exp2((double)R - (double)m);
  L = wave_sum(w);
  Rmax = m;
}

// Pass 2 of a pair slice: alpha over the slice and the residual mass per
// wave chunk, from exponentials held in registers.
__device__ __forceinline__ void pair_overlap(const float (&et)[kSteps][kVec],
                                             const float (&ed)[kSteps][kVec], float at, float ad,
                                             float* red4, float& alpha_slice, float& chunk_mass) {
  float sa = 0.f, sr = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float p = et[i][j] * at;
      const float q = ed[i][j] * ad;
      const float mn = fminf(p, q);
      sa += mn;
      sr += p - mn;
    }
  chunk_mass = wave_sum(sr);
  alpha_slice = block_sum(sa, red4);
}

// Argmax of one slice of raw logits (lowest index among equal values; NaN
// flagged), one 8-token group at a time.
template <int kDtype, bool kVecOk>
__device__ __forceinline__ ArgMax slice_argmax(const void* row, int64_t V, int s, ArgMax* sh) {
  const int64_t base = elem_base(s);
  ArgMax best{-INFINITY, INT_MAX, 0};
#pragma unroll 1
  for (int i = 0; i < kSteps; ++i) {
    float x[kVec];
    load8_nt<kDtype, kVecOk>(row, base + i * kStepStride, V, x);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int64_t idx = base + i * kStepStride + j;
      if (idx < V) {
        const float v = x[j];
        if (isnan(v)) best.nan = 1;
        else if (v > best.v || (v == best.v && idx < best.i)) {
          best.v = v;
          best.i = int32_t(idx);
        }
      }
    }
  }
  return block_argmax(best, sh);
}

// Streaming forms of slice_stats / pair_overlap for the recompute path: the
// slice is re-read from HBM one 8-token group at a time (few registers),
// with the same per-thread accumulation order and the same reductions, so
// the results are bit-identical to the register-held path.
template <int kDtype, bool kVecOk, bool kTwo>
__device__ __forceinline__ void stream_stats(const void* trow, const void* drow, int64_t V, int s,
                                             float inv_t, bool unit, Red2& sh, SliceStats& st,
                                             SliceStats& sd) {
  const int64_t base = elem_base(s);
  float mt = -INFINITY, md = -INFINITY;
#pragma unroll 1
  for (int i = 0; i < kSteps; ++i) {
    float xt[kVec], xd[kVec];
    load8_nt<kDtype, kVecOk>(trow, base + i * kStepStride, V, xt);
    if constexpr (kTwo) load8_nt<kDtype, kVecOk>(drow, base + i * kStepStride, V, xd);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      mt = fmaxf(mt, scale_logit(xt[j], inv_t, unit));
      if constexpr (kTwo) md = fmaxf(md, scale_logit(xd[j], inv_t, unit));
    }
  }
  block_max2(mt, md, sh);
  const float rt = (mt == -INFINITY) ? -INFINITY : mt * kL2E;
  const float rd = (md == -INFINITY) ? -INFINITY : md * kL2E;
  const float nt = (mt == -INFINITY) ? 0.f : -rt;
  const float nd = (md == -INFINITY) ? 0.f : -rd;
  float lt = 0.f, ld = 0.f;
#pragma unroll 1
  for (int i = 0; i < kSteps; ++i) {
    float xt[kVec], xd[kVec];
    load8_nt<kDtype, kVecOk>(trow, base + i * kStepStride, V, xt);
    if constexpr (kTwo) load8_nt<kDtype, kVecOk>(drow, base + i * kStepStride, V, xd);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      lt += __builtin_amdgcn_exp2f(__builtin_fmaf(scale_logit(xt[j], inv_t, unit), kL2E, nt));
      if constexpr (kTwo)
        ld += __builtin_amdgcn_exp2f(__builtin_fmaf(scale_logit(xd[j], inv_t, unit), kL2E, nd));
    }
  }
  const float wt = wave_sum(lt), wd = wave_sum(ld);
  float bt = lt, bd = ld;
  block_sum2(bt, bd, sh);
  st = SliceStats{rt, bt, wt};
  sd = SliceStats{rd, bd, wd};
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void stream_overlap(const void* trow, const void* drow, int64_t V, int s,
                                               float inv_t, bool unit, const SliceStats& st,
                                               const SliceStats& sd, float at, float ad,
                                               float* red4, float& alpha_slice,
                                               float& chunk_mass) {
  const int64_t base = elem_base(s);
  const float nt = (st.R == -INFINITY) ? 0.f : -st.R;
  const float nd = (sd.R == -INFINITY) ? 0.f : -sd.R;
  float sa = 0.f, sr = 0.f;
#pragma unroll 1
  for (int i = 0; i < kSteps; ++i) {
    float xt[kVec], xd[kVec];
    load8_nt<kDtype, kVecOk>(trow, base + i * kStepStride, V, xt);
    load8_nt<kDtype, kVecOk>(drow, base + i * kStepStride, V, xd);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(scale_logit(xt[j], inv_t, unit), kL2E, nt));
      const float ed = __builtin_amdgcn_exp2f(__builtin_fmaf(scale_logit(xd[j], inv_t, unit), kL2E, nd));
      const float p = et * at;
      const float q = ed * ad;
      const float mn = fminf(p, q);
      sa += mn;
      sr += p - mn;
    }
  }
  chunk_mass = wave_sum(sr);
  alpha_slice = block_sum(sa, red4);
}

// ------------------------------------------------------------------ shared memory

struct ItemShared {
  Red2 red;
  float red4[kWavesPerBlock];
  float cm4[kWavesPerBlock];
  ArgMax am[kWavesPerBlock];
  uint32_t words[4 * kMaxSlices];
  uint8_t have[4 * kMaxSlices];
  float at, ad;
  float Rt, Rd;
  double Lt, Ld;
  int last;
};

struct FinShared {
  Red2 red;
  double redd[kWavesPerBlock];
  float red4[kWavesPerBlock];
  int redi[kWavesPerBlock];
  ArgMax am[kWavesPerBlock];
  uint32_t words[4 * kMaxSlices * (LVTV_MAX_K + 1)];
  uint8_t have[4 * kMaxSlices * (LVTV_MAX_K + 1)];
  float R[kRowsMax];
  double L[kRowsMax];
  int32_t arg[kRowsMax];
  double alpha[LVTV_MAX_K];
  float cm[4 * kMaxSlices];
  float cm4[kWavesPerBlock];
  int status;
  int j;
  int pick;
  double before;
};

struct Shared {
  ItemShared it;
  FinShared fin;
};

// ------------------------------------------------------------------ recomputation

// The statistics words a (b, k, s) workgroup publishes, recomputed from the
// inputs (bit-identical to what it publishes).
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void recompute_stat_words(const Args& a, int b, int k, int s, int kb,
                                                     float T, uint32_t (&w)[4], Shared& sh) {
  const int64_t V = a.V;
  const bool pair = k < kb;
  if (T == 0.f) {
    const ArgMax at = slice_argmax<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, sh.it.am);
    ArgMax ad{-INFINITY, INT_MAX, 0};
    if (pair) ad = slice_argmax<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, sh.it.am);
    w[0] = __float_as_uint(at.nan ? NAN : at.v);
    w[1] = uint32_t(at.i);
    w[2] = __float_as_uint(ad.nan ? NAN : ad.v);
    w[3] = uint32_t(ad.i);
    return;
  }
  const float inv_t = __fdiv_rn(1.f, T);
  const bool unit = T == 1.f;
  SliceStats st, sd;
  if (pair)
    stream_stats<kDtype, kVecOk, true>(row_ptr<kDtype>(a, b, true, k),
                                       row_ptr<kDtype>(a, b, false, k), V, s, inv_t, unit,
                                       sh.it.red, st, sd);
  else
    stream_stats<kDtype, kVecOk, false>(row_ptr<kDtype>(a, b, true, k), nullptr, V, s, inv_t,
                                        unit, sh.it.red, st, sd);
  w[0] = __float_as_uint(st.R);
  w[1] = __float_as_uint(st.l);
  w[2] = __float_as_uint(pair ? sd.R : 0.f);
  w[3] = __float_as_uint(pair ? sd.l : 1.f);
}

// Slice alpha and the slice's four chunk masses of (b, k, s), recomputed
// from the inputs given the row statistics (cm4 in shared memory).
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void recompute_overlap(const Args& a, int b, int k, int s, int kb,
                                                  float T, float Rt, double Lt, float Rd,
                                                  double Ld, float& alpha_slice, float* cm4,
                                                  Shared& sh) {
  const int64_t V = a.V;
  const bool pair = k < kb;
  const float inv_t = __fdiv_rn(1.f, T);
  const bool unit = T == 1.f;
  const void* trow = row_ptr<kDtype>(a, b, true, k);
  SliceStats st, sd;
  float cmass;
  if (pair) {
    const void* drow = row_ptr<kDtype>(a, b, false, k);
    stream_stats<kDtype, kVecOk, true>(trow, drow, V, s, inv_t, unit, sh.it.red, st, sd);
    const float at = float(exp2((double)st.R - (double)Rt) / Lt);
    const float ad = float(exp2((double)sd.R - (double)Rd) / Ld);
    stream_overlap<kDtype, kVecOk>(trow, drow, V, s, inv_t, unit, st, sd, at, ad, sh.it.red4,
                                   alpha_slice, cmass);
  } else {
    stream_stats<kDtype, kVecOk, false>(trow, nullptr, V, s, inv_t, unit, sh.it.red, st, sd);
    const float at = float(exp2((double)st.R - (double)Rt) / Lt);
    alpha_slice = 0.f;
    cmass = st.wsum * at;
  }
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) cm4[threadIdx.x / kWave] = cmass;
  __syncthreads();
}

// ------------------------------------------------------------------ completion

__device__ __forceinline__ void complete_unit(const Args& a, uint32_t epoch) {
  const uint32_t old = __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (old == uint32_t(a.B) - 1) {
    __hip_atomic_store(&a.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctl->epoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void write_fault(const Args& a, int b, int status) {
  int32_t* out_tok = a.out_tokens + size_t(b) * (a.Kmax + 1);
  float* out_alpha = a.alpha + size_t(b) * a.Kmax;
  for (int k = threadIdx.x; k <= a.Kmax; k += kBlock) out_tok[k] = -1;
  for (int k = threadIdx.x; k < a.Kmax; k += kBlock) out_alpha[k] = 0.f;
  if (threadIdx.x == 0) {
    a.status[b] = status;
    a.acc_len[b] = -1;
  }
}

// ------------------------------------------------------------------ draw

// fp64 probability of token v of a row under (R_max, L), base-2 convention.
template <int kDtype>
__device__ __forceinline__ double prob64(const void* row, int64_t v, float inv_t, bool unit,
                                         float R, double L) {
  const float s = scale_logit(load1<kDtype>(row, v), inv_t, unit);
  return exp2((double)s * (double)kL2E - (double)R) / L;
}

__device__ __forceinline__ double block_exclusive_scan(double v, double* sh, double& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  __syncthreads();
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  double pre = 0.0;
  for (int w = 0; w < wave; ++w) pre += sh[w];
  total = 0.0;
  for (int w = 0; w < kWavesPerBlock; ++w) total += sh[w];
  return pre + inc - v;
}

__device__ __forceinline__ int block_min_i(int v, int* sh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = sh[0];
  for (int w = 1; w < kWavesPerBlock; ++w) r = min(r, sh[w]);
  return r;
}

// Weights of the draw inside chunk c: 8 consecutive tokens per thread.
template <int kDtype>
__device__ __forceinline__ void chunk_weights(const void* trow, const void* drow, int64_t V,
                                              int c, float inv_t, bool unit, float Rt, double Lt,
                                              float Rd, double Ld, bool residual,
                                              double (&w)[kVec], int64_t& v0) {
  v0 = int64_t(c) * kSpan + threadIdx.x * kVec;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int64_t v = v0 + i;
    double x = 0.0;
    if (v < V) {
      const double p = prob64<kDtype>(trow, v, inv_t, unit, Rt, Lt);
      x = residual ? fmax(0.0, p - prob64<kDtype>(drow, v, inv_t, unit, Rd, Ld)) : p;
    }
    w[i] = x;
  }
}

// Smallest token of chunk c whose cumulative weight exceeds `rem` (weights
// recomputed in fp64); falls back to the last positive-weight token of the
// chunk when rounding leaves `rem` at or above the chunk's fp64 total.
template <int kDtype>
__device__ __forceinline__ int search_chunk(const void* trow, const void* drow, int64_t V, int c, double rem,
                            float inv_t, bool unit, float Rt, double Lt, float Rd, double Ld,
                            bool residual, FinShared& sh) {
  double w[kVec];
  int64_t v0;
  chunk_weights<kDtype>(trow, drow, V, c, inv_t, unit, Rt, Lt, Rd, Ld, residual, w, v0);
  double mine = 0.0;
#pragma unroll
  for (int i = 0; i < kVec; ++i) mine += w[i];
  double total;
  const double exc = block_exclusive_scan(mine, sh.redd, total);
  int pick = INT_MAX, last = -1;
  double run = exc;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    run += w[i];
    if (w[i] > 0.0) {
      last = int(v0 + i);
      if (pick == INT_MAX && run > rem) pick = int(v0 + i);
    }
  }
  int v = block_min_i(pick, sh.redi);
  if (v == INT_MAX) {
    v = -block_min_i(last >= 0 ? -last : INT_MAX, sh.redi);
    if (v == -INT_MAX) v = int(int64_t(c) * kSpan);
  }
  return v;
}

// Inverse-CDF draw from the per-chunk masses `cm` (NC values in LDS).
template <int kDtype>
__device__ __forceinline__ int draw_from_masses(const float* cm, int NC, double u, const void* trow,
                                const void* drow, int64_t V, float inv_t, bool unit, float Rt,
                                double Lt, float Rd, double Ld, bool residual, FinShared& sh) {
  // thread 0 scans the chunk masses in fp64 (NC <= 4 * kMaxSlices)
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int c = 0; c < NC; ++c) total += (double)cm[c];
    const double target = u * total;
    double run = 0.0;
    int pick = -1;
    for (int c = 0; c < NC; ++c) {
      const double nxt = run + (double)cm[c];
      if (nxt > target && cm[c] > 0.f) {
        pick = c;
        break;
      }
      run = nxt;
    }
    if (pick < 0) {            // rounding: target at or past the last sum
      for (int c = NC - 1; c >= 0; --c)
        if (cm[c] > 0.f) {
          pick = c;
          break;
        }
      if (pick < 0) pick = NC - 1;
      run = INFINITY;           // makes the in-chunk search take its last token
      sh.before = INFINITY;
    } else {
      sh.before = target - run;
    }
    sh.pick = pick;
  }
  __syncthreads();
  const int c = sh.pick;
  const double rem = sh.before;
  return search_chunk<kDtype>(trow, drow, V, c, rem, inv_t, unit, Rt, Lt, Rd, Ld, residual, sh);
}

// Draw from p over the whole row when there are no chunk masses for it (a
// rejection where the residual is zero everywhere, p_j == q_j): masses of p
// per chunk in fp64, then the same search.
template <int kDtype>
__device__ __forceinline__ int draw_full_row(int NC, double u, const void* trow, int64_t V, float inv_t,
                             bool unit, float Rt, double Lt, FinShared& sh) {
  for (int c = 0; c < NC; ++c) {
    double w[kVec];
    int64_t v0;
    chunk_weights<kDtype>(trow, nullptr, V, c, inv_t, unit, Rt, Lt, 0.f, 1.0, false, w, v0);
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < kVec; ++i) mine += w[i];
    const double m = block_sum(mine, sh.redd);
    if (threadIdx.x == 0) sh.cm[c] = float(m);
    __syncthreads();
  }
  return draw_from_masses<kDtype>(sh.cm, NC, u, trow, nullptr, V, inv_t, unit, Rt, Lt, 0.f, 1.0,
                                  false, sh);
}

// ------------------------------------------------------------------ finalize

// True when the four words of slice entry e were all seen fresh.
__device__ __forceinline__ bool have4(const uint8_t* have, int e) {
  return have[4 * e] && have[4 * e + 1] && have[4 * e + 2] && have[4 * e + 3];
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void finalize(const Args& a, int b, int kb, float T, uint32_t epoch, Shared& shu) {
  FinShared& sh = shu.fin;
  const uint32_t tag = tag_from_epoch(epoch);
  const int S = a.S;
  const int Kmax = a.Kmax;
  const bool greedy = (T == 0.f);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);

  // draft tokens of this request
  int bad = 0;
  const int32_t* y = a.tokens + size_t(b) * Kmax;
  for (int k = threadIdx.x; k < kb; k += kBlock) bad |= (y[k] < 0 || y[k] >= a.V);
  const int status_tok = __syncthreads_or(bad) ? LVTV_STATUS_BAD_TOKEN : 0;

  // statistics words of every row: [k][s][4] for k = 0..kb
  const int nwords = (kb + 1) * S * 4;
  if (!poll_tagged(a.stat + stat_idx(a, b, 0, 0), nwords, tag, sh.words, sh.have,
                   a.spin_limit)) {
    for (int e = 0; e < (kb + 1) * S; ++e) {
      if (!have4(sh.have, e)) {
        uint32_t w[4];
        recompute_stat_words<kDtype, kVecOk>(a, b, e / S, e % S, kb, T, w, shu);
        __syncthreads();
        if (threadIdx.x == 0)
          for (int i = 0; i < 4; ++i) sh.words[4 * e + i] = w[i];
        __syncthreads();
      }
    }
  }

  // per-row statistics; rows r = k (target, k <= kb) and r = kb + 1 + k
  // (draft, k < kb); wave w takes rows r = w, w + 4, ...
  int fault = 0;
  for (int r = wave; r < 2 * kb + 1; r += kWavesPerBlock) {
    const bool tgt = r <= kb;
    const int k = tgt ? r : r - kb - 1;
    const int off = tgt ? 0 : 2;
    const uint32_t* words = sh.words + size_t(k) * S * 4;
    if (greedy) {
      ArgMax cand{-INFINITY, INT_MAX, 0};
      if (lane < S) {
        const float v = __uint_as_float(words[4 * lane + off]);
        if (isnan(v)) cand.nan = 1;
        else {
          cand.v = v;
          cand.i = int32_t(words[4 * lane + off + 1]);
        }
      }
      const ArgMax best = wave_argmax(cand);
      if (lane == 0) sh.arg[r] = best.i;
      fault |= best.nan || !isfinite(best.v);
    } else {
      float Rm;
      double L;
      combine_row_wave(words, S, off, off + 1, Rm, L);
      if (lane == 0) {
        sh.R[r] = Rm;
        sh.L[r] = L;
      }
      fault |= !isfinite(Rm) || !isfinite(L) || !(L > 0.0);
    }
  }
  fault = __syncthreads_or(fault);
  const int status = status_tok | (fault ? LVTV_STATUS_NONFINITE : 0);

  int32_t* out_tok = a.out_tokens + size_t(b) * (Kmax + 1);
  float* out_alpha = a.alpha + size_t(b) * Kmax;
  if (status) {
    write_fault(a, b, status);
    return;
  }

  if (greedy) {
    if (threadIdx.x == 0) {
      int j = kb;
      for (int k = 0; k < kb; ++k)
        if (y[k] != sh.arg[k]) {
          j = k;
          break;
        }
      for (int k = 0; k < Kmax; ++k)
        out_alpha[k] = (k < kb) ? (sh.arg[k] == sh.arg[kb + 1 + k] ? 1.f : 0.f) : 0.f;
      for (int k = 0; k <= Kmax; ++k) out_tok[k] = k < j ? y[k] : (k == j ? sh.arg[j] : -1);
      a.acc_len[b] = j;
      a.status[b] = 0;
    }
    return;
  }

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  const int64_t V = a.V;

  // slice alphas: [k][s] for k < kb
  if (kb > 0) {
    const int n = kb * S;
    if (!poll_tagged(a.apart + apart_idx(a, b, 0, 0), n, tag, sh.words, sh.have,
                     a.spin_limit)) {
      for (int e = 0; e < n; ++e)
        if (!sh.have[e]) {
          const int k = e / S;
          float al;
          recompute_overlap<kDtype, kVecOk>(a, b, k, e % S, kb, T, sh.R[k], sh.L[k],
                                            sh.R[kb + 1 + k], sh.L[kb + 1 + k], al, sh.cm4, shu);
          if (threadIdx.x == 0) sh.words[e] = __float_as_uint(al);
          __syncthreads();
        }
    }
    if (threadIdx.x == 0)
      for (int k = 0; k < kb; ++k) {
        double al = 0.0;
        for (int s = 0; s < S; ++s) al += (double)__uint_as_float(sh.words[k * S + s]);
        sh.alpha[k] = al;
      }
    __syncthreads();
  }

  // accept scan (thread 0, at most LVTV_MAX_K steps)
  if (threadIdx.x == 0) {
    for (int k = 0; k < Kmax; ++k) out_alpha[k] = k < kb ? float(sh.alpha[k]) : 0.f;
    int j = kb;
    for (int k = 0; k < kb; ++k) {
      double u, u2;
      verify_uniforms(a.seed[b], uint64_t(b), uint64_t(k), u, u2);
      const int yk = y[k];
      const double p = prob64<kDtype>(row_ptr<kDtype>(a, b, true, k), yk, inv_t, unit, sh.R[k],
                                      sh.L[k]);
      const double q = prob64<kDtype>(row_ptr<kDtype>(a, b, false, k), yk, inv_t, unit,
                                      sh.R[kb + 1 + k], sh.L[kb + 1 + k]);
      const bool ok = (q == 0.0) ? (p > 0.0) : (u < p / q);
      if (!ok) {
        j = k;
        break;
      }
    }
    sh.j = j;
  }
  __syncthreads();
  const int j = sh.j;

  // the draw at position j: chunk masses of row j
  double u_acc, u_draw;
  verify_uniforms(a.seed[b], uint64_t(b), uint64_t(j), u_acc, u_draw);
  const bool residual = j < kb;
  const void* trow = row_ptr<kDtype>(a, b, true, j);
  const void* drow = residual ? row_ptr<kDtype>(a, b, false, j) : nullptr;
  const float Rt = sh.R[j];
  const double Lt = sh.L[j];
  const float Rd = residual ? sh.R[kb + 1 + j] : 0.f;
  const double Ld = residual ? sh.L[kb + 1 + j] : 1.0;
  const int NC = a.NC;
  if (!poll_tagged(a.chunk + chunk_idx(a, b, j, 0), NC, tag, sh.words, sh.have, a.spin_limit)) {
    for (int s = 0; s < S; ++s)
      if (!have4(sh.have, s)) {
        float al;
        recompute_overlap<kDtype, kVecOk>(a, b, j, s, kb, T, Rt, Lt, Rd, Ld, al, sh.cm4, shu);
        if (threadIdx.x < kWavesPerBlock)
          sh.words[4 * s + threadIdx.x] = __float_as_uint(sh.cm4[threadIdx.x]);
        __syncthreads();
      }
  }
  for (int c = threadIdx.x; c < NC; c += kBlock) sh.cm[c] = __uint_as_float(sh.words[c]);
  __syncthreads();
  if (threadIdx.x == 0) {
    double z = 0.0;
    for (int c = 0; c < NC; ++c) z += (double)sh.cm[c];
    sh.before = z;
  }
  __syncthreads();
  int v;
  if (residual && !(sh.before > 0.0)) {
    __syncthreads();
    v = draw_full_row<kDtype>(NC, u_draw, trow, V, inv_t, unit, Rt, Lt, sh);
  } else {
    __syncthreads();
    v = draw_from_masses<kDtype>(sh.cm, NC, u_draw, trow, drow, V, inv_t, unit, Rt, Lt, Rd, Ld,
                                 residual, sh);
  }
  if (v < 0 || v >= a.V) v = a.V - 1;  // unreachable: the chosen chunk has positive mass
  if (threadIdx.x == 0) {
    for (int k = 0; k <= Kmax; ++k) out_tok[k] = k < j ? y[k] : (k == j ? v : -1);
    a.acc_len[b] = j;
    a.status[b] = 0;
  }
}

// ------------------------------------------------------------------ the kernel

template <int kDtype, bool kVecOk, bool kPair>
__device__ __forceinline__ void stochastic_item(const Args& a, int b, int k, int s, int kb, float T,
                                                uint32_t& epoch, Shared& shu) {
  ItemShared& sh = shu.it;
  const int S = a.S;
  const int64_t V = a.V;
  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  float xt[kSteps][kVec], xd[kSteps][kVec];
  load_slice<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, xt);
  if constexpr (kPair) load_slice<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, xd);
  epoch = read_epoch(a.ctl);
  const uint32_t tag = tag_from_epoch(epoch);
  SliceStats st, sd;
  slice_stats<kPair>(xt, xd, inv_t, unit, sh.red, st, sd);
  if (threadIdx.x == 0) {
    uint64_t* w = a.stat + stat_idx(a, b, k, s);
    tag_store(w + 0, tag, __float_as_uint(st.R));
    tag_store(w + 1, tag, __float_as_uint(st.l));
    tag_store(w + 2, tag, __float_as_uint(kPair ? sd.R : 0.f));
    tag_store(w + 3, tag, __float_as_uint(kPair ? sd.l : 1.f));
  }
  // collect the statistics of every slice of these rows
  const bool fresh = poll_tagged(a.stat + stat_idx(a, b, k, 0), 4 * S, tag, sh.words, sh.have,
                                 a.spin_limit);
  float alpha_slice = 0.f, cmass;
  if (fresh) {
    if (threadIdx.x < kWave) {
      float Rt, Rd = 0.f;
      double Lt, Ld = 1.0;
      combine_row_wave(sh.words, S, 0, 1, Rt, Lt);
      if constexpr (kPair) combine_row_wave(sh.words, S, 2, 3, Rd, Ld);
      if (threadIdx.x == 0) {
        sh.at = float(exp2((double)st.R - (double)Rt) / Lt);
        sh.ad = kPair ? float(exp2((double)sd.R - (double)Rd) / Ld) : 0.f;
      }
    }
    __syncthreads();
    if constexpr (kPair) {
      pair_overlap(xt, xd, sh.at, sh.ad, sh.red4, alpha_slice, cmass);
    } else {
      cmass = st.wsum * sh.at;
    }
  } else {
    // Rare: some slice's statistics did not arrive within the spin limit.
    // Recompute them, then redo this slice from the inputs too (its register
    // copy is dropped so the recomputation has the registers).
    for (int s2 = 0; s2 < S; ++s2)
      if (!have4(sh.have, s2)) {
        uint32_t w[4];
        recompute_stat_words<kDtype, kVecOk>(a, b, k, s2, kb, T, w, shu);
        __syncthreads();
        if (threadIdx.x == 0)
          for (int i = 0; i < 4; ++i) sh.words[4 * s2 + i] = w[i];
        __syncthreads();
      }
    if (threadIdx.x < kWave) {
      float Rt, Rd = 0.f;
      double Lt, Ld = 1.0;
      combine_row_wave(sh.words, S, 0, 1, Rt, Lt);
      if constexpr (kPair) combine_row_wave(sh.words, S, 2, 3, Rd, Ld);
      if (threadIdx.x == 0) {
        sh.Rt = Rt;
        sh.Lt = Lt;
        sh.Rd = Rd;
        sh.Ld = Ld;
      }
    }
    __syncthreads();
    recompute_overlap<kDtype, kVecOk>(a, b, k, s, kb, T, sh.Rt, sh.Lt, sh.Rd, sh.Ld, alpha_slice,
                                      sh.cm4, shu);
    cmass = sh.cm4[threadIdx.x / kWave];
    __syncthreads();
  }
  if ((threadIdx.x & (kWave - 1)) == 0)
    tag_store(a.chunk + chunk_idx(a, b, k, kWavesPerBlock * s + threadIdx.x / kWave), tag,
              __float_as_uint(cmass));
  if (kPair && threadIdx.x == 0)
    tag_store(a.apart + apart_idx(a, b, k, s), tag, __float_as_uint(alpha_slice));
}

template <int kDtype, bool kVecOk>
__global__ __launch_bounds__(kBlock) void verify_fused_kernel(Args a) {
  __shared__ Shared shu;
  ItemShared& sh = shu.it;
  const int S = a.S;
  const int per_req = (a.Kmax + 1) * S;
  const int item = blockIdx.x;
  const int b = item / per_req;
  const int rem = item - b * per_req;
  const int k = rem / S;
  const int s = rem - k * S;
  const int kb = a.kreq[b];
  const float T = a.temp[b];

  if (!(kb >= 0 && kb <= a.Kmax && temperature_ok(T))) {
    // invalid request: one workgroup writes the fault and completes it
    if (k == 0 && s == 0) {
      const uint32_t epoch = read_epoch(a.ctl);
      int st = 0;
      if (!temperature_ok(T)) st |= LVTV_STATUS_BAD_TEMPERATURE;
      if (kb < 0 || kb > a.Kmax) st |= LVTV_STATUS_BAD_K;
      write_fault(a, b, st);
      __syncthreads();
      if (threadIdx.x == 0) complete_unit(a, epoch);
    }
    return;
  }
  if (k > kb) return;

  uint32_t epoch;
  if (T == 0.f) {
    uint32_t w[4];
    recompute_stat_words<kDtype, kVecOk>(a, b, k, s, kb, T, w, shu);
    epoch = read_epoch(a.ctl);
    if (threadIdx.x == 0) {
      const uint32_t tag = tag_from_epoch(epoch);
      uint64_t* dst = a.stat + stat_idx(a, b, k, s);
      tag_store(dst + 0, tag, w[0]);
      tag_store(dst + 1, tag, w[1]);
      tag_store(dst + 2, tag, w[2]);
      tag_store(dst + 3, tag, w[3]);
    }
  } else if (k < kb) {
    stochastic_item<kDtype, kVecOk, true>(a, b, k, s, kb, T, epoch, shu);
  } else {
    stochastic_item<kDtype, kVecOk, false>(a, b, k, s, kb, T, epoch, shu);
  }

  // count this workgroup in; the request's last one finalises it
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.req + b, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sh.last = (old == uint32_t((kb + 1) * S - 1));
  }
  __syncthreads();
  if (!sh.last) return;
  finalize<kDtype, kVecOk>(a, b, kb, T, epoch, shu);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(a.req + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete_unit(a, epoch);
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  int S, NC;
  size_t off_stat, off_apart, off_chunk, total;
};

Layout make_layout(int B, int Kmax, int V) {
  Layout L;
  L.S = (V + kSlice - 1) / kSlice;
  L.NC = L.S * kWavesPerBlock;
  size_t off = kReservedBytes;
  L.off_stat = off;
  off = align256(off + sizeof(uint64_t) * size_t(B) * (Kmax + 1) * L.S * 4);
  L.off_apart = off;
  off = align256(off + sizeof(uint64_t) * size_t(B) * (Kmax > 0 ? Kmax : 1) * L.S);
  L.off_chunk = off;
  off = align256(off + sizeof(uint64_t) * size_t(B) * (Kmax + 1) * L.NC);
  L.total = off;
  return L;
}

template <int kDtype, bool kVecOk>
hipError_t launch(const Args& a, hipStream_t stream) {
  const size_t grid = size_t(a.B) * (a.Kmax + 1) * a.S;
  hipLaunchKernelGGL((verify_fused_kernel<kDtype, kVecOk>), dim3(unsigned(grid)), dim3(kBlock), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

bool applicable(int B, int Kmax, int V) {
  const int S = (V + kSlice - 1) / kSlice;
  return S <= kMaxSlices && size_t(B) * (Kmax + 1) * S < (size_t(1) << 31);
}

size_t workspace_bytes(int B, int Kmax, int V) { return make_layout(B, Kmax, V).total; }

hipError_t run(const VerifyCall& c, void* workspace, hipStream_t stream) {
  const Layout L = make_layout(c.B, c.Kmax, c.V);
  Args a;
  a.target = c.target;
  a.draft = c.draft;
  a.tokens = c.tokens;
  a.kreq = c.kreq;
  a.temp = c.temp;
  a.seed = c.seed;
  a.B = c.B;
  a.Kmax = c.Kmax;
  a.V = c.V;
  a.spin_limit = c.spin_limit;
  a.acc_len = c.acc_len;
  a.out_tokens = c.out_tokens;
  a.alpha = c.alpha;
  a.status = c.status;
  a.S = L.S;
  a.NC = L.NC;
  char* ws = static_cast<char*>(workspace);
  a.ctl = workspace_ctl(workspace);
  a.req = workspace_counters(workspace);
  a.stat = reinterpret_cast<uint64_t*>(ws + L.off_stat);
  a.apart = reinterpret_cast<uint64_t*>(ws + L.off_apart);
  a.chunk = reinterpret_cast<uint64_t*>(ws + L.off_chunk);
  if (c.dtype == LVTV_BF16)
    return c.vec_ok ? launch<1, true>(a, stream) : launch<1, false>(a, stream);
  return c.vec_ok ? launch<0, true>(a, stream) : launch<0, false>(a, stream);
}

}  // namespace vf
}  // namespace lvtv
