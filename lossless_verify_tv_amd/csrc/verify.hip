// spec_verify: speculative-sampling verify step on gfx950.
//
// Pipeline (three launches on the caller's stream, no host sync):
//
//   1. row_stats    grid (slice, row, request): per slice of every used row,
//                   the softmax statistics (max m, sum exp(s - m)) of the
//                   scaled logits, or for greedy requests (T = 0) the argmax
//                   and a NaN flag of the raw logits.
//   2. overlap      grid (slice, position, request): combines the slice
//                   statistics of target row k and draft row k, then over its
//                   slice accumulates alpha_k = sum min(p, q) and, per
//                   512-element chunk, the residual mass sum max(0, p - q);
//                   for the bonus row k = K_b it keeps the chunk masses of p.
//   3. finalize     grid (request): status checks, alpha_k in fp64, the
//                   accept scan with Philox uniforms, and the inverse-CDF
//                   draw: chunk choice from the chunk masses, then an fp64
//                   search inside the chosen chunk.
//
// Cites (page title, section): "Reading Qwen Bebop and DeepSeek DSpark",
// "Formulas" (alpha(y) = min(1, p/q); alpha_RS = sum min(p, q) = 1 - d_TV);
// "Speculative Decoding and MTP" survey, section 2 (ordered acceptance, bonus
// distribution), section 3 (residual max(0, p - q)/Z), section 4 (same
// temperature for p and q; greedy argmax rule), section 21 (acceptance and
// residual sampling fused on the GPU, no per-cycle CPU sync).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include <cstdlib>
#include <cstring>

#include "../../include/lvtv.h"
#include "device_common.hpp"
#include "fused_common.hpp"
#include "philox.hpp"
#include "verify_fused.hpp"

namespace lvtv {
namespace {

constexpr int kSlice = kBlock * kVec * 4;     // 8192 elements per slice
constexpr int kChunk = kWave * kVec;          // 512 elements per chunk
constexpr int kChunksPerSlice = kSlice / kChunk;
constexpr int kSteps = kSlice / (kBlock * kVec);

struct Layout {
  int S;    // slices per row
  int NC;   // chunks per row
  int R;    // rows per request in the stats arrays: Kmax+1 target, Kmax draft
  size_t off_stat, off_arg, off_alpha, off_chunk, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int B, int Kmax, int V) {
  Layout L;
  L.S = (V + kSlice - 1) / kSlice;
  L.NC = (V + kChunk - 1) / kChunk;
  L.R = 2 * Kmax + 1;
  size_t off = kReservedBytes;  // the fixed region stays untouched by this path
  L.off_stat = off;
  off = align256(off + sizeof(SliceStat) * size_t(B) * L.R * L.S);
  L.off_arg = off;
  off = align256(off + sizeof(ArgMax) * size_t(B) * L.R * L.S);
  L.off_alpha = off;
  off = align256(off + sizeof(double) * size_t(B) * (Kmax > 0 ? Kmax : 1) * L.S);
  L.off_chunk = off;
  off = align256(off + sizeof(double) * size_t(B) * (Kmax + 1) * L.NC);
  L.total = off;
  return L;
}

struct Args {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* kreq;
  const float* temp;
  const uint64_t* seed;
  int B, Kmax, V;
  bool vec_ok;
  int32_t* acc_len;
  int32_t* out_tokens;
  float* alpha;
  int32_t* status;
  Layout L;
  SliceStat* stat;
  ArgMax* arg;
  double* alpha_part;
  double* chunk;
};

__device__ __forceinline__ bool temperature_ok(float t) { return (t >= 0.f) && !isinf(t); }

__device__ __forceinline__ const void* row_ptr(const Args& a, int dtype_size, int b, bool target,
                                               int k) {
  const int64_t row = target ? (int64_t(b) * (a.Kmax + 1) + k) : (int64_t(b) * a.Kmax + k);
  const char* base = static_cast<const char*>(target ? a.target : a.draft);
  return base + row * int64_t(a.V) * dtype_size;
}

// ------------------------------------------------------------------ kernel 1

template <int kDtype>
__global__ __launch_bounds__(kBlock) void row_stats_kernel(Args a) {
  constexpr int kSize = kDtype == 1 ? 2 : 4;
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int kb = a.kreq[b];
  const float T = a.temp[b];
  if (kb < 0 || kb > a.Kmax || !temperature_ok(T)) return;
  const bool is_target = r <= a.Kmax;
  const int k = is_target ? r : r - (a.Kmax + 1);
  if (is_target ? (k > kb) : (k >= kb)) return;
  const void* row = row_ptr(a, kSize, b, is_target, k);
  const int64_t V = a.V;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const size_t slot = (size_t(b) * a.L.R + r) * a.L.S + s;

  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];
  __shared__ ArgMax sa[kWavesPerBlock];

  if (T == 0.f) {
    ArgMax best{-INFINITY, INT_MAX, 0};
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int64_t e = int64_t(s) * kSlice + it * (kBlock * kVec) + wave * kChunk + lane * kVec;
      float x[kVec];
      load8<kDtype>(row, e, V, a.vec_ok, x);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const int64_t idx = e + i;
        if (idx < V) {
          if (isnan(x[i])) {
            best.nan = 1;
          } else if (x[i] > best.v || (x[i] == best.v && idx < best.i)) {
            best.v = x[i];
            best.i = int32_t(idx);
          }
        }
      }
    }
    best = block_argmax(best, sa);
    if (threadIdx.x == 0) a.arg[slot] = best;
    return;
  }

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  float x[kSteps][kVec];
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t e = int64_t(s) * kSlice + it * (kBlock * kVec) + wave * kChunk + lane * kVec;
    load8<kDtype>(row, e, V, a.vec_ok, x[it]);
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      x[it][i] = scale_logit(x[it][i], inv_t, unit);
      m = fmaxf(m, x[it][i]);
    }
  }
  m = block_max(m, sf);
  const float ref = (m == -INFINITY) ? 0.f : m;
  const float neg = -ref * kLog2e;
  double l = 0.0;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc += exp_shifted(x[it][i], neg);
    l += acc;
  }
  l = block_sum(l, sd);
  if (threadIdx.x == 0) a.stat[slot] = SliceStat{(double)m, l};
}

// ------------------------------------------------------------------ kernel 2

template <int kDtype>
__global__ __launch_bounds__(kBlock) void overlap_kernel(Args a) {
  constexpr int kSize = kDtype == 1 ? 2 : 4;
  const int s = blockIdx.x, k = blockIdx.y, b = blockIdx.z;
  const int kb = a.kreq[b];
  const float T = a.temp[b];
  if (kb < 0 || kb > a.Kmax || !temperature_ok(T) || T == 0.f || k > kb) return;
  const int64_t V = a.V;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];

  const SliceStat* st_t = a.stat + (size_t(b) * a.L.R + k) * a.L.S;
  double Mt, Lt;
  combine_row_stats(st_t, a.L.S, sd, sf, Mt, Lt);
  const bool pair = k < kb;
  double Md = 0.0, Ld = 1.0;
  if (pair) {
    const SliceStat* st_d = a.stat + (size_t(b) * a.L.R + a.Kmax + 1 + k) * a.L.S;
    combine_row_stats(st_d, a.L.S, sd, sf, Md, Ld);
  }
  if (!isfinite(Mt) || !isfinite(Lt) || !isfinite(Md) || !isfinite(Ld)) return;

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  const float neg_t = -float(Mt) * kLog2e;
  const float neg_d = -float(Md) * kLog2e;
  const float inv_lt = float(1.0 / Lt);
  const float inv_ld = float(1.0 / Ld);
  const void* trow = row_ptr(a, kSize, b, true, k);
  const void* drow = pair ? row_ptr(a, kSize, b, false, k) : nullptr;
  double* chunk = a.chunk + (size_t(b) * (a.Kmax + 1) + k) * a.L.NC;

  double alpha = 0.0;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int c = s * kChunksPerSlice + it * kWavesPerBlock + wave;
    const int64_t e = int64_t(c) * kChunk + lane * kVec;
    float xt[kVec];
    load8<kDtype>(trow, e, V, a.vec_ok, xt);
    float mass = 0.f;
    if (pair) {
      float xd[kVec];
      load8<kDtype>(drow, e, V, a.vec_ok, xd);
      float amin = 0.f;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const float p = exp_shifted(scale_logit(xt[i], inv_t, unit), neg_t) * inv_lt;
        const float q = exp_shifted(scale_logit(xd[i], inv_t, unit), neg_d) * inv_ld;
        amin += fminf(p, q);
        mass += fmaxf(0.f, p - q);
      }
      alpha += amin;
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        mass += exp_shifted(scale_logit(xt[i], inv_t, unit), neg_t) * inv_lt;
    }
    const double cm = wave_sum((double)mass);
    if (lane == 0 && c < a.L.NC) chunk[c] = cm;
  }
  if (pair) {
    alpha = block_sum(alpha, sd);
    if (threadIdx.x == 0) a.alpha_part[(size_t(b) * a.Kmax + k) * a.L.S + s] = alpha;
  }
}

// ------------------------------------------------------------------ kernel 3

// Inclusive scan over the block of one fp64 value per thread, in a fixed
// order (Hillis-Steele inside each wave, then wave totals in wave order).
__device__ double block_inclusive_scan(double v, double* sd) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  __syncthreads();
  if (lane == kWave - 1) sd[wave] = v;
  __syncthreads();
  double pre = 0.0;
  for (int w = 0; w < wave; ++w) pre += sd[w];
  return v + pre;
}

__device__ int block_min_int(int v, int* si) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) si[wave] = v;
  __syncthreads();
  int r = si[0];
  for (int w = 1; w < kWavesPerBlock; ++w) r = min(r, si[w]);
  return r;
}

// Probability of element v of a row in fp64 from the canonical fp32 scaled
// logit and the row statistics.
template <int kDtype>
__device__ __forceinline__ double prob64(const void* row, int64_t v, float inv_t, bool unit,
                                         double M, double L) {
  const float s = scale_logit(load1<kDtype>(row, v), inv_t, unit);
  return exp((double)s - M) / L;
}

struct RowStat64 {
  double M, L;
};

// Weight of token v for the draw: residual max(0, p - q) or p alone.
template <int kDtype>
__device__ __forceinline__ double draw_weight(const void* trow, const void* drow, int64_t v,
                                              float inv_t, bool unit, RowStat64 st,
                                              RowStat64 sd_, bool residual) {
  const double p = prob64<kDtype>(trow, v, inv_t, unit, st.M, st.L);
  if (!residual) return p;
  const double q = prob64<kDtype>(drow, v, inv_t, unit, sd_.M, sd_.L);
  return fmax(0.0, p - q);
}

// Inverse-CDF draw over a row given the per-chunk masses of its weights:
// returns the smallest v whose cumulative weight exceeds u * total. The
// chunk is chosen from the chunk masses; the position inside the chunk from
// an fp64 recomputation of the weights.
template <int kDtype>
__device__ int draw_from_chunks(const double* masses, int NC, int64_t V, double u,
                                const void* trow, const void* drow, float inv_t, bool unit,
                                RowStat64 st, RowStat64 sdr, bool residual, double* sd,
                                int* si) {
  // blocked inclusive scan of the chunk masses
  const int per = (NC + kBlock - 1) / kBlock;
  const int c0 = threadIdx.x * per;
  double local = 0.0;
  for (int c = c0; c < min(NC, c0 + per); ++c) local += masses[c];
  const double incl = block_inclusive_scan(local, sd);
  __shared__ double total_sh;
  if (threadIdx.x == kBlock - 1) total_sh = incl;
  __syncthreads();
  const double total = total_sh;
  const double target = u * total;
  // first chunk whose inclusive cumulative mass exceeds the target
  int cand = INT_MAX;
  double run = incl - local;
  for (int c = c0; c < min(NC, c0 + per); ++c) {
    run += masses[c];
    if (run > target) {
      cand = c;
      break;
    }
  }
  int cstar = block_min_int(cand, si);
  __shared__ double before_sh;
  if (cand == cstar && cand != INT_MAX) {
    double before = incl - local;
    for (int c = c0; c < cstar; ++c) before += masses[c];
    before_sh = before;
  }
  __syncthreads();
  double rem;
  if (cstar != INT_MAX) {
    rem = target - before_sh;
  } else {
    // rounding put the target at or past the last cumulative value: take
    // the last chunk with positive mass and, inside it, its last element
    // with positive weight
    int lastc = -1;
    for (int c = c0; c < min(NC, c0 + per); ++c)
      if (masses[c] > 0.0) lastc = c;
    cstar = -block_min_int(lastc >= 0 ? -lastc : INT_MAX, si);
    if (cstar == -INT_MAX) cstar = NC - 1;
    rem = INFINITY;
  }
  // inside the chunk: 2 elements per thread, fp64 weights
  const int64_t base = int64_t(cstar) * kChunk;
  const int64_t v0 = base + 2 * threadIdx.x;
  double w0 = 0.0, w1 = 0.0;
  if (v0 < V) w0 = draw_weight<kDtype>(trow, drow, v0, inv_t, unit, st, sdr, residual);
  if (v0 + 1 < V) w1 = draw_weight<kDtype>(trow, drow, v0 + 1, inv_t, unit, st, sdr, residual);
  const double inc = block_inclusive_scan(w0 + w1, sd);
  const double exc = inc - (w0 + w1);
  int pick = INT_MAX;
  if (exc + w0 > rem && w0 > 0.0)
    pick = int(v0);
  else if (inc > rem && w1 > 0.0)
    pick = int(v0 + 1);
  int v = block_min_int(pick, si);
  if (v == INT_MAX) {
    // the fp64 weights of the chunk sum to slightly less than its fp32 mass:
    // take the last element of the chunk with positive weight
    int last = -1;
    if (w1 > 0.0 && v0 + 1 < V) last = int(v0 + 1);
    else if (w0 > 0.0 && v0 < V) last = int(v0);
    v = -block_min_int(last >= 0 ? -last : INT_MAX, si);
    if (v == -INT_MAX) v = int(base);
  }
  return v;
}

// Draw from p over the whole row when no chunk masses exist (rejection with a
// zero residual, i.e. p_j == q_j): two passes, first the total, then the
// first chunk whose cumulative mass passes the target.
template <int kDtype>
__device__ int draw_full_row(int64_t V, double u, const void* trow, float inv_t, bool unit,
                             RowStat64 st, double* sd, int* si) {
  const int NC = int((V + kChunk - 1) / kChunk);
  double total = 0.0;
  for (int c = 0; c < NC; ++c) {
    double w = 0.0;
    for (int64_t v = int64_t(c) * kChunk + threadIdx.x; v < min(V, int64_t(c + 1) * kChunk);
         v += kBlock)
      w += prob64<kDtype>(trow, v, inv_t, unit, st.M, st.L);
    total += block_sum(w, sd);
  }
  const double target = u * total;
  double run = 0.0;
  for (int c = 0; c < NC; ++c) {
    double w = 0.0;
    for (int64_t v = int64_t(c) * kChunk + threadIdx.x; v < min(V, int64_t(c + 1) * kChunk);
         v += kBlock)
      w += prob64<kDtype>(trow, v, inv_t, unit, st.M, st.L);
    const double m = block_sum(w, sd);
    if (run + m > target || c == NC - 1) {
      // sequential search inside the chunk by thread 0
      __shared__ int res;
      if (threadIdx.x == 0) {
        double r = run;
        int pick = -1, last = -1;
        for (int64_t v = int64_t(c) * kChunk; v < min(V, int64_t(c + 1) * kChunk); ++v) {
          const double pv = prob64<kDtype>(trow, v, inv_t, unit, st.M, st.L);
          if (pv > 0.0) last = int(v);
          r += pv;
          if (r > target && pv > 0.0) {
            pick = int(v);
            break;
          }
        }
        res = pick >= 0 ? pick : last;
      }
      __syncthreads();
      return res;
    }
    run += m;
  }
  return -1;
}

template <int kDtype>
__global__ __launch_bounds__(kBlock) void finalize_kernel(Args a) {
  constexpr int kSize = kDtype == 1 ? 2 : 4;
  const int b = blockIdx.x;
  const int Kmax = a.Kmax;
  const int kb = a.kreq[b];
  const float T = a.temp[b];
  const int64_t V = a.V;

  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];
  __shared__ int si[kWavesPerBlock];
  __shared__ ArgMax sa[kWavesPerBlock];
  __shared__ int status_sh;
  __shared__ RowStat64 stats[2 * LVTV_MAX_K + 1];
  __shared__ ArgMax argmaxes[2 * LVTV_MAX_K + 1];
  __shared__ int j_sh;

  // ---- status
  int status = 0;
  if (!temperature_ok(T)) status |= LVTV_STATUS_BAD_TEMPERATURE;
  if (kb < 0 || kb > Kmax) {
    status |= LVTV_STATUS_BAD_K;
  } else {
    int bad = 0;
    for (int k = threadIdx.x; k < kb; k += kBlock) {
      const int y = a.tokens[size_t(b) * Kmax + k];
      bad |= (y < 0 || y >= a.V);
    }
    if (block_min_int(bad ? 0 : 1, si) == 0) status |= LVTV_STATUS_BAD_TOKEN;
  }
  const bool greedy = (T == 0.f);
  if ((status & (LVTV_STATUS_BAD_K | LVTV_STATUS_BAD_TEMPERATURE)) == 0) {
    int fault = 0;
    for (int r = 0; r < 2 * kb + 1; ++r) {
      const int rr = r <= kb ? r : (Kmax + 1) + (r - kb - 1);   // stats row index
      const size_t base = (size_t(b) * a.L.R + rr) * a.L.S;
      if (greedy) {
        ArgMax best{-INFINITY, INT_MAX, 0};
        for (int s = threadIdx.x; s < a.L.S; s += kBlock) best = argmax_combine(best, a.arg[base + s]);
        best = block_argmax(best, sa);
        if (threadIdx.x == 0) argmaxes[r] = best;
        fault |= best.nan || !isfinite(best.v);
      } else {
        double M, L;
        combine_row_stats(a.stat + base, a.L.S, sd, sf, M, L);
        if (threadIdx.x == 0) stats[r] = RowStat64{M, L};
        fault |= !isfinite(M) || !isfinite(L);
      }
    }
    if (fault) status |= LVTV_STATUS_NONFINITE;
  }
  if (threadIdx.x == 0) status_sh = status;
  __syncthreads();
  status = status_sh;

  int32_t* out_tok = a.out_tokens + size_t(b) * (Kmax + 1);
  float* out_alpha = a.alpha + size_t(b) * Kmax;
  if (status) {
    for (int k = threadIdx.x; k <= Kmax; k += kBlock) out_tok[k] = -1;
    for (int k = threadIdx.x; k < Kmax; k += kBlock) out_alpha[k] = 0.f;
    if (threadIdx.x == 0) {
      a.status[b] = status;
      a.acc_len[b] = -1;
    }
    return;
  }

  const int32_t* y = a.tokens + size_t(b) * Kmax;
  if (greedy) {
    if (threadIdx.x == 0) {
      int j = kb;
      for (int k = 0; k < kb; ++k)
        if (y[k] != argmaxes[k].i) {
          j = k;
          break;
        }
      for (int k = 0; k < Kmax; ++k)
        out_alpha[k] = (k < kb) ? (argmaxes[k].i == argmaxes[kb + 1 + k].i ? 1.f : 0.f) : 0.f;
      for (int k = 0; k <= Kmax; ++k) out_tok[k] = k < j ? y[k] : (k == j ? argmaxes[j].i : -1);
      a.acc_len[b] = j;
      a.status[b] = 0;
    }
    return;
  }

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  const uint64_t seed = a.seed[b];

  // ---- alpha and the accept scan (thread 0; at most LVTV_MAX_K steps)
  if (threadIdx.x == 0) {
    for (int k = 0; k < Kmax; ++k) {
      double al = 0.0;
      if (k < kb)
        for (int s = 0; s < a.L.S; ++s) al += a.alpha_part[(size_t(b) * Kmax + k) * a.L.S + s];
      out_alpha[k] = float(al);
    }
    int j = kb;
    for (int k = 0; k < kb; ++k) {
      double u, u2;
      verify_uniforms(seed, uint64_t(b), uint64_t(k), u, u2);
      const int yk = y[k];
      const RowStat64 ts = stats[k], ds = stats[kb + 1 + k];
      const double p = prob64<kDtype>(row_ptr(a, kSize, b, true, k), yk, inv_t, unit, ts.M, ts.L);
      const double q = prob64<kDtype>(row_ptr(a, kSize, b, false, k), yk, inv_t, unit, ds.M, ds.L);
      const bool ok = (q == 0.0) ? (p > 0.0) : (u < p / q);
      if (!ok) {
        j = k;
        break;
      }
    }
    j_sh = j;
  }
  __syncthreads();
  const int j = j_sh;

  // ---- the draw at position j
  double u_acc, u_draw;
  verify_uniforms(seed, uint64_t(b), uint64_t(j), u_acc, u_draw);
  const bool residual = j < kb;
  const void* trow = row_ptr(a, kSize, b, true, j);
  const void* drow = residual ? row_ptr(a, kSize, b, false, j) : nullptr;
  const RowStat64 ts = stats[j];
  const RowStat64 ds = residual ? stats[kb + 1 + j] : RowStat64{0.0, 1.0};
  const double* masses = a.chunk + (size_t(b) * (Kmax + 1) + j) * a.L.NC;

  double tot_local = 0.0;
  for (int c = threadIdx.x; c < a.L.NC; c += kBlock) tot_local += masses[c];
  const double total = block_sum(tot_local, sd);
  int v;
  if (residual && !(total > 0.0)) {
    v = draw_full_row<kDtype>(V, u_draw, trow, inv_t, unit, ts, sd, si);
  } else {
    v = draw_from_chunks<kDtype>(masses, a.L.NC, V, u_draw, trow, drow, inv_t, unit, ts, ds,
                                 residual, sd, si);
  }
  if (threadIdx.x == 0) {
    for (int k = 0; k <= Kmax; ++k) out_tok[k] = k < j ? y[k] : (k == j ? v : -1);
    a.acc_len[b] = j;
    a.status[b] = 0;
  }
}

template <int kDtype>
hipError_t launch_all(const Args& a, hipStream_t stream) {
  dim3 g1(a.L.S, a.L.R, a.B);
  hipLaunchKernelGGL(row_stats_kernel<kDtype>, g1, dim3(kBlock), 0, stream, a);
  dim3 g2(a.L.S, a.Kmax + 1, a.B);
  hipLaunchKernelGGL(overlap_kernel<kDtype>, g2, dim3(kBlock), 0, stream, a);
  hipLaunchKernelGGL(finalize_kernel<kDtype>, dim3(a.B), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

bool sizes_ok(int32_t B, int32_t Kmax, int32_t V) {
  return B >= 1 && B <= 65535 && Kmax >= 0 && Kmax <= LVTV_MAX_K && V >= 1 && V <= LVTV_MAX_V;
}

}  // namespace
}  // namespace lvtv

namespace lvtv {
namespace {

// The single-read kernel serves every size it can hold; the two-read
// pipeline above serves the rest, and can be forced with
// LVTV_VERIFY_PATH=two-read (used to cross-check the two).
bool use_fused(int32_t B, int32_t Kmax, int32_t V) {
  const char* path = std::getenv("LVTV_VERIFY_PATH");
  if (path && std::strcmp(path, "two-read") == 0) return false;
  return vf::applicable(B, Kmax, V);
}

// Rounds a workgroup polls for a word before recomputing it itself
// (LVTV_SPIN_LIMIT; 0 makes every wait take the recompute path, which the
// tests use to exercise it).
int spin_limit() {
  const char* v = std::getenv("LVTV_SPIN_LIMIT");
  if (!v || !*v) return 1 << 16;
  const long n = std::strtol(v, nullptr, 10);
  return n < 0 ? 0 : (n > (1 << 30) ? (1 << 30) : int(n));
}

}  // namespace
}  // namespace lvtv

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t Kmax, int32_t V, int dtype) {
  if (!lvtv::sizes_ok(B, Kmax, V) || (dtype != LVTV_F32 && dtype != LVTV_BF16)) return 0;
  size_t n = lvtv::make_layout(B, Kmax, V).total;
  if (lvtv::vf::applicable(B, Kmax, V)) {
    const size_t f = lvtv::vf::workspace_bytes(B, Kmax, V);
    if (f > n) n = f;
  }
  return n;
}

extern "C" int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                           const int32_t* draft_tokens, const int32_t* k_per_req,
                           const float* temperature, const uint64_t* seed, int32_t B,
                           int32_t Kmax, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                           float* alpha, int32_t* status, void* workspace,
                           size_t workspace_bytes, void* stream) {
  using namespace lvtv;
  if (dtype != LVTV_F32 && dtype != LVTV_BF16) return LVTV_ERR_DTYPE;
  if (!sizes_ok(B, Kmax, V)) return LVTV_ERR_SHAPE;
  if (!target_logits || !k_per_req || !temperature || !seed || !accepted_len || !out_tokens ||
      !status)
    return LVTV_ERR_NULL;
  if (Kmax > 0 && (!draft_logits || !draft_tokens || !alpha)) return LVTV_ERR_NULL;
  const Layout L = make_layout(B, Kmax, V);
  if (!workspace || workspace_bytes < spec_verify_workspace_bytes(B, Kmax, V, dtype) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LVTV_ERR_WORKSPACE;
  const uintptr_t mis0 = reinterpret_cast<uintptr_t>(target_logits) |
                         reinterpret_cast<uintptr_t>(draft_logits);
  if (use_fused(B, Kmax, V)) {
    vf::VerifyCall c;
    c.target = target_logits;
    c.draft = draft_logits;
    c.dtype = dtype;
    c.vec_ok = (V % kVec == 0) && ((mis0 & 15) == 0);
    c.tokens = draft_tokens;
    c.kreq = k_per_req;
    c.temp = temperature;
    c.seed = seed;
    c.B = B;
    c.Kmax = Kmax;
    c.V = V;
    c.spin_limit = spin_limit();
    c.acc_len = accepted_len;
    c.out_tokens = out_tokens;
    c.alpha = alpha;
    c.status = status;
    const hipError_t e = vf::run(c, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
  }
  Args a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.kreq = k_per_req;
  a.temp = temperature;
  a.seed = seed;
  a.B = B;
  a.Kmax = Kmax;
  a.V = V;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(target_logits) |
                        reinterpret_cast<uintptr_t>(draft_logits);
  a.vec_ok = (V % kVec == 0) && ((mis & 15) == 0);
  a.acc_len = accepted_len;
  a.out_tokens = out_tokens;
  a.alpha = alpha;
  a.status = status;
  a.L = L;
  char* ws = static_cast<char*>(workspace);
  a.stat = reinterpret_cast<SliceStat*>(ws + L.off_stat);
  a.arg = reinterpret_cast<ArgMax*>(ws + L.off_arg);
  a.alpha_part = reinterpret_cast<double*>(ws + L.off_alpha);
  a.chunk = reinterpret_cast<double*>(ws + L.off_chunk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      dtype == LVTV_BF16 ? launch_all<1>(a, s) : launch_all<0>(a, s);
  return err == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}
