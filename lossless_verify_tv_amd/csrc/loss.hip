// e2e_tv_loss_fwd_bwd: E2E-TV prefix-product loss and its gradient on gfx950,
// and draft_loss_fwd_bwd: the same machinery under the per-position
// comparators the pages set against it (per-step TV, CE, KL).
//
// Definition (page title, section): "SpecOPD: Branch-Parallel On-Policy
// Distillation for Speculative Decoding", prerequisite "Acceptance length and
// the E2E-TV objective" (alpha = sum min(q, p) = 1 - TV; prefix products of
// alpha aggregate it) and method step (6) (the prefix product of the
// per-position overlaps gives the loss; only the draft probabilities are
// differentiated, samples and target are constants); "Reading Qwen Bebop and
// DeepSeek DSpark", section "Bebop's solution" (E[tau] = sum_j prod_{k<=j}
// (1 - d_TV)).
//
// Pipeline (launches on the caller's stream, no host sync):
//   1. row_stats  grid (slice, position, branch): per slice (m, sum exp(z - m)).
//   2. overlap    grid (slice, position, branch): q = softmax(z) from the
//                 combined statistics; per slice alpha = sum min(q, p),
//                 S = sum_{q<p} q and S' = sum_{q>=p} q, in fp64.
//   3. branch     grid (branch): alpha_k, S_k, S'_k; prefix products P_j,
//                 suffix sums R_k = 1 + alpha_{k+1} R_{k+1}, the branch loss
//                 L_n = -sum_j P_j and dL_n/dalpha_k = -P_{k-1} R_k; the
//                 per-row gradient coefficients.
//   4. reduce     one workgroup: loss = (1/N) sum_n L_n in fixed order.
//   5. grad       grid (slice, position, branch): dz = q (G/N) S' where q < p,
//                 -q (G/N) S elsewhere; bfloat16 round-to-nearest-even.
//
// Comparators ("Reading Qwen Bebop and DeepSeek DSpark", section "Bebop's
// solution": CE = -sum p log q, KL(p || q) = sum p log(p / q), per-step
// L_TV = 1 - sum min(p, q)), each summed over a branch's positions and
// averaged over branches:
//   * per-step TV: G = -1 for every position, the rest as above;
//   * CE and KL: the overlap pass also sums p, p z and (KL) p ln p per row;
//     CE_k = -sum p z + (M + ln L) sum p (log q = z - M - ln L), KL_k = CE_k +
//     sum p ln p; dz = q (sum p)/N - p/N, one fused multiply-add.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/lvtv.h"
#include "device_common.hpp"
#include "fused_common.hpp"
#include "loss_fused.hpp"

#include <cmath>

namespace lvtv {
namespace {

constexpr int kSlice = kBlock * kVec * 4;  // 8192 elements per slice
constexpr int kSteps = kSlice / (kBlock * kVec);

struct RowFinal {
  float neg_m_log2e;  // -M c (c = log2(e) fl32(1/T), log2(e) without a temperature)
  float inv_l;        // 1 / L
  float c_below;      // (G/N) S'   applied where q < p    (CE, KL: (sum p)/N, the weight of q)
  float c_above;      // -(G/N) S   applied where q >= p   (CE, KL: 1/N, the weight of p)
  float neg_t;        // target given as logits: -M_t c of the target row
  float inv_lt;       // ... and 1 / L_t
};

struct Part {
  double alpha, s_below, s_above;
  double sp, spz, splp;  // CE and KL: sum p, sum p z, sum p ln p (0 otherwise)
};

struct Layout {
  int S;
  size_t off_stat, off_part, off_fin, off_branch, total;
};

// Statistics are kept for two rows per (branch, position): the draft row,
// then (target given as logits) the target row.
constexpr int kStatSets = 2;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int N, int W, int V) {
  Layout L;
  L.S = (V + kSlice - 1) / kSlice;
  const size_t rows = size_t(N) * W;
  size_t off = kReservedBytes;
  L.off_stat = off;
  off = align256(off + sizeof(SliceStat) * rows * L.S * kStatSets);
  L.off_part = off;
  off = align256(off + sizeof(Part) * rows * L.S);
  L.off_fin = off;
  off = align256(off + sizeof(RowFinal) * rows);
  L.off_branch = off;
  off = align256(off + sizeof(double) * size_t(N));
  L.total = off;
  return L;
}

struct Args {
  const uint16_t* z;
  const float* p;         // target probabilities (null when the target is logits)
  const uint16_t* t;      // target logits (null when the target is probabilities)
  float c;                // exponent scale log2(e) fl32(1/T) (log2(e) at T = 1)
  double stat_scale;      // c ln 2 (1 at T = 1): weight of a shift of the maximum
  double inv_t;           // chain factor fl32(1/T) of the gradient (1 at T = 1)
  int N, W, V;
  int objective;  // LVTV_OBJ_*
  bool vec_ok;
  float* loss;
  float* alpha;
  uint16_t* dz;
  float* dz32;  // debug: the fp32 gradient before rounding, or null
  Layout L;
  SliceStat* stat;
  Part* part;
  RowFinal* fin;
  double* branch_loss;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);  // quiet NaN
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void load8_p(const float* row, int64_t e, int64_t V, bool vec_ok,
                                        float (&x)[kVec]) {
  if (vec_ok && e + kVec <= V) {
    const float4 a = *reinterpret_cast<const float4*>(row + e);
    const float4 b = *reinterpret_cast<const float4*>(row + e + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < kVec; ++i) x[i] = (e + i < V) ? row[e + i] : 0.f;
  }
}

__device__ __forceinline__ int64_t elem_index(int s, int it) {
  return int64_t(s) * kSlice + it * (kBlock * kVec) + threadIdx.x * kVec;
}

// 2^(x c + neg), c the exponent scale of the call.
__device__ __forceinline__ float exp_c(float x, float c, float neg) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, neg));
}

// Grid (slice, position, branch); with a logits target the second half of
// the slices' blocks take the target row.
__global__ __launch_bounds__(kBlock) void row_stats_kernel(Args a) {
  const bool tgt = int(blockIdx.x) >= a.L.S;
  const int s = int(blockIdx.x) - (tgt ? a.L.S : 0);
  const size_t row = size_t(blockIdx.z) * a.W + blockIdx.y;
  const size_t rows = size_t(a.N) * a.W;
  const uint16_t* z = (tgt ? a.t : a.z) + row * a.V;
  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];
  float x[kSteps][kVec];
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    load8<1>(z, elem_index(s, it), a.V, a.vec_ok, x[it]);
#pragma unroll
    for (int i = 0; i < kVec; ++i) m = fmaxf(m, x[it][i]);
  }
  m = block_max(m, sf);
  const float ref = (m == -INFINITY) ? 0.f : m;
  const float neg = -ref * a.c;
  double l = 0.0;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc += exp_c(x[it][i], a.c, neg);
    l += acc;
  }
  l = block_sum(l, sd);
  if (threadIdx.x == 0) a.stat[(tgt ? rows : 0) * a.L.S + row * a.L.S + s] = SliceStat{(double)m, l};
}

// Row statistics (M, L) of the draft row (set 0) or the target row (set 1),
// L = sum 2^((x - M) c) over the row.
__device__ __forceinline__ void row_stats(const Args& a, size_t row, int set, double* sd,
                                          float* sf, double& M, double& L) {
  const size_t rows = size_t(a.N) * a.W;
  combine_row_stats(a.stat + (set ? rows : 0) * a.L.S + row * a.L.S, a.L.S, sd, sf, M, L,
                    a.stat_scale);
}

// Target probabilities of the group at e: loaded (probability target) or
// p = 2^(t c - M_t c) / L_t from the target logits; 0 past V either way.
__device__ __forceinline__ void target_group(const Args& a, const float* p, const uint16_t* t,
                                             int64_t e, float neg_t, float inv_lt,
                                             float (&xp)[kVec]) {
  if (t != nullptr) {
    float xt[kVec];
    load8<1>(t, e, a.V, a.vec_ok, xt);
#pragma unroll
    for (int i = 0; i < kVec; ++i) xp[i] = exp_c(xt[i], a.c, neg_t) * inv_lt;
  } else {
    load8_p(p, e, a.V, a.vec_ok, xp);
  }
}

__global__ __launch_bounds__(kBlock) void overlap_kernel(Args a) {
  const int s = blockIdx.x;
  const size_t row = size_t(blockIdx.z) * a.W + blockIdx.y;
  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];
  double M, L;
  row_stats(a, row, 0, sd, sf, M, L);
  const float neg = -float(M) * a.c;
  const float inv_l = float(1.0 / L);
  const uint16_t* z = a.z + row * a.V;
  const bool logits = a.t != nullptr;
  const float* p = logits ? nullptr : a.p + row * a.V;
  const uint16_t* t = logits ? a.t + row * a.V : nullptr;
  float neg_t = 0.f, inv_lt = 0.f;
  if (logits) {
    double Mt, Lt;
    row_stats(a, row, 1, sd, sf, Mt, Lt);
    neg_t = -float(Mt) * a.c;
    inv_lt = float(1.0 / Lt);
  }
  const bool xent = a.objective == LVTV_OBJ_CE || a.objective == LVTV_OBJ_KL;
  const bool kl = a.objective == LVTV_OBJ_KL;
  double al = 0.0, sb = 0.0, sa = 0.0, sp = 0.0, spz = 0.0, splp = 0.0;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t e = elem_index(s, it);
    float xz[kVec], xp[kVec], xt[kVec];
    load8<1>(z, e, a.V, a.vec_ok, xz);
    if (logits) {
      load8<1>(t, e, a.V, a.vec_ok, xt);
#pragma unroll
      for (int i = 0; i < kVec; ++i) xp[i] = exp_c(xt[i], a.c, neg_t) * inv_lt;
    } else {
      load8_p(p, e, a.V, a.vec_ok, xp);
    }
    float a_min = 0.f, a_below = 0.f, a_above = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const float q = exp_c(xz[i], a.c, neg) * inv_l;
      a_min += fminf(q, xp[i]);
      const bool below = q < xp[i];
      a_below += below ? q : 0.f;
      a_above += below ? 0.f : q;
    }
    al += a_min;
    sb += a_below;
    sa += a_above;
    if (xent) {
      float b_p = 0.f, b_pz = 0.f, b_plp = 0.f;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const int64_t v = e + i;
        // tokens past V read z = -inf and p = 0: they add nothing
        if (v < a.V) {
          b_p += xp[i];
          b_pz += xp[i] * xz[i];
          // KL: sum p ln p for a probability target; for a logits target
          // sum p (t - z), from which the branch kernel forms
          // sum p (ln p - ln q) without a cancellation against CE
          if (kl && logits && xp[i] > 0.f) b_plp += xp[i] * (xt[i] - xz[i]);
          if (kl && !logits && xp[i] > 0.f) b_plp += xp[i] * logf(xp[i]);
        }
      }
      sp += b_p;
      spz += b_pz;
      splp += b_plp;
    }
  }
  al = block_sum(al, sd);
  sb = block_sum(sb, sd);
  sa = block_sum(sa, sd);
  if (xent) {
    sp = block_sum(sp, sd);
    spz = block_sum(spz, sd);
    splp = block_sum(splp, sd);
  }
  if (threadIdx.x == 0) a.part[row * a.L.S + s] = Part{al, sb, sa, sp, spz, splp};
}

__global__ __launch_bounds__(kBlock) void branch_kernel(Args a) {
  const int n = blockIdx.x;
  const int W = a.W;
  __shared__ double sd[kWavesPerBlock];
  __shared__ float sf[kWavesPerBlock];
  __shared__ double al[LVTV_MAX_W], sb[LVTV_MAX_W], sa[LVTV_MAX_W];
  __shared__ double Ms[LVTV_MAX_W], Ls[LVTV_MAX_W], Mts[LVTV_MAX_W], Lts[LVTV_MAX_W];
  __shared__ double sps[LVTV_MAX_W], spzs[LVTV_MAX_W], splps[LVTV_MAX_W];
  for (int k = 0; k < W; ++k) {
    const size_t row = size_t(n) * W + k;
    double M, L, Mt = 0.0, Lt = 1.0;
    row_stats(a, row, 0, sd, sf, M, L);
    if (a.t != nullptr) row_stats(a, row, 1, sd, sf, Mt, Lt);
    double x = 0.0, y = 0.0, w = 0.0, u = 0.0, t = 0.0, r = 0.0;
    for (int s = threadIdx.x; s < a.L.S; s += kBlock) {
      const Part pt = a.part[row * a.L.S + s];
      x += pt.alpha;
      y += pt.s_below;
      w += pt.s_above;
      u += pt.sp;
      t += pt.spz;
      r += pt.splp;
    }
    x = block_sum(x, sd);
    y = block_sum(y, sd);
    w = block_sum(w, sd);
    u = block_sum(u, sd);
    t = block_sum(t, sd);
    r = block_sum(r, sd);
    if (threadIdx.x == 0) {
      al[k] = x;
      sb[k] = y;
      sa[k] = w;
      Ms[k] = M;
      Ls[k] = L;
      Mts[k] = Mt;
      Lts[k] = Lt;
      sps[k] = u;
      spzs[k] = t;
      splps[k] = r;
    }
  }
  __syncthreads();
  // the row's exponent references; gradient coefficients carry the chain
  // factor of the temperature scaling
  auto row_final = [&](int k) {
    RowFinal f{-float(Ms[k]) * a.c, float(1.0 / Ls[k]), 0.f, 0.f, 0.f, 0.f};
    if (a.t != nullptr) {
      f.neg_t = -float(Mts[k]) * a.c;
      f.inv_lt = float(1.0 / Lts[k]);
    }
    return f;
  };
  if (threadIdx.x == 0 && a.objective != LVTV_OBJ_E2E_TV) {
    const double inv_n = 1.0 / double(a.N);
    double loss_n = 0.0;
    for (int k = 0; k < W; ++k) {
      const size_t row = size_t(n) * W + k;
      RowFinal fin = row_final(k);
      if (a.objective == LVTV_OBJ_STEP_TV) {
        loss_n += 1.0 - al[k];
        fin.c_below = float(-inv_n * sa[k] * a.inv_t);
        fin.c_above = float(inv_n * sb[k] * a.inv_t);
      } else {
        // log q = s - M_s - ln L with s = z fl32(1/T) and M_s = M fl32(1/T),
        // so -sum p log q = -fl32(1/T) sum p z + (M_s + ln L) sum p
        const double ce = -a.inv_t * spzs[k] + (a.inv_t * Ms[k] + log(Ls[k])) * sps[k];
        if (a.objective == LVTV_OBJ_CE)
          loss_n += ce;
        else if (a.t == nullptr)
          loss_n += ce + splps[k];
        else  // ln p - ln q = (t - z)/T - (M_t - M)/T - ln L_t + ln L
          loss_n += a.inv_t * splps[k] -
                    (a.inv_t * (Mts[k] - Ms[k]) + log(Lts[k]) - log(Ls[k])) * sps[k];
        fin.c_below = float(sps[k] * inv_n * a.inv_t);
        fin.c_above = float(inv_n * a.inv_t);
      }
      a.fin[row] = fin;
      a.alpha[row] = float(al[k]);
    }
    a.branch_loss[n] = loss_n;
  }
  if (threadIdx.x == 0 && a.objective == LVTV_OBJ_E2E_TV) {
    double prefix[LVTV_MAX_W], suffix[LVTV_MAX_W];
    double run = 1.0, loss_n = 0.0;
    for (int k = 0; k < W; ++k) {
      run *= al[k];
      prefix[k] = run;
      loss_n -= run;
    }
    suffix[W - 1] = 1.0;
    for (int k = W - 2; k >= 0; --k) suffix[k] = 1.0 + al[k + 1] * suffix[k + 1];
    const double inv_n = 1.0 / double(a.N);
    for (int k = 0; k < W; ++k) {
      const double g = -(k > 0 ? prefix[k - 1] : 1.0) * suffix[k] * inv_n * a.inv_t;
      const size_t row = size_t(n) * W + k;
      RowFinal fin = row_final(k);
      fin.c_below = float(g * sa[k]);
      fin.c_above = float(-g * sb[k]);
      a.fin[row] = fin;
      a.alpha[row] = float(al[k]);
    }
    a.branch_loss[n] = loss_n;
  }
}

__global__ __launch_bounds__(kBlock) void reduce_kernel(Args a) {
  __shared__ double sd[kWavesPerBlock];
  // fixed order: contiguous blocks per thread, then the block tree
  const int per = (a.N + kBlock - 1) / kBlock;
  double x = 0.0;
  for (int n = threadIdx.x * per; n < min(a.N, (int(threadIdx.x) + 1) * per); ++n)
    x += a.branch_loss[n];
  x = block_sum(x, sd);
  if (threadIdx.x == 0) a.loss[0] = float(x / double(a.N));
}

__global__ __launch_bounds__(kBlock) void grad_kernel(Args a) {
  const int s = blockIdx.x;
  const size_t row = size_t(blockIdx.z) * a.W + blockIdx.y;
  const RowFinal f = a.fin[row];
  const bool xent = a.objective == LVTV_OBJ_CE || a.objective == LVTV_OBJ_KL;
  const uint16_t* z = a.z + row * a.V;
  const bool logits = a.t != nullptr;
  const float* p = logits ? nullptr : a.p + row * a.V;
  const uint16_t* t = logits ? a.t + row * a.V : nullptr;
  uint16_t* dz = a.dz + row * a.V;
  float* dz32 = a.dz32 ? a.dz32 + row * a.V : nullptr;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t e = elem_index(s, it);
    if (e >= a.V) break;
    float xz[kVec], xp[kVec];
    load8<1>(z, e, a.V, a.vec_ok, xz);
    target_group(a, p, t, e, f.neg_t, f.inv_lt, xp);
    float g[kVec];
    if (xent) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const float q = exp_c(xz[i], a.c, f.neg_m_log2e) * f.inv_l;
        g[i] = __builtin_fmaf(q, f.c_below, -(xp[i] * f.c_above));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const float q = exp_c(xz[i], a.c, f.neg_m_log2e) * f.inv_l;
        g[i] = q * (q < xp[i] ? f.c_below : f.c_above);
      }
    }
    uint16_t out[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) out[i] = f32_to_bf16_rne(g[i]);
    if (a.vec_ok && e + kVec <= a.V) {
      uint4 w;
      w.x = uint32_t(out[0]) | (uint32_t(out[1]) << 16);
      w.y = uint32_t(out[2]) | (uint32_t(out[3]) << 16);
      w.z = uint32_t(out[4]) | (uint32_t(out[5]) << 16);
      w.w = uint32_t(out[6]) | (uint32_t(out[7]) << 16);
      *reinterpret_cast<uint4*>(dz + e) = w;
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        if (e + i < a.V) dz[e + i] = out[i];
    }
    if (dz32) {
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        if (e + i < a.V) dz32[e + i] = g[i];
    }
  }
}

bool sizes_ok(int32_t N, int32_t W, int32_t V) {
  return N >= 1 && N <= LVTV_MAX_N && W >= 1 && W <= LVTV_MAX_W && V >= 1 && V <= LVTV_MAX_V;
}

}  // namespace
}  // namespace lvtv

namespace lvtv {
namespace {

// Rounds a half-row workgroup of the single-read kernel polls for the rest
// of its branch before leaving its row to the call's last launch.
constexpr int kSpinLimit = 1 << 16;

// How a call is run. The product entry points take the defaults; the debug
// entry point lvtv_debug_draft_loss sets them (the tests use it to compare
// the two paths, to force the repair path and to read the fp32 gradient).
struct Options {
  int path = LVTV_PATH_AUTO;
  int spin_limit = kSpinLimit;
  float* dz32 = nullptr;
};

// The single-read kernel serves every V it can hold; the multi-pass
// pipeline above serves the rest.
bool use_fused(const Options& o, int32_t N, int32_t W, int32_t V) {
  if (o.path == LVTV_PATH_MULTI_PASS) return false;
  return lf::applicable(N, W, V);
}

}  // namespace
}  // namespace lvtv

namespace lvtv {
namespace {

size_t loss_workspace_bytes(int32_t N, int32_t W, int32_t V) {
  if (!sizes_ok(N, W, V)) return 0;
  size_t n = make_layout(N, W, V).total;
  if (lf::applicable(N, W, V)) {
    const size_t f = lf::workspace_bytes(N, W, V);
    if (f > n) n = f;
  }
  return n;
}

// The target of a call: probabilities used as given, or logits with a
// temperature applied to both rows.
struct Target {
  const float* probs;
  const uint16_t* logits;
  float temperature;
};

int run_loss(const uint16_t* draft_logits, const Target& tg, int32_t N, int32_t W, int32_t V,
             int objective, float* loss, float* alpha, uint16_t* dlogits, void* workspace,
             size_t workspace_bytes, void* stream, const Options& opt = Options()) {
  if (!sizes_ok(N, W, V)) return LVTV_ERR_SHAPE;
  if (objective < LVTV_OBJ_E2E_TV || objective > LVTV_OBJ_KL) return LVTV_ERR_OBJECTIVE;
  const bool logits = tg.logits != nullptr || tg.probs == nullptr;
  if (!draft_logits || (logits ? !tg.logits : !tg.probs) || !loss || !alpha || !dlogits)
    return LVTV_ERR_NULL;
  if (logits && !(tg.temperature > 0.f && std::isfinite(tg.temperature) &&
                  std::isfinite(1.f / tg.temperature)))
    return LVTV_ERR_TEMPERATURE;
  const Layout L = make_layout(N, W, V);
  if (!workspace || workspace_bytes < loss_workspace_bytes(N, W, V) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LVTV_ERR_WORKSPACE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(draft_logits) |
                        reinterpret_cast<uintptr_t>(logits ? static_cast<const void*>(tg.logits)
                                                           : static_cast<const void*>(tg.probs)) |
                        reinterpret_cast<uintptr_t>(dlogits);
  const bool vec_ok = (V % kVec == 0) && ((mis & 15) == 0);
  // Exponent scale c = fl32(log2(e) fl32(1/T)) (log2(e) itself at T = 1, and
  // for a probability target, which has no temperature).
  const bool unit = !logits || tg.temperature == 1.f;
  const float inv_t = unit ? 1.f : 1.f / tg.temperature;
  const float c = unit ? kLog2e : kLog2e * inv_t;
  // the single-read kernel serves the TV objectives (their gradients need
  // only the held z, the mask and per-row scalars) and, for a probability
  // target, CE and KL (their gradient written in the pass over p, and
  // rewritten from a second pass where a row's target does not sum to one
  // closely enough)
  const bool tv = objective == LVTV_OBJ_E2E_TV || objective == LVTV_OBJ_STEP_TV;
  const bool fused_ok = tv ? (!logits || lf::logits_supported()) : lf::xent_supported(logits);
  if (fused_ok && use_fused(opt, N, W, V)) {
    lf::LossCall lc;
    lc.z = draft_logits;
    lc.p = logits ? nullptr : tg.probs;
    lc.t = logits ? tg.logits : nullptr;
    lc.c = c;
    lc.inv_t = double(inv_t);
    lc.N = N;
    lc.W = W;
    lc.V = V;
    lc.objective = objective;
    lc.vec_ok = vec_ok;
    lc.spin_limit = opt.spin_limit;
    lc.reread = opt.path == LVTV_PATH_REREAD;
    lc.loss = loss;
    lc.alpha = alpha;
    lc.dz = dlogits;
    lc.dz32 = opt.dz32;
    const hipError_t e = lf::run(lc, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
  }
  Args a;
  a.z = draft_logits;
  a.p = logits ? nullptr : tg.probs;
  a.t = logits ? tg.logits : nullptr;
  a.c = c;
  a.stat_scale = unit ? 1.0 : double(c) * 0.69314718055994530942;
  a.inv_t = double(inv_t);
  a.N = N;
  a.W = W;
  a.V = V;
  a.objective = objective;
  a.vec_ok = vec_ok;
  a.loss = loss;
  a.alpha = alpha;
  a.dz = dlogits;
  a.dz32 = opt.dz32;
  a.L = L;
  char* ws = static_cast<char*>(workspace);
  a.stat = reinterpret_cast<SliceStat*>(ws + L.off_stat);
  a.part = reinterpret_cast<Part*>(ws + L.off_part);
  a.fin = reinterpret_cast<RowFinal*>(ws + L.off_fin);
  a.branch_loss = reinterpret_cast<double*>(ws + L.off_branch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(L.S, W, N);
  const dim3 grid_stats(L.S * (logits ? 2 : 1), W, N);
  hipLaunchKernelGGL(row_stats_kernel, grid_stats, dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(overlap_kernel, grid, dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(branch_kernel, dim3(N), dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(reduce_kernel, dim3(1), dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(grad_kernel, grid, dim3(kBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}

}  // namespace
}  // namespace lvtv

extern "C" size_t e2e_tv_loss_workspace_bytes(int32_t N, int32_t W, int32_t V) {
  return lvtv::loss_workspace_bytes(N, W, V);
}

extern "C" size_t draft_loss_workspace_bytes(int32_t N, int32_t W, int32_t V) {
  return lvtv::loss_workspace_bytes(N, W, V);
}

extern "C" int e2e_tv_loss_fwd_bwd(const uint16_t* draft_logits, const float* target_probs,
                                   int32_t N, int32_t W, int32_t V, float* loss, float* alpha,
                                   uint16_t* dlogits, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const lvtv::Target tg{target_probs, nullptr, 1.f};
  return lvtv::run_loss(draft_logits, tg, N, W, V, LVTV_OBJ_E2E_TV, loss, alpha, dlogits,
                        workspace, workspace_bytes, stream);
}

extern "C" int draft_loss_fwd_bwd(const uint16_t* draft_logits, const float* target_probs,
                                  int32_t N, int32_t W, int32_t V, int objective, float* loss,
                                  float* alpha, uint16_t* dlogits, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const lvtv::Target tg{target_probs, nullptr, 1.f};
  return lvtv::run_loss(draft_logits, tg, N, W, V, objective, loss, alpha, dlogits, workspace,
                        workspace_bytes, stream);
}

extern "C" size_t draft_loss_logits_workspace_bytes(int32_t N, int32_t W, int32_t V) {
  return lvtv::loss_workspace_bytes(N, W, V);
}

extern "C" int draft_loss_logits_fwd_bwd(const uint16_t* draft_logits,
                                         const uint16_t* target_logits, float temperature,
                                         int32_t N, int32_t W, int32_t V, int objective,
                                         float* loss, float* alpha, uint16_t* dlogits,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  const lvtv::Target tg{nullptr, target_logits, temperature};
  return lvtv::run_loss(draft_logits, tg, N, W, V, objective, loss, alpha, dlogits, workspace,
                        workspace_bytes, stream);
}

extern "C" int lvtv_debug_draft_loss(const uint16_t* draft_logits, const float* target_probs,
                                     const uint16_t* target_logits, float temperature, int32_t N,
                                     int32_t W, int32_t V, int objective, int path,
                                     int32_t spin_limit, float* loss, float* alpha,
                                     uint16_t* dlogits, float* dlogits_f32, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (path != LVTV_PATH_AUTO && path != LVTV_PATH_MULTI_PASS && path != LVTV_PATH_REREAD)
    return LVTV_ERR_OPTION;
  if ((target_probs == nullptr) == (target_logits == nullptr)) return LVTV_ERR_NULL;
  lvtv::Options opt;
  opt.path = path;
  opt.spin_limit = spin_limit < 0 ? 0 : spin_limit;
  opt.dz32 = dlogits_f32;
  const lvtv::Target tg{target_probs, target_logits, target_logits ? temperature : 1.f};
  return lvtv::run_loss(draft_logits, tg, N, W, V, objective, loss, alpha, dlogits, workspace,
                        workspace_bytes, stream, opt);
}
