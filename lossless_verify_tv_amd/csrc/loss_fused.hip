// e2e_tv_loss_fwd_bwd, single-read kernel for gfx950 (V <= 155648).
//
// One 1024-thread workgroup per (branch n, position j) row:
//   1. loads the row's bf16 draft logits z once and keeps them in registers
//      (19 groups of 8 tokens per thread, packed two per register);
//   2. the softmax statistics of z from the registers: the maximum M, then
//      L = sum 2^((z - M) log2 e) (fp32 per group of 8, fp64 across groups);
//   3. streams the fp32 target probabilities p once: q = softmax(z) from the
//      registers, alpha_j = sum min(q, p), S_j = sum_{q<p} q,
//      S'_j = sum_{q>=p} q (fp64 across groups), and one bit [q < p] per
//      token, kept in registers;
//   4. publishes (alpha_j, S_j, S'_j) and its row statistics to the branch
//      and collects those of the branch's other rows (tagged words; see
//      fused_common.hpp). The wait is bounded: a row that gives up is marked
//      unfinished and a repair launch, which runs once every row has
//      published, completes it with the same per-group steps (bit-identical);
//   5. the branch scalars in fp64: prefix products P_k, the loss
//      L_n = -sum_k P_k, R_k = 1 + alpha_{k+1} R_{k+1} and
//      dL_n/dalpha_j = -P_{j-1} R_j; the gradient
//      dz(u) = (G_j / N) q(u) ([q(u) < p(u)] - S_j), evaluated as
//      (G_j/N) S'_j q(u) where the bit is set and -(G_j/N) S_j q(u) elsewhere,
//      rounded to bf16 (nearest even) and written once.
// Then the repair launch (normally a no-op) and a last launch that averages
// the branch losses in a fixed order and advances the workspace's call epoch.
//
// Definition (page title, section): "SpecOPD: Branch-Parallel On-Policy
// Distillation for Speculative Decoding", prerequisite on acceptance length
// and the E2E-TV objective (alpha = sum min(q, p) = 1 - TV; prefix products
// of alpha aggregate it) and method step (6) (the prefix product of the
// per-position overlaps gives the loss; only the draft probabilities are
// differentiated, the target is a constant); "Reading Qwen Bebop and DeepSeek
// DSpark", section "Bebop's solution" (E[tau] = sum_j prod_{k<=j}(1 - d_TV)).
// Gradient: d alpha / d q(v) = [q(v) < p(v)] and the softmax Jacobian
// dq(v)/dz(u) = q(v)(delta_uv - q(u)).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/lvtv.h"
#include "device_common.hpp"
#include "fused_common.hpp"
#include "loss_fused.hpp"
#include "wave_dpp.hpp"

namespace lvtv {
namespace lf {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;         // 16
constexpr int kTile = kThreads * kVec;           // 8192 tokens per group index
constexpr int kZG = kMaxGroups;                  // groups of z held per thread
constexpr int kZL = 8;                           // ... of which in LDS (128 KB per workgroup)
constexpr int kZR = kZG - kZL;                   // ... and in registers
constexpr int kMaskWords = (kZG * kVec + 31) / 32;
constexpr int kPBatch = 4;                       // groups of p in flight together
constexpr int kWords = 8;  // tagged words per row: alpha, S, S' (fp64 pairs), -M log2 e, 1/L
constexpr float kL2E = 1.44269504088896340736f;
static_assert(kZG * kTile >= kMaxV, "held groups cover the largest V");

struct Args {
  const uint16_t* z;
  const float* p;
  int N, W, V;
  int spin_limit;
  float* alpha;
  uint16_t* dz;
  float* loss;
  FusedCtl* ctl;
  uint64_t* words;      // [N][W][kWords] tagged words
  uint64_t* unfinished; // [N][W] tagged: this call left the row's dz to the repair launch
  double* branch_loss;  // [N]
};

// ------------------------------------------------------------------ loads

// This thread's first token in group g is tb + g * kTile, tb = 8 * thread.
// Each phase takes tb through opaque() so the compiler recomputes the
// per-group offsets where they are used instead of keeping all 19 alive in
// registers for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ int group_elem(int g) { return g * kTile + threadIdx.x * kVec; }

// z group g of a row: 8 bf16 tokens packed in 4 registers; tokens at or
// beyond V read as -inf.
// With kVecOk (16-byte aligned rows, V % 8 == 0) a group lies wholly inside
// or wholly past the end of the row; the load is unconditional (a
// past-the-end group reads the row's first group) and the select comes
// after it, so no branch splits a batch of loads.
template <bool kVecOk>
__device__ __forceinline__ u32x4 load_z(const uint16_t* row, int V, int e) {
  if constexpr (kVecOk) {
    const bool in = e < V;
    const u32x4 v = ld_nt16(row + (in ? e : 0));
    const uint32_t f = 0xff80ff80u;
    return u32x4{in ? v[0] : f, in ? v[1] : f, in ? v[2] : f, in ? v[3] : f};
  } else {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = (e + 2 * h < V) ? row[e + 2 * h] : 0xff80u;
      const uint32_t hi = (e + 2 * h + 1 < V) ? row[e + 2 * h + 1] : 0xff80u;
      r[h] = lo | (hi << 16);
    }
    return r;
  }
}

// p group g of a row: 8 fp32 values; values at or beyond V read as 0.
template <bool kVecOk>
__device__ __forceinline__ void load_p(const float* row, int V, int e, u32x4& a, u32x4& b) {
  if constexpr (kVecOk) {
    const bool in = e < V;
    const float* q = row + (in ? e : 0);
    const u32x4 x = ld_nt16(q), y = ld_nt16(q + 4);
    a = u32x4{in ? x[0] : 0u, in ? x[1] : 0u, in ? x[2] : 0u, in ? x[3] : 0u};
    b = u32x4{in ? y[0] : 0u, in ? y[1] : 0u, in ? y[2] : 0u, in ? y[3] : 0u};
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      a[h] = (e + h < V) ? __float_as_uint(row[e + h]) : 0u;
      b[h] = (e + 4 + h < V) ? __float_as_uint(row[e + 4 + h]) : 0u;
    }
  }
}

__device__ __forceinline__ float zelem(const u32x4& g, int j) {
  const uint32_t w = g[j >> 1];
  return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}

// The held row: groups [0, kZL) in LDS (each thread its own 16-byte slot
// per group, so no barrier is needed between a thread's write and its
// reads), groups [kZL, kZG) in registers.
struct Held {
  u32x4 r[kZR];
  u32x4 (*lds)[kThreads];
  // The LDS slot address goes through opaque() so each read stays where it
  // is used (not hoisted, all at once, to the start of a phase).
  __device__ __forceinline__ u32x4 get(int g) const {
    if (g < kZL) {
      const int slot = opaque(int(threadIdx.x));
      return lds[g][slot];
    }
    return r[g - kZL];
  }
};

// Makes the compiler treat the held z registers as rewritten, so each phase
// recomputes its exponentials from them instead of carrying the previous
// phase's (up to 152 values per thread) across a block reduction or the
// exchange.
__device__ __forceinline__ void launder(Held& h) {
#pragma unroll
  for (int g = 0; g < kZR; ++g) asm volatile("" : "+v"(h.r[g]));
}

__device__ __forceinline__ float pelem(const u32x4& a, const u32x4& b, int j) {
  return __uint_as_float(j < 4 ? a[j] : b[j - 4]);
}

// q of one token: 2^(z log2 e - M log2 e) / L, as in the oracle's softmax up
// to fp32 rounding.
__device__ __forceinline__ float qval(float z, float nm, float inv_l) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(z, kL2E, nm)) * inv_l;
}

// ------------------------------------------------------------------ block reductions

struct Shared {
  float f[kWaves];
  double d[kWaves][3];
  uint32_t words[LVTV_MAX_W * kWords];
  uint8_t have[LVTV_MAX_W * kWords];
  double coef[2];
};

__device__ __forceinline__ float block_max(float v, Shared& sh) {
  v = wmax(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.f[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh.f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sh.f[w]);
  return r;
}

__device__ __forceinline__ void block_sum3(double& a, double& b, double& c, Shared& sh) {
  a = wsum(a);
  b = wsum(b);
  c = wsum(c);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.d[threadIdx.x / kWave][0] = a;
    sh.d[threadIdx.x / kWave][1] = b;
    sh.d[threadIdx.x / kWave][2] = c;
  }
  __syncthreads();
  a = sh.d[0][0];
  b = sh.d[0][1];
  c = sh.d[0][2];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    a += sh.d[w][0];
    b += sh.d[w][1];
    c += sh.d[w][2];
  }
}

// ------------------------------------------------------------------ per-group steps
//
// Shared by the register path and the streaming recomputation, so both give
// the same bits (same element order, same reduction tree).

__device__ __forceinline__ float grp_max(const u32x4& g, float m) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) m = fmaxf(m, zelem(g, j));
  return m;
}

__device__ __forceinline__ float grp_expsum(const u32x4& g, float nm) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) s += __builtin_amdgcn_exp2f(__builtin_fmaf(zelem(g, j), kL2E, nm));
  return s;
}

// alpha, S and S' parts of a group, and its 8 mask bits.
__device__ __forceinline__ uint32_t grp_overlap(const u32x4& g, const u32x4& pa, const u32x4& pb,
                                                float nm, float inv_l, double& al, double& sb,
                                                double& sa) {
  float a = 0.f, b = 0.f, c = 0.f;
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float q = qval(zelem(g, j), nm, inv_l);
    const float p = pelem(pa, pb, j);
    a += fminf(q, p);
    const bool below = q < p;
    b += below ? q : 0.f;
    c += below ? 0.f : q;
    bits |= below ? (1u << j) : 0u;
  }
  al += (double)a;
  sb += (double)b;
  sa += (double)c;
  return bits;
}

// Row statistics (M log2 e as the exponent offset, 1/L) from per-thread
// partials.
struct RowStats {
  float nm;     // -M log2 e (0 when M = -inf)
  float inv_l;  // fl32(1 / L)
};

__device__ __forceinline__ RowStats finish_stats(float m, double l, Shared& sh) {
  // every thread's m is already the block maximum here
  double x = l, unused0 = 0.0, unused1 = 0.0;
  block_sum3(x, unused0, unused1, sh);
  RowStats r;
  r.nm = (m == -INFINITY) ? 0.f : -(m * kL2E);
  r.inv_l = float(1.0 / x);
  return r;
}

// ------------------------------------------------------------------ the kernel

// fp64 value from two consecutive 32-bit exchange words (low half first).
__device__ __forceinline__ double word_f64(const uint32_t* w, int i) {
  return __longlong_as_double((long long)((uint64_t(w[i + 1]) << 32) | w[i]));
}

// Branch scalars from the W rows' words (thread 0, fp64): the branch loss
// (written by row 0), alpha_j, and this row's two gradient coefficients in
// sh.coef: (G_j/N) S'_j where q < p, -(G_j/N) S_j elsewhere.
__device__ __forceinline__ void branch_scalars(const Args& a, int n, int j, size_t row,
                                               Shared& sh) {
  const int W = a.W;
  if (threadIdx.x == 0) {
    double run = 1.0, loss_n = 0.0, before = 1.0;
    for (int k = 0; k < W; ++k) {
      if (k == j) before = run;
      run *= word_f64(sh.words, k * kWords);
      loss_n -= run;
    }
    double suffix = 1.0;  // R_{W-1} = 1, R_k = 1 + alpha_{k+1} R_{k+1}
    for (int k = W - 2; k >= j; --k) suffix = 1.0 + word_f64(sh.words, (k + 1) * kWords) * suffix;
    const double g = -before * suffix / double(a.N);
    sh.coef[0] = g * word_f64(sh.words, j * kWords + 4);   // S'_j
    sh.coef[1] = -g * word_f64(sh.words, j * kWords + 2);  // S_j
    a.alpha[row] = float(word_f64(sh.words, j * kWords));
    if (j == 0) a.branch_loss[n] = loss_n;
  }
  __syncthreads();
}

// dz of one group of 8 tokens, bf16 (nearest even), from z, the group's
// mask bits and the row's coefficients.
template <bool kVecOk>
__device__ __forceinline__ void dz_group(const u32x4& zv, const uint32_t (&mask)[kMaskWords],
                                         int g, int e, int V, const RowStats& rs, float c_below,
                                         float c_above, uint16_t* dz) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float v2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int jj = 2 * h + t;
      const bool below = (mask[(g * kVec + jj) / 32] >> ((g * kVec + jj) % 32)) & 1u;
      v2[t] = qval(zelem(zv, jj), rs.nm, rs.inv_l) * (below ? c_below : c_above);
    }
    const bf16x2 b = __builtin_convertvector(f32x2{v2[0], v2[1]}, bf16x2);
    out[h] = __builtin_bit_cast(uint32_t, b);
  }
  if (kVecOk) {
    if (e < V) st_nt16(dz + e, out);
  } else {
#pragma unroll
    for (int t = 0; t < kVec; ++t)
      if (e + t < V) dz[e + t] = uint16_t(out[t >> 1] >> (16 * (t & 1)));
  }
}


template <bool kVecOk>
__device__ __forceinline__ void row_body(const Args& a) {
  __shared__ Shared sh;
  const int W = a.W, V = a.V;
  // uniform row coordinates, kept in scalar registers
  const int n = __builtin_amdgcn_readfirstlane(int(blockIdx.x) / W);
  const int j = __builtin_amdgcn_readfirstlane(int(blockIdx.x) - n * W);
  const size_t row = size_t(blockIdx.x);
  const uint16_t* z = a.z + row * V;
  const float* p = a.p + row * V;
  const uint32_t tag = tag_from_epoch(read_epoch(a.ctl));

  // 1. z into registers
  __shared__ u32x4 zl[kZL][kThreads];
  Held zg;
  zg.lds = zl;
  {
    const int tb = opaque(int(threadIdx.x) * kVec);
    u32x4 tmp[kZL];
#pragma unroll
    for (int g = 0; g < kZL; ++g) tmp[g] = load_z<kVecOk>(z, V, tb + g * kTile);
#pragma unroll
    for (int g = kZL; g < kZG; ++g) zg.r[g - kZL] = load_z<kVecOk>(z, V, tb + g * kTile);
#pragma unroll
    for (int g = 0; g < kZL; ++g) zl[g][threadIdx.x] = tmp[g];
  }

  // 2. statistics
  float m = -INFINITY;
#pragma unroll
  for (int g = 0; g < kZG; ++g) m = grp_max(zg.get(g), m);
  launder(zg);
  m = block_max(m, sh);
  const float nm0 = (m == -INFINITY) ? 0.f : -(m * kL2E);
  double l = 0.0;
#pragma unroll
  for (int g = 0; g < kZG; ++g) l += (double)grp_expsum(zg.get(g), nm0);
  launder(zg);
  const RowStats rs = finish_stats(m, l, sh);

  // 3. one pass over p
  double al = 0.0, sb = 0.0, sa = 0.0;
  uint32_t mask[kMaskWords];
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) mask[w] = 0u;
  const int tbp = opaque(int(threadIdx.x) * kVec);
#pragma unroll
  for (int g0 = 0; g0 < kZG; g0 += kPBatch) {
    u32x4 pa[kPBatch], pb[kPBatch];
#pragma unroll
    for (int i = 0; i < kPBatch; ++i)
      if (g0 + i < kZG) load_p<kVecOk>(p, V, opaque(tbp) + (g0 + i) * kTile, pa[i], pb[i]);
#pragma unroll
    for (int i = 0; i < kPBatch; ++i)
      if (g0 + i < kZG) {
        const int g = g0 + i;
        const uint32_t bits = grp_overlap(zg.get(g), pa[i], pb[i], rs.nm, rs.inv_l, al, sb, sa);
        mask[(g * kVec) / 32] |= bits << ((g * kVec) % 32);
      }
    // keep the next batch's loads behind this batch's arithmetic
    __builtin_amdgcn_sched_barrier(0);
  }
  launder(zg);
  block_sum3(al, sb, sa, sh);

  // 4. exchange within the branch
  if (threadIdx.x == 0) {
    uint64_t* w = a.words + row * kWords;
    const double v[3] = {al, sb, sa};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint64_t bits = uint64_t(__double_as_longlong(v[i]));
      tag_store(w + 2 * i, tag, uint32_t(bits));
      tag_store(w + 2 * i + 1, tag, uint32_t(bits >> 32));
    }
    tag_store(w + 6, tag, __float_as_uint(rs.nm));
    tag_store(w + 7, tag, __float_as_uint(rs.inv_l));
  }
  uint64_t* src = a.words + size_t(n) * W * kWords;
  const int nw = W * kWords;
  for (int i = threadIdx.x; i < nw; i += kThreads) sh.have[i] = 0;
  __syncthreads();
  bool fresh = false;
  for (int round = 0;; ++round) {
    int missing = 0;
    for (int i = threadIdx.x; i < nw; i += kThreads) {
      if (!sh.have[i]) {
        const uint64_t w = tag_load(src + i);
        if (uint32_t(w >> 32) == tag) {
          sh.words[i] = uint32_t(w);
          sh.have[i] = 1;
        } else {
          missing = 1;
        }
      }
    }
    if (!__syncthreads_or(missing)) {
      fresh = true;
      break;
    }
    if (round >= a.spin_limit) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (!fresh) {
    // Rare: the rest of the branch did not arrive within the spin limit
    // (its rows may not be resident yet). Leave this row to the repair
    // launch, which runs after every row has published its words.
    if (threadIdx.x == 0) tag_store(a.unfinished + row, tag, 1u);
    return;
  }
  branch_scalars(a, n, j, row, sh);
  const float c_below = float(sh.coef[0]);
  const float c_above = float(sh.coef[1]);
  // 5. dz from the held row and the mask
  uint16_t* dz = a.dz + row * V;
  const int tbd = opaque(int(threadIdx.x) * kVec);
#pragma unroll
  for (int g = 0; g < kZG; ++g) {
    dz_group<kVecOk>(zg.get(g), mask, g, opaque(tbd) + g * kTile, V, rs, c_below, c_above, dz);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Rows a workgroup left unfinished in this call (see above): every row has
// published its words by now, so the branch scalars are at hand; z and p
// are read again to form the mask and dz with the same per-group steps.
template <bool kVecOk>
__device__ __forceinline__ void repair_body(const Args& a) {
  __shared__ Shared sh;
  const int W = a.W, V = a.V;
  const uint32_t tag = tag_from_epoch(read_epoch(a.ctl));
  const size_t rows = size_t(a.N) * W;
  for (size_t row = blockIdx.x; row < rows; row += gridDim.x) {
    if (uint32_t(tag_load(a.unfinished + row) >> 32) != tag) continue;
    const int n = int(row / W), j = int(row - size_t(n) * W);
    uint64_t* src = a.words + size_t(n) * W * kWords;
    for (int i = threadIdx.x; i < W * kWords; i += kThreads) sh.words[i] = uint32_t(tag_load(src + i));
    __syncthreads();
    RowStats rs;
    rs.nm = __uint_as_float(sh.words[j * kWords + 6]);
    rs.inv_l = __uint_as_float(sh.words[j * kWords + 7]);
    branch_scalars(a, n, j, row, sh);
    const float c_below = float(sh.coef[0]);
    const float c_above = float(sh.coef[1]);
    const uint16_t* z = a.z + row * V;
    const float* p = a.p + row * V;
    uint16_t* dz = a.dz + row * V;
#pragma unroll
    for (int g = 0; g < kZG; ++g) {
      const int e = group_elem(g);
      const u32x4 zv = load_z<kVecOk>(z, V, e);
      u32x4 pa, pb;
      load_p<kVecOk>(p, V, e, pa, pb);
      double x = 0.0, y = 0.0, w = 0.0;
      uint32_t m1[kMaskWords];
#pragma unroll
      for (int i = 0; i < kMaskWords; ++i) m1[i] = 0u;
      m1[(g * kVec) / 32] = grp_overlap(zv, pa, pb, rs.nm, rs.inv_l, x, y, w) << ((g * kVec) % 32);
      dz_group<kVecOk>(zv, m1, g, e, V, rs, c_below, c_above, dz);
    }
    __syncthreads();
  }
}

template <bool kVecOk>
__global__ __launch_bounds__(kThreads) void loss_rows(Args a) {
  row_body<kVecOk>(a);
}

template <bool kVecOk>
__global__ __launch_bounds__(kThreads) void loss_repair(Args a) {
  repair_body<kVecOk>(a);
}

// Mean of the branch losses in a fixed order; then the call epoch advances
// (every row workgroup of this call has finished: it ran before this
// launch).
__global__ __launch_bounds__(256) void loss_reduce(Args a) {
  __shared__ double sd[256 / kWave];
  const int per = (a.N + 255) / 256;
  double x = 0.0;
  for (int n = threadIdx.x * per; n < min(a.N, (int(threadIdx.x) + 1) * per); ++n)
    x += a.branch_loss[n];
  x = wsum(x);
  if ((threadIdx.x & (kWave - 1)) == 0) sd[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < 256 / kWave; ++w) t += sd[w];
    a.loss[0] = float(t / double(a.N));
    const uint32_t e = read_epoch(a.ctl);
    __hip_atomic_store(&a.ctl->epoch, e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t off_words, off_unfinished, off_branch, total;
};

Layout make_layout(int N, int W) {
  Layout L;
  size_t off = kReservedBytes;
  L.off_words = off;
  off = align256(off + sizeof(uint64_t) * size_t(N) * W * kWords);
  L.off_unfinished = off;
  off = align256(off + sizeof(uint64_t) * size_t(N) * W);
  L.off_branch = off;
  off = align256(off + sizeof(double) * size_t(N));
  L.total = off;
  return L;
}

}  // namespace

bool applicable(int N, int W, int V) {
  return V <= kMaxV && size_t(N) * W < (size_t(1) << 31);
}

size_t workspace_bytes(int N, int W, int V) {
  (void)V;
  return make_layout(N, W).total;
}

hipError_t run(const LossCall& c, void* workspace, hipStream_t stream) {
  const Layout L = make_layout(c.N, c.W);
  Args a;
  a.z = c.z;
  a.p = c.p;
  a.N = c.N;
  a.W = c.W;
  a.V = c.V;
  a.spin_limit = c.spin_limit;
  a.alpha = c.alpha;
  a.dz = c.dz;
  a.loss = c.loss;
  char* ws = static_cast<char*>(workspace);
  a.ctl = workspace_ctl(workspace);
  a.words = reinterpret_cast<uint64_t*>(ws + L.off_words);
  a.unfinished = reinterpret_cast<uint64_t*>(ws + L.off_unfinished);
  a.branch_loss = reinterpret_cast<double*>(ws + L.off_branch);
  const unsigned grid = unsigned(size_t(c.N) * c.W);
  if (c.vec_ok)
    hipLaunchKernelGGL(loss_rows<true>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(loss_rows<false>, dim3(grid), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rgrid = grid < 256u ? grid : 256u;
  if (c.vec_ok)
    hipLaunchKernelGGL(loss_repair<true>, dim3(rgrid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(loss_repair<false>, dim3(rgrid), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_reduce, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lf
}  // namespace lvtv
