// e2e_tv_loss_fwd_bwd, single-read kernels for gfx950 (V <= 155648).
//
// Each (branch n, position j) row is split in two halves of up to 19 tiles
// of 4096 tokens; one 512-thread workgroup per half, two per compute unit
// (so one can compute while the other streams). A half-row workgroup:
//   1. loads its half of the bf16 draft logits z once and keeps it: 19 groups
//      of 8 tokens per thread, 8 groups in LDS (64 KB) and 11 in registers;
//   2. computes the half's softmax statistics (maximum M_h, sum of
//      2^((z - M_h) log2 e)), swaps them with the other half through tagged
//      words and combines both into the row's M and L (the same arithmetic,
//      in the same order, in both halves);
//   3. streams its half of the fp32 target probabilities p once: q = softmax(z)
//      from the held copy, and the half's parts of alpha_j = sum min(q, p),
//      S_j = sum_{q<p} q and S'_j = sum_{q>=p} q (fp64 across groups), with one
//      bit [q < p] per token kept in registers;
//   4. publishes those parts and collects the parts of every half of the
//      branch's rows (tagged words; see fused_common.hpp); alpha_k, S_k and
//      S'_k are the two halves' sums, half 0 first;
//   5. the branch scalars in fp64: prefix products P_k, the loss
//      L_n = -sum_k P_k, R_k = 1 + alpha_{k+1} R_{k+1} and
//      dL_n/dalpha_j = -P_{j-1} R_j; the gradient
//      dz(u) = (G_j / N) q(u) ([q(u) < p(u)] - S_j), evaluated as
//      (G_j/N) S'_j q(u) where the bit is set and -(G_j/N) S_j q(u) elsewhere,
//      rounded to bf16 (nearest even) and written once.
// With the target given as bf16 logits (draft_loss_logits_fwd_bwd), step 2
// also streams the half of the target row once for its statistics (a running
// maximum and sum per thread), swapped with the other half like the draft's,
// and step 3 streams it again, forming p = softmax(t) per token instead of
// loading it; both rows take the exponent scale c = log2(e) fl32(1/T), and
// the gradient coefficients carry the chain factor fl32(1/T).
// Every wait is bounded: a half that gives up marks its row unfinished and
// stops. The call's last launch, one workgroup that runs once every half has
// finished, completes such rows from the published words, recomputing
// whatever is missing with the same per-group steps and reductions
// (bit-identical); it then averages the branch losses in a fixed order and
// advances the workspace's call epoch.
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

#include <climits>
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

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;         // 8
constexpr int kTile = kThreads * kVec;           // 4096 tokens per group index
constexpr int kZG = kMaxGroups;                  // groups of z held per thread (one half)
constexpr int kHalf = kZG * kTile;               // tokens per half row
constexpr int kZL = 8;                           // ... of which in LDS (64 KB per workgroup)
constexpr int kZR = kZG - kZL;                   // ... and in registers
constexpr int kWholeMaxV = kHalf;                 // rows up to this take one workgroup
constexpr int kMaskWords = (kZG * kVec + 31) / 32;
constexpr int kPBatch = 4;                       // groups of p in flight together
static_assert(2 * kHalf >= kMaxV, "two halves cover the largest V");

// Tagged words per half row: the half's statistics, then its parts of the
// branch sums.
constexpr int kStatWords = 3;    // M_h (fp32), L_h (fp64)
constexpr int kPartWords = 6;    // alpha_h, S_h, S'_h (fp64)
constexpr int kSlotWords = 16;   // per half: [0,3) statistics, [4,10) parts,
constexpr int kTStatWord = 10;   // [10,13) the target row's statistics (logits target)

struct Args {
  const uint16_t* z;
  const float* p;        // target probabilities, or
  const uint16_t* t;     // target logits (kLogits)
  float c;               // exponent scale log2(e) fl32(1/T) (log2(e) at T = 1)
  double inv_t;          // chain factor fl32(1/T) of the gradient
  int N, W, V;
  int objective;  // LVTV_OBJ_E2E_TV or LVTV_OBJ_STEP_TV
  int spin_limit;
  int whole;      // 1: one workgroup takes a whole row (its second half is empty)
  int reread;     // CE / KL: 1 rewrites every row's dz from a second read of p
  float* alpha;
  uint16_t* dz;
  float* dz32;           // debug output: the fp32 gradient before rounding (kDbg only)
  float* loss;
  FusedCtl* ctl;
  uint64_t* words;       // [N][W][2][kSlotWords] tagged words
  uint64_t* unfinished;  // [N][W] tagged: the row is left to the last launch
  double* branch_loss;   // [N]
};

// ------------------------------------------------------------------ loads

// Keeps a value opaque to the compiler: per-group offsets derived from it
// are recomputed where used instead of being kept alive in registers for the
// whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A row's halves: [0, hv) and [hv, V). With two workgroups a row, hv =
// ceil(V / 2) rounded up to a whole group (at most kHalf), so that both get
// about the same work whatever V is; with one (whole, V <= kHalf), hv is V
// rounded up to a group and the second half is empty.
__host__ __device__ __forceinline__ int half_len(int V, int whole) {
  const int hv = ((whole ? V : (V + 1) / 2) + kVec - 1) / kVec * kVec;
  return hv < kHalf ? hv : kHalf;
}

// End of half h: its tokens are read up to here (the rest as past the end).
__host__ __device__ __forceinline__ int half_end(int V, int hv, int h) {
  const int e = (h + 1) * hv;
  return e < V ? e : V;
}

// Groups (a thread's kVec tokens in each of kTile) that half h reaches;
// the rest hold no token of it and are skipped (they would add only zeros).
__host__ __device__ __forceinline__ int half_groups(int V, int hv, int h) {
  const int n = half_end(V, hv, h) - h * hv;
  return n > 0 ? (n + kTile - 1) / kTile : 0;
}

// First token of this thread's group g in half h.
__device__ __forceinline__ int group_elem(int hv, int h, int g) {
  return h * hv + g * kTile + int(threadIdx.x) * kVec;
}

// z group of a row: 8 bf16 tokens packed in 4 registers; tokens at or beyond
// V read as -inf. With kVecOk (16-byte aligned rows, V % 8 == 0) a group lies
// wholly inside or wholly past the end of the row; the load is unconditional
// (a past-the-end group reads the row's first group) and the select comes
// after it, so no branch splits a batch of loads.
template <bool kVecOk>
__device__ __forceinline__ u32x4 load_z(const uint16_t* row, int V, int e) {
  if constexpr (kVecOk) {
    const bool in = e < V;
    const u32x4 v = ld_nt16(row + (in ? e : 0));
    const uint32_t f = 0xff80ff80u;
    return u32x4{in ? v[0] : f, in ? v[1] : f, in ? v[2] : f, in ? v[3] : f};
  } else {
    // rows that are not 16-byte aligned (V >= 8 on this kernel): one
    // unaligned vector load of the 16 bytes that end at the group's end or
    // at the row's end, whichever comes first (always inside the row), and
    // the tokens moved into place (no move inside the row). No branch, so
    // nothing splits a batch of loads.
    const int es = min(e, V - kVec);
    return shift_bf16(ld_nt16_u(row + es), uint32_t(e - es), 0xff80ff80u);
  }
}

// p group of a row: 8 fp32 values; values at or beyond V read as 0.
template <bool kVecOk>
__device__ __forceinline__ void load_p(const float* row, int V, int e, u32x4& a, u32x4& b) {
  if constexpr (kVecOk) {
    const bool in = e < V;
    const float* q = row + (in ? e : 0);
    const u32x4 x = ld_nt16(q), y = ld_nt16(q + 4);
    a = u32x4{in ? x[0] : 0u, in ? x[1] : 0u, in ? x[2] : 0u, in ? x[3] : 0u};
    b = u32x4{in ? y[0] : 0u, in ? y[1] : 0u, in ? y[2] : 0u, in ? y[3] : 0u};
  } else {
    // rows that are not 16-byte aligned, as for z
    const int es = min(e, V - kVec);
    a = ld_nt16_u(row + es);
    b = ld_nt16_u(row + es + 4);
    shift_f32(a, b, uint32_t(e - es), 0u);
  }
}

__device__ __forceinline__ float zelem(const u32x4& g, int j) {
  const uint32_t w = g[j >> 1];
  return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ float pelem(const u32x4& a, const u32x4& b, int j) {
  return __uint_as_float(j < 4 ? a[j] : b[j - 4]);
}

// The held half row: groups [0, kZL) in LDS (each thread its own 16-byte
// slot per group, so no barrier is needed between a thread's write and its
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

// Makes the compiler treat the held registers as rewritten, so each phase
// recomputes its exponentials from them instead of carrying the previous
// phase's across a block reduction or an exchange.
__device__ __forceinline__ void launder(Held& h) {
#pragma unroll
  for (int g = 0; g < kZR; ++g) asm volatile("" : "+v"(h.r[g]));
}

// q of one token: 2^(z c - M c) / L (c = log2 e without a temperature).
__device__ __forceinline__ float qval(float z, float c, float nm, float inv_l) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(z, c, nm)) * inv_l;
}

// ------------------------------------------------------------------ block reductions

struct Shared {
  float f[kWaves];
  double d[kWaves][3];
  uint32_t words[LVTV_MAX_W * 2 * kSlotWords];
  uint8_t have[LVTV_MAX_W * 2 * kSlotWords];
  double coef[2];
  int imin[kWaves];
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
// Shared by the workgroups and the last launch, so both give the same bits
// (same element order, same reduction tree).

__device__ __forceinline__ float grp_max(const u32x4& g, float m) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) m = fmaxf(m, zelem(g, j));
  return m;
}

__device__ __forceinline__ float grp_expsum(const u32x4& g, float c, float nm) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) s += __builtin_amdgcn_exp2f(__builtin_fmaf(zelem(g, j), c, nm));
  return s;
}

// Reference and inverse sum of a row's softmax: p or q = 2^(x c + nm) inv_l.
struct RowStats {
  float nm;     // -M c (0 when M = -inf)
  float inv_l;  // fl32(1 / L)
};

// alpha, S and S' parts of a group, and its 8 mask bits. The target's group
// is (pa, pb), 8 probabilities, or (kLogits) pa, 8 bf16 logits whose p is
// formed with the target row's statistics ts.
template <bool kLogits>
__device__ __forceinline__ uint32_t grp_overlap(const u32x4& g, const u32x4& pa, const u32x4& pb,
                                                float cz, const RowStats& rs, const RowStats& ts,
                                                double& al, double& sb, double& sa) {
  float a = 0.f, b = 0.f, c = 0.f;
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float q = qval(zelem(g, j), cz, rs.nm, rs.inv_l);
    const float p = kLogits ? qval(zelem(pa, j), cz, ts.nm, ts.inv_l) : pelem(pa, pb, j);
    const bool below = q < p;
    a += below ? q : p;
    b += below ? q : 0.f;
    c += below ? 0.f : q;
    bits |= below ? (1u << j) : 0u;
  }
  al += (double)a;
  sb += (double)b;
  sa += (double)c;
  return bits;
}

// Stores a group's dz (8 bf16 in out; kDbg: their fp32 values g32 in dz32
// as well): one 16-byte store inside the row, token by token in a ragged
// last group.
template <bool kVecOk, bool kDbg>
__device__ __forceinline__ void store_dz(const u32x4& out, const float (&g32)[kVec], int e, int V,
                                         uint16_t* dz, float* dz32) {
  if (kVecOk) {
    if (e < V) st_nt16(dz + e, out);
  } else if (e + kVec <= V) {
    st_nt16_u(dz + e, out);
  } else {
#pragma unroll
    for (int t = 0; t < kVec; ++t)
      if (e + t < V) dz[e + t] = uint16_t(out[t >> 1] >> (16 * (t & 1)));
  }
  if constexpr (kDbg) {
#pragma unroll
    for (int t = 0; t < kVec; ++t)
      if (e + t < V) dz32[e + t] = g32[t];
  }
}

// Cross-entropy and KL parts of a group (probability target): alpha's part
// sum min(q, p), sum p, and the loss part sum p (M + ln L - z) = -sum p ln q
// (KL adds p ln p per token), each in fp32 over the group and fp64 across
// groups; mlnl = fl32(M + ln L) of the row. Tokens at or past V (z = -inf,
// p = 0) add nothing (with kVecOk a group lies wholly inside or past the
// row). kDz: the group's dz as well, fma(q, c_p, -(p c_p)) from the same q,
// in fp32 (g32) and as bf16 pairs (out): the gradient q (sum p)/N - p/N
// whenever the row's coefficient (sum p)/N rounds to the same binary32 as
// c_p = 1/N (times fl32(1/T) in both).
constexpr float kLn2f = 0.693147180559945309f;

template <bool kVecOk, bool kDz = false>
__device__ __forceinline__ void grp_xent(const u32x4& g, const u32x4& pa, const u32x4& pb, int e,
                                         int V, float cz, const RowStats& rs, float mlnl, bool kl,
                                         double& al, double& sp, double& sl, float c_p = 0.f,
                                         float* g32 = nullptr, u32x4* out = nullptr) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  float a = 0.f, b = 0.f, c = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const bool in = kVecOk ? (e < V) : (e + j < V);
    const float x = zelem(g, j);
    const float p = pelem(pa, pb, j);
    const float q = qval(x, cz, rs.nm, rs.inv_l);
    a += fminf(q, p);
    b += p;
    // -ln q, plus ln p for KL (from the hardware base-2 logarithm; p below
    // the smallest normal float takes ln p as 0: its term is below 1e-36)
    float t = mlnl - x;
    if (kl) t += (p >= 1.17549435e-38f) ? __builtin_amdgcn_logf(p) * kLn2f : 0.f;
    c += in ? p * t : 0.f;
    if constexpr (kDz) {
      g32[j] = __builtin_fmaf(q, c_p, -(p * c_p));
      if (j & 1) {
        const bf16x2 v = __builtin_convertvector(f32x2{g32[j - 1], g32[j]}, bf16x2);
        (*out)[j >> 1] = __builtin_bit_cast(uint32_t, v);
      }
    }
  }
  al += (double)a;
  sp += (double)b;
  sl += (double)c;
}

// A buffer resource over the n bytes at p (raw, 32-bit data: the resource
// word 0x00020000 of gfx9 parts). The hardware drops a store through it at
// an offset at or past n, so a group that lies wholly past the end of a
// half needs no branch around its store; a branch there per group makes the
// compiler spill the unrolled pass over p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, int(n), 0x00020000);
}
constexpr int kBufNt = 2;  // the nontemporal bit of a buffer store

// Half statistics from per-thread partials: every thread's m is already the
// block maximum; l is summed over the block.
struct HalfStats {
  float m;   // maximum of the half (-inf for a half past the end of the row)
  double l;  // sum of 2^((z - m) log2 e) over the half
};

__device__ __forceinline__ double block_sum1(double v, Shared& sh) {
  double u0 = 0.0, u1 = 0.0;
  block_sum3(v, u0, u1, sh);
  return v;
}

// Row statistics from the two halves' statistics, half 0 first: M = max,
// L = sum_h l_h 2^((m_h - M) log2 e) in fp64 (a half of maximum -inf weighs
// l_h * 0, which keeps a NaN). Both halves and the last launch call this
// with the same values, so they agree bit for bit.
__device__ __forceinline__ RowStats combine_halves(float m0, double l0, float m1, double l1,
                                                   float c) {
  const float M = fmaxf(m0, m1);
  const double w0 = (m0 == -INFINITY) ? l0 * 0.0
                                      : l0 * (double)__builtin_amdgcn_exp2f((m0 - M) * c);
  const double w1 = (m1 == -INFINITY) ? l1 * 0.0
                                      : l1 * (double)__builtin_amdgcn_exp2f((m1 - M) * c);
  RowStats r;
  r.nm = (M == -INFINITY) ? 0.f : -(M * c);
  r.inv_l = float(1.0 / (w0 + w1));
  return r;
}

// fp64 value from two consecutive 32-bit words (low half first).
__device__ __forceinline__ double word_f64(const uint32_t* w, int i) {
  return __longlong_as_double((long long)((uint64_t(w[i + 1]) << 32) | w[i]));
}

// Row statistics from the words [first, first + 3) of a row's two half
// slots, laid out slot after slot from `w`.
__device__ __forceinline__ RowStats row_stats_from(const uint32_t* w, int first, float c) {
  return combine_halves(__uint_as_float(w[first]), word_f64(w, first + 1),
                        __uint_as_float(w[kSlotWords + first]), word_f64(w, kSlotWords + first + 1),
                        c);
}


// M + ln L of a row in fp64 (natural log; the row's maximum raw logit and
// sum of e^(z - M), from the words [first, first + 3) of its two half slots
// in the same arithmetic as combine_halves): -ln q(v) = M + ln L - z(v).
__device__ __forceinline__ double row_mlnl_from(const uint32_t* w, int first, float c) {
  const float m0 = __uint_as_float(w[first]), m1 = __uint_as_float(w[kSlotWords + first]);
  const double l0 = word_f64(w, first + 1), l1 = word_f64(w, kSlotWords + first + 1);
  const float M = fmaxf(m0, m1);
  const double w0 = (m0 == -INFINITY) ? l0 * 0.0
                                      : l0 * (double)__builtin_amdgcn_exp2f((m0 - M) * c);
  const double w1 = (m1 == -INFINITY) ? l1 * 0.0
                                      : l1 * (double)__builtin_amdgcn_exp2f((m1 - M) * c);
  return (double)M + log(w0 + w1);
}

__device__ __forceinline__ void f64_words(double v, uint32_t& lo, uint32_t& hi) {
  const uint64_t bits = uint64_t(__double_as_longlong(v));
  lo = uint32_t(bits);
  hi = uint32_t(bits >> 32);
}

// Block-wide poll of words [first, first + count) of nslots consecutive half
// slots starting at `slots`; word k of slot s lands in
// sh.words[s * kSlotWords + k]. Returns whether all were fresh within the
// spin limit. Every thread calls it.
__device__ __forceinline__ bool poll_slots(uint64_t* slots, int nslots, int first, int count,
                                           uint32_t tag, int spin_limit, Shared& sh) {
  const int n = nslots * count;
  for (int i = threadIdx.x; i < n; i += kThreads) sh.have[i] = 0;
  __syncthreads();
  for (int round = 0;; ++round) {
    int missing = 0;
    for (int i = threadIdx.x; i < n; i += kThreads) {
      if (!sh.have[i]) {
        const int s = i / count, k = first + (i - s * count);
        const uint64_t w = tag_load(slots + s * kSlotWords + k);
        if (uint32_t(w >> 32) == tag) {
          sh.words[s * kSlotWords + k] = uint32_t(w);
          sh.have[i] = 1;
        } else {
          missing = 1;
        }
      }
    }
    if (!__syncthreads_or(missing)) return true;
    if (round >= spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// ------------------------------------------------------------------ branch scalars

// Branch scalars (thread 0, fp64) from the branch's parts in sh.words laid
// out [k][h][kSlotWords] with the parts at offset 4: alpha_k, S_k, S'_k are
// the sums of the two halves (half 0 first). Writes sh.coef for row j
// ((G_j/N) S'_j where q < p, -(G_j/N) S_j elsewhere), alpha[row], and the
// branch loss when j == 0.
__device__ __forceinline__ void branch_scalars(const Args& a, int n, int j, size_t row,
                                               Shared& sh) {
  const int W = a.W;
  if (threadIdx.x == 0) {
    auto part = [&](int k, int which) {
      const int b0 = (k * 2) * kSlotWords + 4 + 2 * which;
      const int b1 = (k * 2 + 1) * kSlotWords + 4 + 2 * which;
      return word_f64(sh.words, b0) + word_f64(sh.words, b1);
    };
    double loss_n = 0.0, g = 0.0;
    if (a.objective == LVTV_OBJ_CE || a.objective == LVTV_OBJ_KL) {
      // parts (alpha, sum p, the half's loss part): the branch loss is the
      // sum of the rows' parts; dz = q (sum p)/N - p/N
      for (int k = 0; k < W; ++k) loss_n += part(k, 2);
      sh.coef[0] = part(j, 1) / double(a.N) * a.inv_t;
      sh.coef[1] = 1.0 / double(a.N) * a.inv_t;
      a.alpha[row] = float(part(j, 0));
      if (j == 0) a.branch_loss[n] = loss_n;
    } else if (a.objective == LVTV_OBJ_STEP_TV) {
      // sum_k (1 - alpha_k); d/dalpha_j = -1
      for (int k = 0; k < W; ++k) loss_n += 1.0 - part(k, 0);
      g = -1.0 / double(a.N);
    } else {
      double run = 1.0, before = 1.0;
      for (int k = 0; k < W; ++k) {
        if (k == j) before = run;
        run *= part(k, 0);
        loss_n -= run;
      }
      double suffix = 1.0;  // R_{W-1} = 1, R_k = 1 + alpha_{k+1} R_{k+1}
      for (int k = W - 2; k >= j; --k) suffix = 1.0 + part(k + 1, 0) * suffix;
      g = -before * suffix / double(a.N);
    }
    if (a.objective == LVTV_OBJ_E2E_TV || a.objective == LVTV_OBJ_STEP_TV) {
      sh.coef[0] = g * part(j, 2) * a.inv_t;   // S'_j
      sh.coef[1] = -g * part(j, 1) * a.inv_t;  // S_j
      a.alpha[row] = float(part(j, 0));
      if (j == 0) a.branch_loss[n] = loss_n;
    }
  }
  __syncthreads();
}

// dz of one group of 8 tokens, bf16 (nearest even), from z, the group's mask
// bits and the row's coefficients. kDbg: the fp32 values before rounding go
// to dz32 as well.
template <bool kVecOk, bool kDbg>
__device__ __forceinline__ void dz_group(const u32x4& zv, uint32_t bits8, int e, int V,
                                         float cz, const RowStats& rs, float c_below,
                                         float c_above, uint16_t* dz, float* dz32) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  u32x4 out;
  float g32[kVec];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float v2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int jj = 2 * h + t;
      const bool below = (bits8 >> jj) & 1u;
      v2[t] = qval(zelem(zv, jj), cz, rs.nm, rs.inv_l) * (below ? c_below : c_above);
      g32[jj] = v2[t];
    }
    const bf16x2 b = __builtin_convertvector(f32x2{v2[0], v2[1]}, bf16x2);
    out[h] = __builtin_bit_cast(uint32_t, b);
  }
  store_dz<kVecOk, kDbg>(out, g32, e, V, dz, dz32);
}

// CE / KL dz of one group, bf16 (nearest even): fma(q, c_q, -(p c_p)) with
// c_q = (sum p)/N and c_p = 1/N (each times the chain factor fl32(1/T)).
template <bool kVecOk, bool kDbg>
__device__ __forceinline__ void dz_xent_group(const u32x4& zv, const u32x4& pa, const u32x4& pb,
                                              int e, int V, float cz, const RowStats& rs,
                                              float c_q, float c_p, uint16_t* dz, float* dz32) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  u32x4 out;
  float g32[kVec];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float v2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int jj = 2 * h + t;
      const float q = qval(zelem(zv, jj), cz, rs.nm, rs.inv_l);
      v2[t] = __builtin_fmaf(q, c_q, -(pelem(pa, pb, jj) * c_p));
      g32[jj] = v2[t];
    }
    const bf16x2 b = __builtin_convertvector(f32x2{v2[0], v2[1]}, bf16x2);
    out[h] = __builtin_bit_cast(uint32_t, b);
  }
  store_dz<kVecOk, kDbg>(out, g32, e, V, dz, dz32);
}

__device__ __forceinline__ uint32_t mask_bits(const uint32_t (&mask)[kMaskWords], int g) {
  return (mask[(g * kVec) / 32] >> ((g * kVec) % 32)) & 0xffu;
}

// Statistics of half h of a target logits row, streamed once from memory:
// per thread a running maximum m and sum l = sum 2^(t c - m c) over batches
// of groups (the sum rescaled when the maximum moves), then the block's
// maximum M_h and sum over threads of l 2^((m - M_h) c). The half workgroups
// and the last launch call this with the same thread layout, so they agree
// bit for bit.
template <bool kVecOk>
__device__ __forceinline__ HalfStats target_half_stats(const uint16_t* t, int V, int hv, int h,
                                                       float c, Shared& sh) {
  float m = -INFINITY;
  double l = 0.0;
  const int tb = opaque(group_elem(hv, h, 0));
  const int ve = half_end(V, hv, h);
  const int ng = half_groups(V, hv, h);
#pragma unroll 1
  for (int g0 = 0; g0 < ng; g0 += kPBatch) {
    u32x4 x[kPBatch];
#pragma unroll
    for (int i = 0; i < kPBatch; ++i)
      if (g0 + i < kZG) x[i] = load_z<kVecOk>(t, ve, opaque(tb) + (g0 + i) * kTile);
    float bm = m;
#pragma unroll
    for (int i = 0; i < kPBatch; ++i)
      if (g0 + i < kZG) bm = grp_max(x[i], bm);
    if (bm > m) {
      l = (m == -INFINITY) ? 0.0 : l * (double)__builtin_amdgcn_exp2f((m - bm) * c);
      m = bm;
    }
    const float nm = (m == -INFINITY) ? 0.f : -(m * c);
#pragma unroll
    for (int i = 0; i < kPBatch; ++i)
      if (g0 + i < kZG) l += (double)grp_expsum(x[i], c, nm);
    __builtin_amdgcn_sched_barrier(0);
  }
  const float M = block_max(m, sh);
  const double w = (m == -INFINITY) ? l * 0.0 : l * (double)__builtin_amdgcn_exp2f((m - M) * c);
  return HalfStats{M, block_sum1(w, sh)};
}

// Publishes half statistics in words [first, first + 3) of a half slot.
__device__ __forceinline__ void publish_stats(uint64_t* slot, int first, uint32_t tag,
                                              const HalfStats& hs) {
  uint32_t lo, hi;
  f64_words(hs.l, lo, hi);
  tag_store(slot + first, tag, __float_as_uint(hs.m));
  tag_store(slot + first + 1, tag, lo);
  tag_store(slot + first + 2, tag, hi);
}

// ------------------------------------------------------------------ half-row kernel

// Row modes: two workgroups a row, groups past a half's end skipped
// (kSplit); the same when both halves reach every group, V near the
// largest, so the tests of the group count fold away (kSplitAll); one
// workgroup a row, V <= kWholeMaxV (kWhole).
constexpr int kSplit = 0, kSplitAll = 1, kWhole = 2;

template <bool kVecOk, bool kLogits, bool kDbg, bool kXent, int kMode>
__device__ __forceinline__ void half_body(const Args& a) {
  static_assert(!(kLogits && kXent), "CE and KL take a probability target here");
  __shared__ Shared sh;
  __shared__ u32x4 zl[kZL][kThreads];
  const int W = a.W, V = a.V;
  // uniform coordinates, kept in scalar registers
  constexpr bool whole = kMode == kWhole;
  const int r = __builtin_amdgcn_readfirstlane(whole ? int(blockIdx.x) : int(blockIdx.x) >> 1);
  const int h = __builtin_amdgcn_readfirstlane(whole ? 0 : int(blockIdx.x) & 1);
  const int hv = half_len(V, whole);
  const int n = __builtin_amdgcn_readfirstlane(r / W);
  const int j = __builtin_amdgcn_readfirstlane(r - n * W);
  const size_t row = size_t(r);
  const uint16_t* z = a.z + row * V;
  const float* p = kLogits ? nullptr : a.p + row * V;
  const uint16_t* t = kLogits ? a.t + row * V : nullptr;
  const float c = a.c;
  const uint32_t tag = tag_from_epoch(read_epoch(a.ctl));
  uint64_t* slot = a.words + (row * 2 + h) * kSlotWords;

  // 1. this half of z into the held copy
  Held zg;
  zg.lds = zl;
  const int ve = half_end(V, hv, h);  // this half's tokens end here
  // groups past ng are skipped (uniform tests)
  const int ng = kMode == kSplitAll ? kZG : half_groups(V, hv, h);
  {
    const int tb = opaque(group_elem(hv, h, 0));
    u32x4 tmp[kZL];
#pragma unroll
    for (int g = 0; g < kZL; ++g)
      if (g < ng) tmp[g] = load_z<kVecOk>(z, ve, tb + g * kTile);
#pragma unroll
    for (int g = kZL; g < kZG; ++g)
      if (g < ng) zg.r[g - kZL] = load_z<kVecOk>(z, ve, tb + g * kTile);
#pragma unroll
    for (int g = 0; g < kZL; ++g)
      if (g < ng) zl[g][threadIdx.x] = tmp[g];
  }

  // 2. half statistics, swapped with the other half
  float m = -INFINITY;
#pragma unroll
  for (int g = 0; g < kZG; ++g)
    if (g < ng) m = grp_max(zg.get(g), m);
  launder(zg);
  m = block_max(m, sh);
  const float nm0 = (m == -INFINITY) ? 0.f : -(m * c);
  double l = 0.0;
#pragma unroll
  for (int g = 0; g < kZG; ++g)
    if (g < ng) l += (double)grp_expsum(zg.get(g), c, nm0);
  launder(zg);
  l = block_sum1(l, sh);
  if (threadIdx.x == 0) {
    publish_stats(slot, 0, tag, HalfStats{m, l});
    // a whole row: the empty second half's words, as its workgroup would
    // have published them
    if constexpr (whole) publish_stats(slot + kSlotWords, 0, tag, HalfStats{-INFINITY, 0.0});
  }
  if constexpr (kLogits) {
    const HalfStats ht = target_half_stats<kVecOk>(t, V, hv, h, c, sh);
    launder(zg);
    if (threadIdx.x == 0) {
      publish_stats(slot, kTStatWord, tag, ht);
      if constexpr (whole)
        publish_stats(slot + kSlotWords, kTStatWord, tag, HalfStats{-INFINITY, 0.0});
    }
  }
  uint64_t* rslots = a.words + row * 2 * kSlotWords;
  if (!poll_slots(rslots, 2, 0, kStatWords, tag, a.spin_limit, sh) ||
      (kLogits && !poll_slots(rslots, 2, kTStatWord, kStatWords, tag, a.spin_limit, sh))) {
    if (threadIdx.x == 0) tag_store(a.unfinished + row, tag, 1u);
    return;
  }
  const RowStats rs = row_stats_from(sh.words, 0, c);
  const RowStats ts = kLogits ? row_stats_from(sh.words, kTStatWord, c) : RowStats{0.f, 0.f};

  // 3. one pass over this half of p (or of the target logits)
  double al = 0.0, sb = 0.0, sa = 0.0;
  uint32_t mask[kMaskWords];
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) mask[w] = 0u;
  const int tbp = opaque(group_elem(hv, h, 0));
  const bool kl = a.objective == LVTV_OBJ_KL;
  const float mlnl = kXent ? float(row_mlnl_from(sh.words, 0, c)) : 0.f;
  // CE / KL on 16-byte aligned rows: dz is written in this pass with the
  // coefficient of a target row that sums to one (step 5 rewrites it where
  // that is not so)
  constexpr bool kDz = kXent && kVecOk;
  const float c_one = kXent ? float(1.0 / double(a.N) * a.inv_t) : 0.f;
  // (resources that end where this half's tokens end: a group past them
  // holds zeros, which must not land on the other half's tokens)
  const __amdgpu_buffer_rsrc_t dzr = row_rsrc(a.dz + row * V, uint32_t(ve) * 2u);
  const __amdgpu_buffer_rsrc_t dz32r =
      kDbg ? row_rsrc(a.dz32 + row * V, uint32_t(ve) * 4u) : row_rsrc(a.dz, 0u);
  constexpr int kB = kPBatch;
#pragma unroll
  for (int g0 = 0; g0 < kZG; g0 += kB) {
    u32x4 pa[kB], pb[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (g0 + i < kZG && g0 + i < ng) {
        if constexpr (kLogits)
          pa[i] = load_z<kVecOk>(t, ve, opaque(tbp) + (g0 + i) * kTile);
        else
          load_p<kVecOk>(p, ve, opaque(tbp) + (g0 + i) * kTile, pa[i], pb[i]);
      }
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (g0 + i < kZG && g0 + i < ng) {
        const int g = g0 + i;
        if constexpr (kXent) {
          // al, sum p (in sb), the loss part (in sa); dz
          float g32[kVec];
          u32x4 out;
          grp_xent<kVecOk, kDz>(zg.get(g), pa[i], pb[i], opaque(tbp) + g * kTile, ve, c, rs,
                                mlnl, kl, al, sb, sa, c_one, g32, &out);
          if constexpr (kDz) {
            const int e = opaque(tbp) + g * kTile;
            __builtin_amdgcn_raw_buffer_store_b128(out, dzr, e * 2, 0, kBufNt);
            if constexpr (kDbg) {
              __builtin_amdgcn_raw_buffer_store_b128(
                  u32x4{__float_as_uint(g32[0]), __float_as_uint(g32[1]), __float_as_uint(g32[2]),
                        __float_as_uint(g32[3])},
                  dz32r, e * 4, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(
                  u32x4{__float_as_uint(g32[4]), __float_as_uint(g32[5]), __float_as_uint(g32[6]),
                        __float_as_uint(g32[7])},
                  dz32r, e * 4 + 16, 0, 0);
            }
          }
        } else {
          const uint32_t bits =
              grp_overlap<kLogits>(zg.get(g), pa[i], pb[i], c, rs, ts, al, sb, sa);
          mask[(g * kVec) / 32] |= bits << ((g * kVec) % 32);
        }
      }
    // keep the next batch's loads behind this batch's arithmetic
    __builtin_amdgcn_sched_barrier(0);
  }
  launder(zg);
  block_sum3(al, sb, sa, sh);

  // 4. the branch's parts
  if (threadIdx.x == 0) {
    const double v[3] = {al, sb, sa};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      uint32_t lo, hi;
      f64_words(v[i], lo, hi);
      tag_store(slot + 4 + 2 * i, tag, lo);
      tag_store(slot + 5 + 2 * i, tag, hi);
      if constexpr (whole) {  // the empty second half's parts: 0.0
        tag_store(slot + kSlotWords + 4 + 2 * i, tag, 0u);
        tag_store(slot + kSlotWords + 5 + 2 * i, tag, 0u);
      }
    }
  }
  if (!poll_slots(a.words + size_t(n) * W * 2 * kSlotWords, 2 * W, 4, kPartWords, tag,
                  a.spin_limit, sh)) {
    if (threadIdx.x == 0) tag_store(a.unfinished + row, tag, 1u);
    return;
  }
  branch_scalars(a, n, j, row, sh);
  const float c_below = float(sh.coef[0]);
  const float c_above = float(sh.coef[1]);

  // 5. dz of this half from the held copy and the mask (CE / KL: written in
  //    step 3 unless the row is not 16-byte aligned or its coefficient
  //    (sum p)/N is not c_one's binary32; then from p, streamed again)
  uint16_t* dz = a.dz + row * V;
  float* dz32 = kDbg ? a.dz32 + row * V : nullptr;
  const int tbd = opaque(group_elem(hv, h, 0));
  if constexpr (kXent) {
    if (kDz && c_below == c_above && !a.reread) return;  // c_above is c_one
#pragma unroll
    for (int g0 = 0; g0 < kZG; g0 += kB) {
      u32x4 pa[kB], pb[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (g0 + i < kZG && g0 + i < ng)
          load_p<kVecOk>(p, ve, opaque(tbd) + (g0 + i) * kTile, pa[i], pb[i]);
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (g0 + i < kZG && g0 + i < ng)
          dz_xent_group<kVecOk, kDbg>(zg.get(g0 + i), pa[i], pb[i], opaque(tbd) + (g0 + i) * kTile,
                                      ve, c, rs, c_below, c_above, dz, dz32);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int g = 0; g < kZG; ++g) {
      if (g < ng)
        dz_group<kVecOk, kDbg>(zg.get(g), mask_bits(mask, g), opaque(tbd) + g * kTile, ve, c, rs,
                               c_below, c_above, dz, dz32);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ------------------------------------------------------------------ repair

// Statistics of half h of a row, streamed from memory (same steps and
// reductions as a half workgroup).
template <bool kVecOk>
__device__ __forceinline__ HalfStats stream_half_stats(const uint16_t* z, int V, int hv, int h,
                                                       float c, Shared& sh) {
  float m = -INFINITY;
  const int ve = half_end(V, hv, h);
  const int ng = half_groups(V, hv, h);
#pragma unroll 1
  for (int g = 0; g < ng; ++g) m = grp_max(load_z<kVecOk>(z, ve, group_elem(hv, h, g)), m);
  m = block_max(m, sh);
  const float nm0 = (m == -INFINITY) ? 0.f : -(m * c);
  double l = 0.0;
#pragma unroll 1
  for (int g = 0; g < ng; ++g)
    l += (double)grp_expsum(load_z<kVecOk>(z, ve, group_elem(hv, h, g)), c, nm0);
  l = block_sum1(l, sh);
  return HalfStats{m, l};
}

// The target's group at token e: 8 probabilities in (pa, pb), or (kLogits)
// 8 bf16 logits in pa.
template <bool kVecOk, bool kLogits>
__device__ __forceinline__ void load_target(const Args& a, size_t row, int e, int ve, u32x4& pa,
                                            u32x4& pb) {
  if constexpr (kLogits) {
    pa = load_z<kVecOk>(a.t + row * a.V, ve, e);
    pb = pa;
  } else {
    load_p<kVecOk>(a.p + row * a.V, ve, e, pa, pb);
  }
}

// Parts of half h of a row, streamed from memory.
template <bool kVecOk, bool kLogits>
__device__ __forceinline__ void stream_half_parts(const Args& a, size_t row, int h,
                                                  const RowStats& rs, const RowStats& ts,
                                                  double& al, double& sb, double& sa, Shared& sh) {
  al = sb = sa = 0.0;
  const uint16_t* z = a.z + row * a.V;
  const int hv = half_len(a.V, a.whole);
  const int ve = half_end(a.V, hv, h);
  const int ng = half_groups(a.V, hv, h);
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    const int e = group_elem(hv, h, g);
    u32x4 pa, pb;
    load_target<kVecOk, kLogits>(a, row, e, ve, pa, pb);
    (void)grp_overlap<kLogits>(load_z<kVecOk>(z, ve, e), pa, pb, a.c, rs, ts, al, sb, sa);
  }
  block_sum3(al, sb, sa, sh);
}

// CE / KL parts of half h of a row, streamed from memory (same per-group
// steps, order and reductions as a half workgroup): alpha's part, sum p and
// the half's part of the row's loss.
template <bool kVecOk>
__device__ __forceinline__ void stream_half_xent(const Args& a, size_t row, int h,
                                                 const RowStats& rs, float mlnl, double& al,
                                                 double& sp, double& part, Shared& sh) {
  const bool kl = a.objective == LVTV_OBJ_KL;
  al = sp = part = 0.0;
  const uint16_t* z = a.z + row * a.V;
  const int hv = half_len(a.V, a.whole);
  const int ve = half_end(a.V, hv, h);
  const int ng = half_groups(a.V, hv, h);
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    const int e = group_elem(hv, h, g);
    u32x4 pa, pb;
    load_target<kVecOk, false>(a, row, e, ve, pa, pb);
    grp_xent<kVecOk>(load_z<kVecOk>(z, ve, e), pa, pb, e, ve, a.c, rs, mlnl, kl, al, sp, part);
  }
  block_sum3(al, sp, part, sh);
}

// Writes half statistics into words [first, first + 3) of slot s of a
// branch's word copy.
__device__ __forceinline__ void put_stats(uint32_t* bw, int s, int first, const HalfStats& hs) {
  uint32_t lo, hi;
  f64_words(hs.l, lo, hi);
  bw[s * kSlotWords + first] = __float_as_uint(hs.m);
  bw[s * kSlotWords + first + 1] = lo;
  bw[s * kSlotWords + first + 2] = hi;
}

// A row a half left unfinished in this call. Every half workgroup has
// stopped, so every word that will ever be published is there; what is
// missing is recomputed from the inputs with the same steps and reductions.
// Then both halves' dz are written (the mask recomputed from z and p). Every
// thread of the block calls it.
template <bool kVecOk, bool kLogits, bool kDbg, bool kXent>
__device__ __forceinline__ void repair_row(const Args& a, int row, uint32_t tag, Shared& sh,
                                           uint32_t* bw) {
  const int W = a.W, V = a.V;
  const float c = a.c;
  {
    const int n = row / W, j = row - n * W;
    // the branch's published words (stale ones recomputed below)
    uint64_t* base = a.words + size_t(n) * W * 2 * kSlotWords;
    for (int i = threadIdx.x; i < W * 2 * kSlotWords; i += kThreads)
      bw[i] = uint32_t(tag_load(base + i));
    __syncthreads();
    // per half slot: 1 = draft statistics, 2 = parts, 4 = target statistics
    // are fresh
    for (int s = threadIdx.x; s < 2 * W; s += kThreads) {
      bool st = true, pt = true, tt = true;
      for (int k = 0; k < kStatWords; ++k)
        st &= uint32_t(tag_load(base + s * kSlotWords + k) >> 32) == tag;
      for (int k = 4; k < 4 + kPartWords; ++k)
        pt &= uint32_t(tag_load(base + s * kSlotWords + k) >> 32) == tag;
      for (int k = kTStatWord; k < kTStatWord + kStatWords; ++k)
        tt &= uint32_t(tag_load(base + s * kSlotWords + k) >> 32) == tag;
      sh.have[s] = uint8_t((st ? 1 : 0) | (pt ? 2 : 0) | ((tt || !kLogits) ? 4 : 0));
    }
    __syncthreads();
    for (int k = 0; k < W; ++k) {
      const size_t rk = size_t(n) * W + k;
      const uint16_t* zk = a.z + rk * V;
      // statistics of both halves
      for (int hh = 0; hh < 2; ++hh) {
        const int s = 2 * k + hh;
        if (!(sh.have[s] & 1)) {
          const HalfStats hs = stream_half_stats<kVecOk>(zk, V, half_len(V, a.whole), hh, c, sh);
          __syncthreads();
          if (threadIdx.x == 0) put_stats(bw, s, 0, hs);
          __syncthreads();
        }
        if (!(sh.have[s] & 4)) {
          const HalfStats hs =
              target_half_stats<kVecOk>(a.t + rk * V, V, half_len(V, a.whole), hh, c, sh);
          __syncthreads();
          if (threadIdx.x == 0) put_stats(bw, s, kTStatWord, hs);
          __syncthreads();
        }
      }
      const RowStats rs = row_stats_from(bw + 2 * k * kSlotWords, 0, c);
      const RowStats ts =
          kLogits ? row_stats_from(bw + 2 * k * kSlotWords, kTStatWord, c) : RowStats{0.f, 0.f};
      for (int hh = 0; hh < 2; ++hh) {
        const int s = 2 * k + hh;
        if (!(sh.have[s] & 2)) {
          double x, y, w;
          if constexpr (kXent)
            stream_half_xent<kVecOk>(a, rk, hh, rs,
                                     float(row_mlnl_from(bw + 2 * k * kSlotWords, 0, c)), x, y,
                                     w, sh);
          else
            stream_half_parts<kVecOk, kLogits>(a, rk, hh, rs, ts, x, y, w, sh);
          __syncthreads();
          if (threadIdx.x == 0) {
            const double v[3] = {x, y, w};
            for (int i = 0; i < 3; ++i) {
              uint32_t lo, hi;
              f64_words(v[i], lo, hi);
              bw[s * kSlotWords + 4 + 2 * i] = lo;
              bw[s * kSlotWords + 5 + 2 * i] = hi;
            }
          }
          __syncthreads();
        }
      }
    }
    for (int i = threadIdx.x; i < W * 2 * kSlotWords; i += kThreads) sh.words[i] = bw[i];
    __syncthreads();
    branch_scalars(a, n, j, size_t(row), sh);
    const float c_below = float(sh.coef[0]);
    const float c_above = float(sh.coef[1]);
    const RowStats rs = row_stats_from(bw + 2 * j * kSlotWords, 0, c);
    const RowStats ts =
        kLogits ? row_stats_from(bw + 2 * j * kSlotWords, kTStatWord, c) : RowStats{0.f, 0.f};
    const uint16_t* z = a.z + size_t(row) * V;
    uint16_t* dz = a.dz + size_t(row) * V;
    for (int hh = 0; hh < 2; ++hh) {
      const int hv = half_len(V, a.whole);
      const int ve = half_end(V, hv, hh);
      const int ng = half_groups(V, hv, hh);
#pragma unroll 1
      for (int g = 0; g < ng; ++g) {
        const int e = group_elem(hv, hh, g);
        const u32x4 zv = load_z<kVecOk>(z, ve, e);
        u32x4 pa, pb;
        load_target<kVecOk, kLogits>(a, size_t(row), e, ve, pa, pb);
        if constexpr (kXent) {
          dz_xent_group<kVecOk, kDbg>(zv, pa, pb, e, ve, c, rs, c_below, c_above, dz,
                                      kDbg ? a.dz32 + size_t(row) * V : nullptr);
        } else {
          double x = 0.0, y = 0.0, w = 0.0;
          const uint32_t bits = grp_overlap<kLogits>(zv, pa, pb, c, rs, ts, x, y, w);
          dz_group<kVecOk, kDbg>(zv, bits, e, ve, c, rs, c_below, c_above, dz,
                                 kDbg ? a.dz32 + size_t(row) * V : nullptr);
        }
      }
    }
    __syncthreads();
  }
}

template <bool kVecOk, bool kLogits, bool kDbg, bool kXent, int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
loss_halves(Args a) {
  half_body<kVecOk, kLogits, kDbg, kXent, kMode>(a);
}

__device__ __forceinline__ int block_min(int v, Shared& sh) {
  v = wmin(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.imin[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = sh.imin[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = min(r, sh.imin[w]);
  return r;
}

// The call's last launch, one workgroup; every half workgroup has stopped.
// (1) Rows a half left unfinished are completed, in row order: the flags of
// up to 32 rows per thread are read at once, so the usual case (no flag) costs
// one round of loads. (2) The loss is the mean of the branch losses, summed
// in a fixed order. (3) The call epoch advances.
template <bool kVecOk, bool kLogits, bool kDbg, bool kXent>
__global__ __launch_bounds__(kThreads) void loss_finish(Args a) {
  __shared__ Shared sh;
  __shared__ uint32_t bw[LVTV_MAX_W * 2 * kSlotWords];  // a branch's words
  __shared__ double sd[kWaves];
  const uint32_t tag = tag_from_epoch(read_epoch(a.ctl));
  const int rows = a.N * a.W;
  for (int r0 = 0; r0 < rows; r0 += kThreads * 32) {
    uint32_t mine = 0;  // bit i: row r0 + tid + i * kThreads is flagged
#pragma unroll 8
    for (int i = 0; i < 32; ++i) {
      const int row = r0 + int(threadIdx.x) + i * kThreads;
      if (row < rows && uint32_t(tag_load(a.unfinished + row) >> 32) == tag) mine |= 1u << i;
    }
    while (__syncthreads_or(mine != 0)) {
      const int cand = mine ? r0 + int(threadIdx.x) + __builtin_ctz(mine) * kThreads : INT_MAX;
      const int row = block_min(cand, sh);
      if (cand == row) mine &= mine - 1u;
      repair_row<kVecOk, kLogits, kDbg, kXent>(a, row, tag, sh, bw);
    }
  }
  const int per = (a.N + kThreads - 1) / kThreads;
  double x = 0.0;
  for (int n = threadIdx.x * per; n < min(a.N, (int(threadIdx.x) + 1) * per); ++n)
    x += a.branch_loss[n];
  x = wsum(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sd[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) t += sd[w];
    a.loss[0] = float(t / double(a.N));
    __hip_atomic_store(&a.ctl->epoch, read_epoch(a.ctl) + 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
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
  off = align256(off + sizeof(uint64_t) * size_t(N) * W * 2 * kSlotWords);
  L.off_unfinished = off;
  off = align256(off + sizeof(uint64_t) * size_t(N) * W);
  L.off_branch = off;
  off = align256(off + sizeof(double) * size_t(N));
  L.total = off;
  return L;
}

// Zeroes the call's tagged words and row flags (16-byte stores; the region
// is a multiple of 256 bytes), so that nothing a workspace held before the
// call (an earlier call of either op, or garbage) can read as fresh: a zero
// word never carries a tag.
__global__ __launch_bounds__(256) void clear_words(u32x4* w, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    w[i] = u32x4{0u, 0u, 0u, 0u};
}

template <bool kDbg, bool kXent, int kMode>
void launch_halves(const Args& a, bool vec_ok, bool logits, unsigned rows, hipStream_t stream) {
  const unsigned blocks = kMode == kWhole ? rows : 2 * rows;
  auto halves = vec_ok ? (logits ? loss_halves<true, true, kDbg, false, kMode>
                                 : loss_halves<true, false, kDbg, kXent, kMode>)
                       : (logits ? loss_halves<false, true, kDbg, false, kMode>
                                 : loss_halves<false, false, kDbg, kXent, kMode>);
  hipLaunchKernelGGL(halves, dim3(blocks), dim3(kThreads), 0, stream, a);
}

template <bool kDbg, bool kXent>
hipError_t launch_kernels(const Args& a, bool vec_ok, bool logits, unsigned rows,
                          hipStream_t stream) {
  auto finish = vec_ok ? (logits ? loss_finish<true, true, kDbg, false>
                                 : loss_finish<true, false, kDbg, kXent>)
                       : (logits ? loss_finish<false, true, kDbg, false>
                                 : loss_finish<false, false, kDbg, kXent>);
  const int hv = half_len(a.V, a.whole);
  if (a.whole)
    launch_halves<kDbg, kXent, kWhole>(a, vec_ok, logits, rows, stream);
  else if (half_groups(a.V, hv, 0) == kZG && half_groups(a.V, hv, 1) == kZG)
    launch_halves<kDbg, kXent, kSplitAll>(a, vec_ok, logits, rows, stream);
  else
    launch_halves<kDbg, kXent, kSplit>(a, vec_ok, logits, rows, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finish, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool kDbg>
hipError_t launch_all(const Args& a, bool vec_ok, bool logits, unsigned rows, size_t clear_bytes,
                      void* clear_base, hipStream_t stream) {
  const size_t n16 = clear_bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(clear_words, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<u32x4*>(clear_base), n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool xent = a.objective == LVTV_OBJ_CE || a.objective == LVTV_OBJ_KL;
  return xent ? launch_kernels<kDbg, true>(a, vec_ok, false, rows, stream)
              : launch_kernels<kDbg, false>(a, vec_ok, logits, rows, stream);
}

}  // namespace

bool logits_supported() { return true; }

bool xent_supported(bool logits) { return !logits; }

bool applicable(int N, int W, int V) {
  // rows of at least one group: a row that is not 16-byte aligned is read
  // 16 bytes at a time, always inside the row
  return V >= kVec && V <= kMaxV && size_t(N) * W * 2 < (size_t(1) << 31);
}

size_t workspace_bytes(int N, int W, int V) {
  (void)V;
  return make_layout(N, W).total;
}

hipError_t run(const LossCall& c, void* workspace, hipStream_t stream) {
  const bool xent = c.objective == LVTV_OBJ_CE || c.objective == LVTV_OBJ_KL;
  if (xent && !xent_supported(c.t != nullptr)) return hipErrorInvalidValue;
  const Layout L = make_layout(c.N, c.W);
  Args a;
  a.z = c.z;
  a.p = c.p;
  a.t = c.t;
  a.c = c.c;
  a.inv_t = c.inv_t;
  a.N = c.N;
  a.W = c.W;
  a.V = c.V;
  a.objective = c.objective;
  a.spin_limit = c.spin_limit;
  // rows that fit one workgroup's held copy go to one workgroup each: half
  // as many workgroups, each with twice the tokens and no partner to wait for
  a.whole = c.V <= kWholeMaxV ? 1 : 0;
  a.reread = c.reread ? 1 : 0;
  a.alpha = c.alpha;
  a.dz = c.dz;
  a.dz32 = c.dz32;
  a.loss = c.loss;
  char* ws = static_cast<char*>(workspace);
  a.ctl = workspace_ctl(workspace);
  a.words = reinterpret_cast<uint64_t*>(ws + L.off_words);
  a.unfinished = reinterpret_cast<uint64_t*>(ws + L.off_unfinished);
  a.branch_loss = reinterpret_cast<double*>(ws + L.off_branch);
  const unsigned rows = unsigned(size_t(c.N) * c.W);
  const bool logits = c.t != nullptr;
  const size_t clear_bytes = L.off_branch - L.off_words;
  return c.dz32 ? launch_all<true>(a, c.vec_ok, logits, rows, clear_bytes, ws + L.off_words, stream)
                : launch_all<false>(a, c.vec_ok, logits, rows, clear_bytes, ws + L.off_words,
                                    stream);
}

}  // namespace lf
}  // namespace lvtv
