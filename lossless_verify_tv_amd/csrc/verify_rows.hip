// spec_verify for gfx950: two launches per call on the caller's stream.
//
//   1. verify_rows      one workgroup per (request b, position k <= K_b):
//                       the pair of target row k and draft row k (k < K_b),
//                       or the target row alone (the bonus row k = K_b).
//                       Sampling (T_b > 0): pass 1 streams both rows once
//                       and keeps an online maximum and sum of exponentials
//                       per thread; the last tiles of the rows stay in
//                       registers. The block combines these into the row
//                       statistics. Pass 2 walks the rows back to front (the
//                       held tiles first, the rest from the cache hierarchy,
//                       where pass 1 just left them) and forms p and q, the
//                       overlap alpha_k = sum min(p, q) and, per 512-token
//                       chunk, the residual mass sum max(0, p - q) (for the
//                       bonus row the mass of p). Greedy (T_b = 0): one pass
//                       taking the argmax of both rows.
//   2. verify_finalize  one workgroup per request: status checks, alpha, the
//                       accept scan with Philox uniforms and the inverse-CDF
//                       draw (chunk from the chunk masses, token from an fp64
//                       evaluation inside the chunk), emitted tokens.
//
// Cites (page title, section): "Reading Qwen Bebop and DeepSeek DSpark",
// "Formulas" (acceptance min(1, p/q); overlap sum min(p, q) = 1 - d_TV);
// "Speculative Decoding and MTP" survey, section 2 (ordered acceptance, the
// bonus token from p_{K+1}), section 3 (residual max(0, p - q)/Z), section 4
// (one temperature for p and q; greedy compares with the target argmax),
// section 21 (acceptance and residual sampling on the GPU, no per-cycle
// host sync).
//
// Arithmetic. Scaled logits s = fl32(x * fl32(1/T)) (x itself at T = 1).
// Exponentials are base 2: a row's statistics are R = fl32(M * log2 e), M the
// row maximum of s, and L = sum_v 2^(s_v log2 e - R), both fp32, so that
// p(v) = 2^(s_v log2 e - R) / L. The finalize step evaluates that formula in
// fp64 for the accept ratios and inside the chosen chunk.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/lvtv.h"
#include "device_common.hpp"
#include "fused_common.hpp"
#include "philox.hpp"
#include "wave_dpp.hpp"

namespace lvtv {
namespace vr {
namespace {

constexpr int kThreads = 512;                 // threads per workgroup
constexpr int kWaves = kThreads / kWave;      // 8
constexpr int kTile = kThreads * kVec;        // 4096 tokens: 8 per thread
constexpr int kChunk = kWave * kVec;          // 512 tokens: one wave's part of a tile
constexpr int kBatch = 4;                     // tiles whose loads are in flight together
constexpr int kCand = 4096;                   // tokens a truncation's LDS list holds
constexpr int kListNC = 1024;                 // chunks a row may have for the list path
constexpr float kL2E = 1.44269504088896340736f;

// Tiles kept in registers between the passes (the last ones of the row).
template <int kDtype>
constexpr int hold_tiles() {
  return kDtype == 1 ? 3 : 2;
}

// Per (request, position) results of the row kernel.
struct RowOut {
  float Rt, Lt;   // target row: R and L (greedy: max value, unused)
  float Rd, Ld;   // draft row
  float alpha;    // sum min(p, q) (greedy: unused)
  int32_t nan;    // greedy: bit 0 target row, bit 1 draft row held a NaN
  // greedy: the argmaxes of the target and the draft row; sampling draft
  // rows: the bits of the accept ratio p(y_k) / q(y_k) in fp64 (low word in
  // arg_t), see set_ratio
  int32_t arg_t;
  int32_t arg_d;
};
static_assert(sizeof(RowOut) == 32, "row record is 32 bytes");

__device__ __forceinline__ void set_ratio(RowOut& o, double r) {
  const uint64_t u = uint64_t(__double_as_longlong(r));
  o.arg_t = int32_t(uint32_t(u));
  o.arg_d = int32_t(uint32_t(u >> 32));
}

__device__ __forceinline__ double get_ratio(const RowOut& o) {
  return __longlong_as_double((long long)((uint64_t(uint32_t(o.arg_d)) << 32) | uint32_t(o.arg_t)));
}

// Tokens a row keeps after top-k / top-p truncation: with d the order key of
// a token's scaled logit s (larger s, smaller d), token v is kept iff
// d < key, or d == key and v <= idx (equal s are kept in token order). R and
// L are the row's statistics over the kept tokens in the row kernel's
// convention (R = fl32(max s log2 e), L = sum 2^(s log2 e - R)), so that the
// row kernel needs a single pass over a truncated row.
struct KeepRow {
  uint32_t key;
  int32_t idx;
  float R, L;
};
struct KeepPair {
  KeepRow t, d;  // the target row and the draft row of one position
};
static_assert(sizeof(KeepPair) == 32, "keep record is 32 bytes");

// Order key of a scaled logit: unsigned order of the key is descending order
// of s (-0 and +0 share one key).
__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = (s == 0.f) ? 0u : __float_as_uint(s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

__device__ __forceinline__ float key_value(uint32_t d) {
  const uint32_t asc = ~d;
  return __uint_as_float((asc & 0x80000000u) ? (asc & 0x7fffffffu) : ~asc);
}

__device__ __forceinline__ bool keeps(const KeepRow& k, float s, int v) {
  const uint32_t d = desc_key(s);
  return d < k.key || (d == k.key && v <= k.idx);
}

struct Args {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* kreq;
  const float* temp;
  const uint64_t* seed;
  int B, Kmax, V;
  int n_tiles;  // tiles per row
  int NC;       // chunks per row (n_tiles * kWaves)
  int32_t* acc_len;
  int32_t* out_tokens;
  float* alpha;
  int32_t* status;
  RowOut* rows;  // one per target row: [B][Kmax+1] (padded) or [total_rows] (packed)
  float* chunk;  // [target rows][NC]
  // Packed layout (toff == nullptr for the padded one): request b owns the
  // target rows [toff[b], toff[b+1]), K_b = toff[b+1] - toff[b] - 1, and the
  // draft rows, draft tokens and alphas from toff[b] - b on.
  const int32_t* toff;
  const int32_t* rowmap;     // [total_rows]: the request of each target row (-1: bad offsets)
  const int32_t* packed_ok;  // the offsets tile [0, total_rows) (written by packed_map)
  int total_rows;
  // top-k / top-p truncation (null when off)
  const int32_t* top_k;  // [B]
  const float* top_p;    // [B]
  KeepPair* keep;        // one per target row, written by trunc_rows
  // Ids of the tokens a target row keeps, when the selection had them all
  // in its LDS list (klen > 0, in no particular order; 0: the row kernel
  // streams the row). Written by trunc_rows for every row it truncates.
  int32_t* klen;   // [target rows]
  int32_t* klist;  // [target rows][kCand]
};

__device__ __forceinline__ KeepRow keep_all() { return KeepRow{0xffffffffu, INT_MAX, 0.f, 0.f}; }

__device__ __forceinline__ bool temperature_ok(float t) { return (t >= 0.f) && !isinf(t); }

// Index of request b's target row k, and of its draft row k (also the index
// of draft token k and of alpha k), in either layout.
__device__ __forceinline__ int64_t target_row(const Args& a, int b, int k) {
  return a.toff ? int64_t(a.toff[b]) + k : int64_t(b) * (a.Kmax + 1) + k;
}

__device__ __forceinline__ int64_t draft_row(const Args& a, int b, int k) {
  return a.toff ? int64_t(a.toff[b]) - b + k : int64_t(b) * a.Kmax + k;
}

template <int kDtype>
__device__ __forceinline__ const void* row_ptr(const Args& a, int b, bool target, int k) {
  constexpr int kSize = kDtype == 1 ? 2 : 4;
  const int64_t row = target ? target_row(a, b, k) : draft_row(a, b, k);
  return static_cast<const char*>(target ? a.target : a.draft) + row * int64_t(a.V) * kSize;
}

// ------------------------------------------------------------------ groups of 8 tokens

// One thread's 8 tokens of one row in a tile, as raw bits: bf16 packed two
// per register, fp32 one per register.
template <int kDtype>
struct Grp {
  u32x4 q[kDtype == 1 ? 1 : 2];
};

template <int kDtype>
__device__ __forceinline__ float gelem(const Grp<kDtype>& g, int j) {
  if constexpr (kDtype == 1) {
    const uint32_t w = g.q[0][j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(g.q[j >> 2][j & 3]);
  }
}

template <int kDtype>
__device__ __forceinline__ void fill_grp(Grp<kDtype>& g) {
  const uint32_t fill = kDtype == 1 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
  for (int q = 0; q < (kDtype == 1 ? 1 : 2); ++q) g.q[q] = u32x4{fill, fill, fill, fill};
}

// First token of this thread's group in tile t.
__device__ __forceinline__ int tile_elem(int t) { return t * kTile + threadIdx.x * kVec; }

// Load of the group starting at token e of a row; tokens at or beyond V read
// as -inf. With kVecOk (16-byte aligned rows, V % 8 == 0) a group is wholly
// inside the row or wholly past its end: past-the-end groups are loaded from
// the row's first group (so the load needs no branch) and then overwritten.
// kNt: streaming (nontemporal) load, for data that is not read again.
template <int kDtype, bool kVecOk, bool kNt>
__device__ __forceinline__ void load_grp(const void* row, int V, int e, Grp<kDtype>& g) {
  if constexpr (kVecOk) {
    const uint32_t off = uint32_t(e < V ? e : 0) * (kDtype == 1 ? 2u : 4u);
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + off);
    if constexpr (kNt) {
      g.q[0] = __builtin_nontemporal_load(p);
      if constexpr (kDtype == 0) g.q[1] = __builtin_nontemporal_load(p + 1);
    } else {
      g.q[0] = p[0];
      if constexpr (kDtype == 0) g.q[1] = p[1];
    }
  } else if constexpr (kDtype == 1) {
    const uint16_t* p = static_cast<const uint16_t*>(row);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = (e + 2 * h < V) ? p[e + 2 * h] : 0xff80u;
      const uint32_t hi = (e + 2 * h + 1 < V) ? p[e + 2 * h + 1] : 0xff80u;
      g.q[0][h] = lo | (hi << 16);
    }
  } else {
    const uint32_t* p = static_cast<const uint32_t*>(row);
#pragma unroll
    for (int h = 0; h < 8; ++h) g.q[h >> 2][h & 3] = (e + h < V) ? p[e + h] : 0xff800000u;
  }
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void mask_grp(Grp<kDtype>& g, int e, int V) {
  if constexpr (kVecOk) {
    if (e >= V) fill_grp(g);
  }
}

// Keeps the compiler from carrying values derived from a group (unpacked or
// exponentiated tokens) from one pass to the next instead of recomputing
// them from the raw bits: that would need several times the registers.
template <int kDtype>
__device__ __forceinline__ void launder(Grp<kDtype>& g) {
#pragma unroll
  for (int q = 0; q < (kDtype == 1 ? 1 : 2); ++q) asm volatile("" : "+v"(g.q[q]));
}

// ------------------------------------------------------------------ block reductions

struct Shared {
  float f[kWaves][4];
  int i[kWaves][4];
  double d[kWaves];
  unsigned long long u[kWaves];
  float yx[2];  // sampling draft rows: the target and draft logits at y_k
  int y;        // y_k, or -1 when it is out of range
};

// Block-wide combination of per-thread online statistics of two rows. A
// thread holds its maximum raw logit m and l = sum 2^(x c - fl32(m c)) over
// its tokens, c = fl32(log2(e) / T) > 0; the block gets the row maximum M,
// R = fl32(M c) and L = sum_threads l 2^(fl32(m c) - R). A thread that saw
// only -inf (m = -inf) contributes l * 0.
__device__ __forceinline__ void block_online(float c, float& m0, float& l0, float& m1, float& l1,
                                             Shared& sh) {
  const float M0w = wmax(m0), M1w = wmax(m1);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.f[threadIdx.x / kWave][0] = M0w;
    sh.f[threadIdx.x / kWave][1] = M1w;
  }
  __syncthreads();
  float M0 = sh.f[0][0], M1 = sh.f[0][1];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    M0 = fmaxf(M0, sh.f[w][0]);
    M1 = fmaxf(M1, sh.f[w][1]);
  }
  const float w0 = (m0 == -INFINITY) ? l0 * 0.f : l0 * __builtin_amdgcn_exp2f(m0 * c - M0 * c);
  const float w1 = (m1 == -INFINITY) ? l1 * 0.f : l1 * __builtin_amdgcn_exp2f(m1 * c - M1 * c);
  const float S0w = wsum(w0), S1w = wsum(w1);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.f[threadIdx.x / kWave][2] = S0w;
    sh.f[threadIdx.x / kWave][3] = S1w;
  }
  __syncthreads();
  float S0 = sh.f[0][2], S1 = sh.f[0][3];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    S0 += sh.f[w][2];
    S1 += sh.f[w][3];
  }
  m0 = M0;
  l0 = S0;
  m1 = M1;
  l1 = S1;
}

__device__ __forceinline__ float block_sum1(float v, Shared& sh) {
  v = wsum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.f[threadIdx.x / kWave][0] = v;
  __syncthreads();
  float r = sh.f[0][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += sh.f[w][0];
  return r;
}

// fp64 probability of token v, logit x, under a row's (R, L), base-2
// convention; 0 for a token the row's truncation drops.
__device__ __forceinline__ double prob64_of(float x, int v, float inv_t, bool unit, float R,
                                           float L, const KeepRow& kr) {
  const float s = scale_logit(x, inv_t, unit);
  if (!keeps(kr, s, v)) return 0.0;
  return exp2((double)s * (double)kL2E - (double)R) / (double)L;
}

// The accept ratio p(y)/q(y) of a draft row, in fp64; q(y) = 0 encodes as
// +inf when p(y) > 0 (accept) and 0 otherwise (reject).
__device__ __forceinline__ double accept_ratio(double p, double q) {
  return (q == 0.0) ? (p > 0.0 ? INFINITY : 0.0) : p / q;
}

// ------------------------------------------------------------------ sampling rows
//
// Exponents are formed as fma(x, c, -r) with x the raw logit and
// c = fl32(log2(e) * fl32(1/T)) (log2(e) itself at T = 1): the temperature
// and the base change in one rounding. Within the kernel this differs from
// the canonical 2^(fl32(x / T) log2 e) by about one ulp of the exponent; the
// accept ratios and the in-chunk draw use the canonical form in fp64.

// Online statistics of a batch of groups of one row: the batch maximum of
// the raw logits first, one rescale of the running sum, then the
// exponentials against the new maximum.
template <int kDtype, int kN>
__device__ __forceinline__ void online_batch(const Grp<kDtype> (&g)[kN], float c, float& m,
                                             float& l) {
  float bm = m;
#pragma unroll
  for (int n = 0; n < kN; ++n)
#pragma unroll
    for (int j = 0; j < kVec; ++j) bm = fmaxf(bm, gelem(g[n], j));
  if (bm > m) {
    l = (m == -INFINITY) ? 0.f : l * __builtin_amdgcn_exp2f(m * c - bm * c);
    m = bm;
  }
  // a -inf maximum: every token so far is -inf and contributes 0
  const float nr = (m == -INFINITY) ? 0.f : -(m * c);
#pragma unroll
  for (int n = 0; n < kN; ++n)
#pragma unroll
    for (int j = 0; j < kVec; ++j) l += __builtin_amdgcn_exp2f(__builtin_fmaf(gelem(g[n], j), c, nr));
}

// Pass 2 over one tile: p = 2^(x c - Rt'), q = 2^(x c - Rd') with the row
// sums folded into the references (R' = R + log2 L), alpha and this wave's
// chunk mass (lane 0 writes it).
template <int kDtype, bool kPair>
__device__ __forceinline__ void overlap_tile(const Grp<kDtype>& gt, const Grp<kDtype>& gd,
                                             float c, float nrt, float nrd, float& sa,
                                             float* chunk_row, int t) {
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(gelem(gt, j), c, nrt));
    if constexpr (kPair) {
      const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(gelem(gd, j), c, nrd));
      const float mn = fminf(p, q);
      sa += mn;
      r += p - mn;
    } else {
      r += p;
    }
  }
  const float cm = wsum(r);
  if ((threadIdx.x & (kWave - 1)) == 0) chunk_row[t * kWaves + threadIdx.x / kWave] = cm;
}

// The group of the last, partial tile: loaded where it lies inside the row,
// -inf elsewhere.
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void load_tail(const void* row, int V, int t, Grp<kDtype>& g) {
  const int e = tile_elem(t);
  if constexpr (kVecOk) {
    if (e < V)
      load_grp<kDtype, kVecOk, true>(row, V, e, g);
    else
      fill_grp(g);
  } else {
    load_grp<kDtype, kVecOk, true>(row, V, e, g);
  }
}

// Tokens of a group (first token e) that the row's truncation drops read as
// -inf from here on. The kept prefix ends at the token of scaled logit sk and
// id idx: a token is kept iff s > sk, or s == sk and its id is at most idx
// (the order key's order, compared as floats).
template <int kDtype>
__device__ __forceinline__ void apply_keep(Grp<kDtype>& g, int e, float sk, int idx, float inv_t,
                                           bool unit) {
  if constexpr (kDtype == 1) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t w = g.q[0][h];
      const float s0 = scale_logit(__uint_as_float(w << 16), inv_t, unit);
      const float s1 = scale_logit(__uint_as_float(w & 0xffff0000u), inv_t, unit);
      const bool k0 = s0 > sk || (s0 == sk && e + 2 * h <= idx);
      const bool k1 = s1 > sk || (s1 == sk && e + 2 * h + 1 <= idx);
      const uint32_t drop = (k0 ? 0u : 0x0000ffffu) | (k1 ? 0u : 0xffff0000u);
      g.q[0][h] = (w & ~drop) | (0xff80ff80u & drop);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float s = scale_logit(__uint_as_float(g.q[j >> 2][j & 3]), inv_t, unit);
      const bool kp = s > sk || (s == sk && e + j <= idx);
      if (!kp) g.q[j >> 2][j & 3] = 0xff800000u;
    }
  }
}

template <int kDtype, bool kVecOk, bool kPair, bool kTrunc>
__device__ __forceinline__ void sampling_row(const Args& a, int b, int k, float T, Shared& sh) {
  constexpr int kHold = hold_tiles<kDtype>();
  const int V = a.V;
  const int nfull = V / kTile;                  // tiles wholly inside the row
  const bool tail = nfull * kTile < V;          // a last, partial tile
  const int held = nfull < kHold ? nfull : kHold;
  const int nstream = nfull - held;             // tiles [0, nstream) are streamed twice
  const float c = (T == 1.f) ? kL2E : __fmul_rn(kL2E, __fdiv_rn(1.f, T));
  const void* trow = row_ptr<kDtype>(a, b, true, k);
  const void* drow = kPair ? row_ptr<kDtype>(a, b, false, k) : nullptr;
  const float inv_t = __fdiv_rn(1.f, T);
  const bool unit = (T == 1.f);
  KeepPair kp{keep_all(), keep_all()};
  if constexpr (kTrunc) kp = a.keep[target_row(a, b, k)];
  // a row that keeps every token is left as it is
  const bool cut_t = kTrunc && kp.t.key != keep_all().key;
  const bool cut_d = kTrunc && kPair && kp.d.key != keep_all().key;
  const float sk_t = key_value(kp.t.key), sk_d = key_value(kp.d.key);
  // the draft token's logits, for the accept ratio the row's statistics
  // give at the end (an out-of-range token faults the request later)
  if constexpr (kPair) {
    if (threadIdx.x == 0) {
      const int y = a.tokens[draft_row(a, b, k)];
      const bool ok = y >= 0 && y < V;
      sh.y = ok ? y : -1;
      sh.yx[0] = ok ? load1<kDtype>(trow, y) : 0.f;
      sh.yx[1] = ok ? load1<kDtype>(drow, y) : 0.f;
    }
  }
  // the row record: statistics, alpha and (draft rows) the accept ratio
  auto write_row = [&](float Rt_, float Lt_, float Rd_, float Ld_, float alpha_) {
    if (threadIdx.x == 0) {
      RowOut o{Rt_, Lt_, Rd_, Ld_, alpha_, 0, -1, -1};
      if constexpr (kPair) {
        if (sh.y >= 0)
          set_ratio(o, accept_ratio(prob64_of(sh.yx[0], sh.y, inv_t, unit, Rt_, Lt_, kp.t),
                                    prob64_of(sh.yx[1], sh.y, inv_t, unit, Rd_, Ld_, kp.d)));
      }
      a.rows[target_row(a, b, k)] = o;
    }
  };
  // drops the truncated tokens of a loaded group of tile t
  auto mk = [&](Grp<kDtype>& gt, Grp<kDtype>& gd, int tt) {
    if constexpr (kTrunc) {
      if (cut_t) apply_keep<kDtype>(gt, tile_elem(tt), sk_t, kp.t.idx, inv_t, unit);
      if constexpr (kPair)
        if (cut_d) apply_keep<kDtype>(gd, tile_elem(tt), sk_d, kp.d.idx, inv_t, unit);
    }
  };

  if constexpr (kTrunc) {
    if (cut_t && (!kPair || cut_d)) {
      // A truncated row (pair): the selection kernel has the statistics of
      // the kept tokens, so one pass over the row does.
      const float Rt = kp.t.R, Lt = kp.t.L;
      const float Rd = kPair ? kp.d.R : 0.f, Ld = kPair ? kp.d.L : 1.f;
      const float nrt = float(-((double)Rt + log2((double)Lt)));
      const float nrd = kPair ? float(-((double)Rd + log2((double)Ld))) : 0.f;
      float* chunk_row = a.chunk + size_t(target_row(a, b, k)) * a.NC;
      const int nlist = a.klen[target_row(a, b, k)];
      if (nlist > 0 && nlist <= kCand && a.NC <= kListNC) {
        // The target row's kept tokens are listed: only they carry p > 0,
        // so alpha and the residual chunk masses are sums over them, each
        // token's p and q formed as the streaming pass forms them (a token
        // the draft row drops has q = 0). The sums are exact in 2^-62
        // fixed point, so the list's order does not show.
        __shared__ unsigned long long cacc[kListNC];
        for (int i = threadIdx.x; i < a.NC; i += kThreads) cacc[i] = 0;
        __syncthreads();
        const int32_t* lst = a.klist + size_t(target_row(a, b, k)) * kCand;
        uint64_t al = 0;
        for (int i = threadIdx.x; i < nlist; i += kThreads) {
          const int v = lst[i];
          if (v < 0 || v >= V) continue;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(load1<kDtype>(trow, v), c, nrt));
          float r = p;
          if constexpr (kPair) {
            const float xd = load1<kDtype>(drow, v);
            const float q = keeps(kp.d, scale_logit(xd, inv_t, unit), v)
                                ? __builtin_amdgcn_exp2f(__builtin_fmaf(xd, c, nrd))
                                : 0.f;
            const float mn = fminf(p, q);
            al += (uint64_t)(mn * 0x1p62f);
            r = p - mn;
          }
          atomicAdd(&cacc[v / kChunk], (unsigned long long)(r * 0x1p62f));
        }
        __syncthreads();
        for (int i = threadIdx.x; i < a.NC; i += kThreads)
          chunk_row[i] = (float)((double)cacc[i] * 0x1p-62);
        float alpha = 0.f;
        if constexpr (kPair) {
#pragma unroll
          for (int o = kWave / 2; o > 0; o >>= 1) al += __shfl_xor(al, o, kWave);
          if ((threadIdx.x & (kWave - 1)) == 0) sh.u[threadIdx.x / kWave] = al;
          __syncthreads();
          uint64_t tot = 0;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) tot += sh.u[w];
          alpha = (float)((double)tot * 0x1p-62);
        }
        write_row(Rt, Lt, Rd, Ld, alpha);
        return;
      }
      float sa = 0.f;
      int t = 0;
      for (; t + kBatch <= nfull; t += kBatch) {
        Grp<kDtype> gt[kBatch], gd[kBatch];
#pragma unroll
        for (int n = 0; n < kBatch; ++n) {
          load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t + n), gt[n]);
          if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t + n), gd[n]);
        }
#pragma unroll
        for (int n = 0; n < kBatch; ++n) {
          mk(gt[n], gd[n], t + n);
          overlap_tile<kDtype, kPair>(gt[n], gd[n], c, nrt, nrd, sa, chunk_row, t + n);
        }
      }
      for (; t < nfull; ++t) {
        Grp<kDtype> gt, gd;
        load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t), gt);
        if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t), gd);
        mk(gt, gd, t);
        overlap_tile<kDtype, kPair>(gt, gd, c, nrt, nrd, sa, chunk_row, t);
      }
      if (tail) {
        Grp<kDtype> gt, gd;
        load_tail<kDtype, kVecOk>(trow, V, nfull, gt);
        if constexpr (kPair) load_tail<kDtype, kVecOk>(drow, V, nfull, gd);
        mk(gt, gd, nfull);
        overlap_tile<kDtype, kPair>(gt, gd, c, nrt, nrd, sa, chunk_row, nfull);
      }
      const float alpha = kPair ? block_sum1(sa, sh) : 0.f;
      write_row(Rt, Lt, Rd, Ld, alpha);
      return;
    }
  }

  // ---- pass 1: streamed full tiles, held full tiles, the partial tile
  float mt = -INFINITY, lt = 0.f, md = -INFINITY, ld = 0.f;
  int t = 0;
  for (; t + kBatch <= nstream; t += kBatch) {
    Grp<kDtype> gt[kBatch], gd[kBatch];
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t + n), gt[n]);
      if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t + n), gd[n]);
      mk(gt[n], gd[n], t + n);
    }
    online_batch<kDtype, kBatch>(gt, c, mt, lt);
    if constexpr (kPair) online_batch<kDtype, kBatch>(gd, c, md, ld);
  }
  for (; t < nstream; ++t) {
    Grp<kDtype> gt[1], gd[1];
    load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t), gt[0]);
    if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t), gd[0]);
    mk(gt[0], gd[0], t);
    online_batch<kDtype, 1>(gt, c, mt, lt);
    if constexpr (kPair) online_batch<kDtype, 1>(gd, c, md, ld);
  }
  Grp<kDtype> ht[kHold], hd[kHold], tt[1], td[1];
  if (held == kHold) {
#pragma unroll
    for (int h = 0; h < kHold; ++h) {
      load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(nstream + h), ht[h]);
      if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(nstream + h), hd[h]);
      mk(ht[h], hd[h], nstream + h);
    }
    online_batch<kDtype, kHold>(ht, c, mt, lt);
    if constexpr (kPair) online_batch<kDtype, kHold>(hd, c, md, ld);
  } else {
#pragma unroll
    for (int h = 0; h < kHold; ++h)
      if (h < held) {
        Grp<kDtype> g1[1], g2[1];
        load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(nstream + h), g1[0]);
        if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(nstream + h), g2[0]);
        mk(g1[0], g2[0], nstream + h);
        online_batch<kDtype, 1>(g1, c, mt, lt);
        if constexpr (kPair) online_batch<kDtype, 1>(g2, c, md, ld);
        ht[h] = g1[0];
        hd[h] = g2[0];
      }
  }
  if (tail) {
    load_tail<kDtype, kVecOk>(trow, V, nfull, tt[0]);
    if constexpr (kPair) load_tail<kDtype, kVecOk>(drow, V, nfull, td[0]);
    mk(tt[0], td[0], nfull);
    online_batch<kDtype, 1>(tt, c, mt, lt);
    if constexpr (kPair) online_batch<kDtype, 1>(td, c, md, ld);
  }
#pragma unroll
  for (int h = 0; h < kHold; ++h) {
    launder(ht[h]);
    if constexpr (kPair) launder(hd[h]);
  }
  launder(tt[0]);
  if constexpr (kPair) launder(td[0]);
  block_online(c, mt, lt, md, ld, sh);
  const float Rt = (mt == -INFINITY) ? -INFINITY : mt * c;
  const float Rd = (md == -INFINITY) ? -INFINITY : md * c;
  // references with the row sums folded in: p = 2^(x c - (R + log2 L))
  const float nrt = float(-((double)Rt + log2((double)lt)));
  const float nrd = kPair ? float(-((double)Rd + log2((double)ld))) : 0.f;

  // ---- pass 2: the partial tile, the held tiles, the rest back to front
  float* chunk_row = a.chunk + size_t(target_row(a, b, k)) * a.NC;
  float sa = 0.f;
  if (tail) overlap_tile<kDtype, kPair>(tt[0], td[0], c, nrt, nrd, sa, chunk_row, nfull);
#pragma unroll
  for (int h = kHold - 1; h >= 0; --h)
    if (h < held) overlap_tile<kDtype, kPair>(ht[h], hd[h], c, nrt, nrd, sa, chunk_row, nstream + h);
  t = nstream;
  for (; t >= kBatch; t -= kBatch) {
    Grp<kDtype> gt[kBatch], gd[kBatch];
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t - 1 - n), gt[n]);
      if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t - 1 - n), gd[n]);
      mk(gt[n], gd[n], t - 1 - n);
    }
#pragma unroll
    for (int n = 0; n < kBatch; ++n)
      overlap_tile<kDtype, kPair>(gt[n], gd[n], c, nrt, nrd, sa, chunk_row, t - 1 - n);
  }
  for (; t > 0; --t) {
    Grp<kDtype> gt, gd;
    load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t - 1), gt);
    if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t - 1), gd);
    mk(gt, gd, t - 1);
    overlap_tile<kDtype, kPair>(gt, gd, c, nrt, nrd, sa, chunk_row, t - 1);
  }
  const float alpha = kPair ? block_sum1(sa, sh) : 0.f;
  write_row(Rt, lt, kPair ? Rd : 0.f, kPair ? ld : 1.f, alpha);
}

// ------------------------------------------------------------------ greedy rows

// Largest value, lowest index holding it (the group's tokens are visited in
// increasing index, so a later equal value never replaces an earlier one),
// NaN flagged and left out.
template <int kDtype>
__device__ __forceinline__ void argmax_grp(const Grp<kDtype>& g, int e, int V, float& bv, int& bi,
                                           int& nan) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float v = gelem(g, j);
    nan |= (v != v);
    if (e + j < V && v > bv) {
      bv = v;
      bi = e + j;
    }
  }
}

__device__ __forceinline__ ArgMax block_argmax2(ArgMax x, Shared& sh, int slot) {
  x = wargmax(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.f[threadIdx.x / kWave][slot] = x.v;
    sh.i[threadIdx.x / kWave][slot] = x.i;
    sh.i[threadIdx.x / kWave][slot + 2] = x.nan;
  }
  __syncthreads();
  ArgMax r{sh.f[0][slot], sh.i[0][slot], sh.i[0][slot + 2]};
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    r = argmax_combine(r, ArgMax{sh.f[w][slot], sh.i[w][slot], sh.i[w][slot + 2]});
  return r;
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void greedy_row(const Args& a, int b, int k, bool pair, Shared& sh) {
  const int V = a.V;
  const void* trow = row_ptr<kDtype>(a, b, true, k);
  const void* drow = pair ? row_ptr<kDtype>(a, b, false, k) : nullptr;
  // a first maximum of -inf is still a valid argmax (lowest index of the
  // row); INT_MAX marks "none yet"
  float vt = -INFINITY, vd = -INFINITY;
  int it = INT_MAX, id = INT_MAX, nt = 0, nd = 0;
  // One tile of loads per step: with every row pair of the call resident at
  // once there are enough loads in flight chip-wide, and batches of 2-8
  // tiles measured slower (58-62 against 56 us per call).
  for (int t = 0; t < a.n_tiles; ++t) {
    const int e = tile_elem(t);
    Grp<kDtype> gt, gd;
    load_grp<kDtype, kVecOk, true>(trow, V, e, gt);
    if (pair) load_grp<kDtype, kVecOk, true>(drow, V, e, gd);
    mask_grp<kDtype, kVecOk>(gt, e, V);
    argmax_grp(gt, e, V, vt, it, nt);
    if (pair) {
      mask_grp<kDtype, kVecOk>(gd, e, V);
      argmax_grp(gd, e, V, vd, id, nd);
    }
  }
  // a thread whose tokens are all -inf reports its first in-range index
  if (it == INT_MAX && tile_elem(0) < V) it = tile_elem(0);
  if (id == INT_MAX && tile_elem(0) < V) id = tile_elem(0);
  const ArgMax bt = block_argmax2(ArgMax{vt, it, nt}, sh, 0);
  const ArgMax bd = block_argmax2(ArgMax{vd, id, nd}, sh, 1);
  if (threadIdx.x == 0) {
    RowOut o;
    o.Rt = bt.v;
    o.Lt = 0.f;
    o.Rd = pair ? bd.v : 0.f;
    o.Ld = 0.f;
    o.alpha = 0.f;
    o.arg_t = bt.i;
    o.arg_d = pair ? bd.i : -1;
    o.nan = (bt.nan ? 1 : 0) | (pair && bd.nan ? 2 : 0);
    a.rows[target_row(a, b, k)] = o;
  }
}

// ------------------------------------------------------------------ row kernel

template <int kDtype, bool kVecOk, bool kTrunc>
__device__ __forceinline__ void rows_body(const Args& a) {
  __shared__ Shared sh;
  int b, k, kb;
  if (a.toff) {
    b = a.rowmap[blockIdx.x];
    if (b < 0) return;  // the offsets are bad: every request is faulted
    k = int(blockIdx.x) - a.toff[b];
    kb = a.toff[b + 1] - a.toff[b] - 1;
  } else {
    b = blockIdx.x / (a.Kmax + 1);
    k = blockIdx.x - b * (a.Kmax + 1);
    kb = a.kreq[b];
  }
  const float T = a.temp[b];
  if (!(kb >= 0 && kb <= a.Kmax && temperature_ok(T)) || k > kb) return;
  if (T == 0.f) {
    greedy_row<kDtype, kVecOk>(a, b, k, k < kb, sh);
  } else if (k < kb) {
    sampling_row<kDtype, kVecOk, true, kTrunc>(a, b, k, T, sh);
  } else {
    sampling_row<kDtype, kVecOk, false, kTrunc>(a, b, k, T, sh);
  }
}

template <bool kVecOk, bool kTrunc>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
verify_rows_bf16(Args a) {
  rows_body<1, kVecOk, kTrunc>(a);
}

template <bool kVecOk, bool kTrunc>
__global__ __launch_bounds__(kThreads) void verify_rows_f32(Args a) {
  rows_body<0, kVecOk, kTrunc>(a);
}

// ------------------------------------------------------------------ truncation
//
// trunc_rows finds, for each used row of a sampling request, the prefix of
// the row's tokens (scaled logit s descending, then token id) that top-k and
// then top-p keep, and stores its last token as a KeepRow. Every pass
// streams the row (a re-read gains nothing from the caches here). Bins are
// first-level LDS histograms over the distance below a reference value in
// 1/32-nat bins, floor((ref - s) 32) (the last bin takes everything further
// down); they follow the order of s and spread the LDS atomics of clustered
// logits over many addresses.
//
// With top-k on, one or two passes in the common case:
//   1. the row maximum M (and faults: such rows are left whole), and R0,
//      the largest s of the row's first tile. For top_k <= 512 the pass
//      lists (order key and token id, in LDS) every token down to a bin
//      below R0 chosen from the first tile's counts, so that about 16 top_k
//      tokens (fewer for a larger top_k) are expected; if it lists at least
//      top_k tokens (and no more than the list holds) it is complete. For a
//      larger top_k the pass counts tokens per bin below R0 (tokens above R0
//      share bin 0) and a block scan finds the bin where the count reaches
//      top_k;
//   2. in that case, if every token down to that bin fits the LDS list
//      (4096 tokens), a second pass gathers them.
// On the list, top-k's boundary and then top-p's, over the tokens top-k
// keeps, are resolved with fixed-point masses below M: for at most 256
// tokens in the bins down to top_k's by ranking each against all the others
// and summing masses in rank order, else by radix selection on the 32-bit
// order key, 10 bits a level, then on the token id among equal keys. The
// ids of the tokens kept are written out for the row kernel, which then
// needs no pass over the row.
// When the list cannot hold them, and for top-p alone, the bins are redone
// below M:
//   2'. token counts for top-k, or fixed-point masses for top-p alone; a
//      block scan picks the bin where the running count reaches top_k, or
//      the running mass top_p times the total;
//   3'. the tokens of the open bins are gathered and resolved as above (with
//      top-k on, all bins down to top-k's own when they fit, their masses
//      taken from the list; else top-k's bin and top-p's, after a mass pass).
// A bin with more tokens than LDS holds is refined by further passes over
// the row instead (a level a pass, then one pass to split equal keys).
//
// Masses are e^(s - M) 2^E truncated to integers (E = 63 - bits(V), so that a
// row's total cannot pass 2^63), formed to about two binary32 ulps whatever
// s - M is and summed exactly in 64 bits: the sums are deterministic, and
// within about 2.4e-7 of the exact ones relative to the kept total.

constexpr int kRes = 32;       // first-level bins per nat below the reference
constexpr int kNB1 = 2048;     // first-level bins
constexpr int kNB = 1024;      // buckets of a refinement level
constexpr int kRankMax = 256;  // lists short enough to rank by comparing every pair
constexpr float kL2ELo = 1.925963033e-8f;  // log2(e) - fl32(log2(e))

struct TruncShared {
  uint32_t cnt1[kNB1];
  unsigned long long mass1[kNB1];
  uint32_t ckey[kCand];
  int32_t cidx[kCand];
  uint32_t cnt[kNB];
  unsigned long long mass[kNB];
  alignas(16) uint32_t vmin[kNB];
  alignas(16) uint32_t vmax[kNB];
  unsigned long long part[kWaves][2];
  unsigned long long r64[2];
  int32_t r32;
  uint32_t ncand;
  uint32_t nrank;
  float fmax[kWaves];
};

// e^(s - M) 2^E truncated, `scale` = 2^E; s <= M, both finite (or s = -inf:
// 0). The difference is split exactly (two-sum) and the base change by an
// FMA, so the exponent's rounding does not grow with M - s.
__device__ __forceinline__ uint64_t fixed_mass(float s, float M, float scale) {
  const float d = s - M;
  const float sv = d + M;
  const float dlo = (s - sv) + (-M - (d - sv));
  const float th = __fmul_rn(d, kL2E);
  const float tl = __builtin_fmaf(d, kL2E, -th) + __builtin_fmaf(d, kL2ELo, dlo * kL2E);
  const float w = __builtin_amdgcn_exp2f(th) * __builtin_fmaf(tl, 0.693147182f, 1.f);
  // th <= -64 leaves w scale below 1 (scale <= 2^62) and s = -inf makes it
  // NaN: 0 either way, chosen without a branch
  const float x = th > -64.f ? __fmul_rn(w, scale) : 0.f;
  // x in [0, 2^63) to an integer: the high word floor(x / 2^32), the low
  // word x - hi 2^32 (exact), each truncated by one conversion
  const float hi = floorf(x * 0x1p-32f);
  const uint32_t lo = (uint32_t)__builtin_fmaf(hi, -0x1p32f, x);
  return (uint64_t(uint32_t(hi)) << 32) | lo;
}

// First-level bin of a token: floor((M - s) 32), the last bin also taking
// everything further down (and -inf). Non-decreasing in the order key.
__device__ __forceinline__ uint32_t l1_bin(float s, float M) {
  return uint32_t(fminf(__fmul_rn(M - s, float(kRes)), float(kNB1 - 1)));
}

// First-level bins below a reference R0 that need not be the row maximum:
// g = fl(32 R0 - 32 s) (one fused multiply-add; R0x32 = 32 R0) and the bin
// floor(g) clamped to [0, kNB1 - 1], so that tokens above R0 fall into bin
// 0 with those just below it and the bins still follow the order of s.
__device__ __forceinline__ float l1_ref_g(float s, float R0x32) {
  return __builtin_fmaf(s, -float(kRes), R0x32);
}

__device__ __forceinline__ uint32_t l1_bin_ref(float s, float R0x32) {
  // the mask only matters for a NaN s, in rows that are left whole
  return uint32_t(__builtin_amdgcn_fmed3f(l1_ref_g(s, R0x32), 0.f, float(kNB1 - 1))) &
         uint32_t(kNB1 - 1);
}

// l1_bin(s, M) <= b for b below the last bin, as one comparison: `lim` =
// b + 1.
__device__ __forceinline__ bool l1_at_most(float s, float M, float lim) {
  return __fmul_rn(M - s, float(kRes)) < lim;
}

// Order keys that bin b can hold, with slack for the rounding of M - s.
__device__ __forceinline__ void l1_key_range(uint32_t b, float M, uint32_t& lo, uint32_t& hi) {
  const double e = 1.0 / 4194304.0;  // 2^-22, above the 2^-24 relative error of fl(M - s)
  lo = desc_key(__double2float_ru((double)M - (double(b) / kRes) * (1.0 - e)));
  hi = (b >= kNB1 - 1) ? 0xff800000u
                       : desc_key(__double2float_rd((double)M - (double(b + 1) / kRes) * (1.0 + e)));
}

// One pass over a row: f(x, v) for every token v < V with its raw logit x,
// four tiles of streaming loads in flight. The rows are read several times
// here, but a re-read gains nothing from the caches on this part while
// ordinary loads stream at about a third of the nontemporal rate, so every
// pass streams. Tiles wholly inside the row take no bounds checks.
template <int kDtype, bool kVecOk, class F>
__device__ __forceinline__ void raw_pass(const void* row, int V, F&& f, int t0 = 0) {
  const int nt = (V + kTile - 1) / kTile;
  const int nfull = V / kTile;
  int t = t0;
  for (; t + kBatch <= nfull; t += kBatch) {
    Grp<kDtype> g[kBatch];
#pragma unroll
    for (int n = 0; n < kBatch; ++n) load_grp<kDtype, kVecOk, true>(row, V, tile_elem(t + n), g[n]);
#pragma unroll
    for (int n = 0; n < kBatch; ++n)
#pragma unroll
      for (int j = 0; j < kVec; ++j) f(gelem(g[n], j), tile_elem(t + n) + j);
  }
  for (; t < nt; ++t) {
    Grp<kDtype> g;
    load_grp<kDtype, kVecOk, true>(row, V, tile_elem(t), g);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = tile_elem(t) + j;
      if (v < V) f(gelem(g, j), v);
    }
  }
}

// The same with the scaled logit s = fl32(x inv_t) (x itself when inv_t = 1).
template <int kDtype, bool kVecOk, class F>
__device__ __forceinline__ void row_pass(const void* row, int V, float inv_t, F&& f) {
  raw_pass<kDtype, kVecOk>(row, V, [&](float x, int v) { f(__fmul_rn(x, inv_t), v); });
}

// Appends (order key, token id) of token v, scaled logit s, to the LDS list
// on the lanes where w holds (ts.ncand counts every append, also past
// kCand). The compiler turns the per-lane increment into one LDS atomic per
// wave and a lane prefix count.
__device__ __forceinline__ void list_append(bool w, float s, int v, TruncShared& ts) {
  if (w) {
    const uint32_t pos = atomicAdd(&ts.ncand, 1u);
    if (pos < uint32_t(kCand)) {
      ts.ckey[pos] = desc_key(s);
      ts.cidx[pos] = v;
    }
  }
}

// Gathers the tokens `want(s)` admits into the LDS list.
template <int kDtype, bool kVecOk, class F>
__device__ __forceinline__ void gather_pass(const void* row, int V, float inv_t, F&& want,
                                            TruncShared& ts) {
  row_pass<kDtype, kVecOk>(row, V, inv_t,
                           [&](float s, int v) { list_append(want(s), s, v, ts); });
}

// Block-wide exclusive scans of two 64-bit integers; totals in ta, tb.
__device__ __forceinline__ void block_exscan2_u64(uint64_t a, uint64_t b, uint64_t& ea,
                                                  uint64_t& eb, uint64_t& ta, uint64_t& tb,
                                                  TruncShared& ts) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint64_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t na = __shfl_up(ia, o, kWave), nb = __shfl_up(ib, o, kWave);
    if (lane >= o) {
      ia += na;
      ib += nb;
    }
  }
  __syncthreads();
  if (lane == kWave - 1) {
    ts.part[wave][0] = ia;
    ts.part[wave][1] = ib;
  }
  __syncthreads();
  uint64_t pa = 0, pb = 0;
  ta = tb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      pa += ts.part[w][0];
      pb += ts.part[w][1];
    }
    ta += ts.part[w][0];
    tb += ts.part[w][1];
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
}

// The bucket b of h[0, nb) whose running sum reaches r (sum h[< b] < r <=
// sum h[<= b], r >= 1; the last bucket if the total is below r), with the
// sums of h and of g before it. nb is a multiple of the block size.
template <class T, class U>
__device__ __forceinline__ int select2(const T* h, const U* g, int nb, uint64_t r, uint64_t& bh,
                                       uint64_t& bg, TruncShared& ts) {
  const int per = nb / kThreads;
  const int b0 = threadIdx.x * per;
  uint64_t mh = 0, mg = 0;
  for (int i = 0; i < per; ++i) {
    mh += h[b0 + i];
    mg += g[b0 + i];
  }
  uint64_t eh, eg, th, tg;
  block_exscan2_u64(mh, mg, eh, eg, th, tg, ts);
  if (eh < r && r <= eh + mh) {
    uint64_t rh = eh, rg = eg;
    int b = b0 + per - 1;
    for (int i = 0; i < per; ++i) {
      if (rh + h[b0 + i] >= r) {
        b = b0 + i;
        break;
      }
      rh += h[b0 + i];
      rg += g[b0 + i];
    }
    ts.r32 = b;
    ts.r64[0] = rh;
    ts.r64[1] = rg;
  } else if (r > th && threadIdx.x == kThreads - 1) {
    ts.r32 = nb - 1;
    ts.r64[0] = th - h[nb - 1];
    ts.r64[1] = tg - g[nb - 1];
  }
  __syncthreads();
  bh = ts.r64[0];
  bg = ts.r64[1];
  const int b = ts.r32;
  __syncthreads();
  return b;
}

// Sum of h[0, b).
template <class T>
__device__ __forceinline__ uint64_t sum_before(const T* h, int nb, int b, TruncShared& ts) {
  const int per = nb / kThreads;
  uint64_t m = 0;
  for (int i = 0; i < per; ++i) {
    const int j = threadIdx.x * per + i;
    if (j < b) m += h[j];
  }
  uint64_t e0, e1, t0, t1;
  block_exscan2_u64(m, 0, e0, e1, t0, t1, ts);
  return t0;
}

__device__ __forceinline__ float block_max_f(float v, TruncShared& ts) {
  v = wmax(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) ts.fmax[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = ts.fmax[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, ts.fmax[w]);
  return r;
}

// Result of a selection: the value (order key or token id) where the
// running count or mass of the admitted tokens reaches the target, what of
// the target is left at that value, and the admitted totals before it and
// at it.
struct Sel {
  uint32_t val;
  uint64_t rest;
  uint64_t bcnt, bmass;
  uint64_t acnt, amass;
};

// Radix selection over the tokens `src` yields and `adm` admits, on the
// order key (or the token id, by_idx) within [lo, hi], 10 bits a level: by
// count, or by mass (by_mass; want_mass also sums masses in count mode).
template <class Src, class Adm>
__device__ __forceinline__ Sel select_value(Src&& src, Adm&& adm, bool by_idx, bool by_mass,
                                            bool want_mass, uint64_t target, uint32_t lo,
                                            uint32_t hi, float M, float scale, TruncShared& ts) {
  Sel r{0, target, 0, 0, 0, 0};
  for (int level = 0; level < 6; ++level) {  // 4 levels cover 32 bits
    const uint32_t span = hi - lo;
    const int sh = span < uint32_t(kNB) ? 0 : (32 - __clz(span)) - 10;
    for (int i = threadIdx.x; i < kNB; i += kThreads) {
      ts.cnt[i] = 0;
      ts.mass[i] = 0;
      ts.vmin[i] = 0xffffffffu;
      ts.vmax[i] = 0;
    }
    __syncthreads();
    src([&](float s, int v, uint32_t d) {
      const uint32_t u = by_idx ? uint32_t(v) : d;
      if (u < lo || u > hi || !adm(s, v, d)) return;
      const uint32_t i = (u - lo) >> sh;
      atomicAdd(&ts.cnt[i], 1u);
      if (want_mass) {
        const uint64_t m = fixed_mass(s, M, scale);
        if (m) atomicAdd(&ts.mass[i], (unsigned long long)m);
      }
      atomicMin(&ts.vmin[i], u);
      atomicMax(&ts.vmax[i], u);
    });
    __syncthreads();
    uint64_t bp, bo;
    const int b = by_mass ? select2(ts.mass, ts.cnt, kNB, r.rest, bp, bo, ts)
                          : select2(ts.cnt, ts.mass, kNB, r.rest, bp, bo, ts);
    r.rest -= bp;
    r.bcnt += by_mass ? bo : bp;
    r.bmass += by_mass ? bp : bo;
    const uint32_t vlo = ts.vmin[b], vhi = ts.vmax[b], c = ts.cnt[b];
    const uint64_t m = ts.mass[b];
    __syncthreads();
    if (vlo == vhi || c == 0) {
      r.val = vlo;
      r.acnt = c;
      r.amass = m;
      return r;
    }
    lo += uint32_t(b) << sh;
    hi = min(hi, lo + ((1u << sh) - 1u));
  }
  return r;
}

// Token id of the n-th token (in id order, n >= 1) whose key is `key`; every
// thread gets it. One pass over the row.
template <int kDtype, bool kVecOk>
__device__ __forceinline__ int nth_with_key(const void* row, int V, float inv_t, uint32_t key,
                                            uint64_t n, TruncShared& ts) {
  if (threadIdx.x == 0) ts.r32 = INT_MAX;
  const int nt = (V + kTile - 1) / kTile;
  uint64_t run = 0;  // matches in the tiles before t
  for (int t = 0; t < nt && run < n; t += 4) {
    Grp<kDtype> g[4];
    uint64_t mine = 0;  // this thread's matches per tile, 16 bits each
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t + i < nt)
        load_grp<kDtype, kVecOk, true>(row, V, tile_elem(t + i), g[i]);
      else
        fill_grp(g[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint64_t c = 0;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int v = tile_elem(t + i) + j;
        c += (t + i < nt && v < V && desc_key(__fmul_rn(gelem(g[i], j), inv_t)) == key);
      }
      mine |= c << (16 * i);
    }
    uint64_t exc, e1, total, t1;
    block_exscan2_u64(mine, 0, exc, e1, total, t1, ts);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t before = run + ((exc >> (16 * i)) & 0xffff);
      const uint64_t c = (mine >> (16 * i)) & 0xffff;
      if (before < n && n <= before + c) {
        uint64_t seen = before;
        for (int j = 0; j < kVec; ++j) {
          const int v = tile_elem(t + i) + j;
          if (v < V && desc_key(__fmul_rn(gelem(g[i], j), inv_t)) == key && ++seen == n) {
            ts.r32 = v;
            break;
          }
        }
      }
      run += (total >> (16 * i)) & 0xffff;
    }
  }
  __syncthreads();
  const int r = ts.r32;
  __syncthreads();
  return r;
}

// ceil(top_p W), clamped to [1, W].
__device__ __forceinline__ uint64_t top_p_need(float top_p, uint64_t W) {
  uint64_t n = (uint64_t)ceil((double)top_p * (double)W);
  return n < 1 ? 1 : (n > W ? W : n);
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void trunc_body(const Args& a) {
  __shared__ TruncShared ts;
  const bool draft = blockIdx.x & 1;
  const int slot = blockIdx.x >> 1;  // target row slot
  int b, k, kb;
  if (a.toff) {
    b = a.rowmap[slot];
    if (b < 0) return;
    k = slot - a.toff[b];
    kb = a.toff[b + 1] - a.toff[b] - 1;
  } else {
    b = slot / (a.Kmax + 1);
    k = slot - b * (a.Kmax + 1);
    kb = a.kreq[b];
  }
  const float T = a.temp[b];
  if (!(kb >= 0 && kb <= a.Kmax && temperature_ok(T)) || T == 0.f || k > kb || (draft && k == kb))
    return;  // a row the rows kernel does not sample
  KeepRow* out = draft ? &a.keep[target_row(a, b, k)].d : &a.keep[target_row(a, b, k)].t;
  const int V = a.V;
  const int top_k = a.top_k[b];
  const float top_p = a.top_p[b];
  const bool k_on = top_k >= 1 && top_k < V;
  const bool p_on = top_p < 1.f;
  if (!(top_p > 0.f) || !(k_on || p_on)) {  // a bad top_p faults the request
    if (threadIdx.x == 0) *out = keep_all();
    return;
  }
  const void* row = row_ptr<kDtype>(a, b, !draft, k);
  // fl32(x * 1) = x, so the unit temperature needs no case of its own
  const float inv_t = __fdiv_rn(1.f, T);
  const float scale = __builtin_ldexpf(1.f, 63 - (32 - __clz(V)));
  auto hbm = [&](auto&& f) {
    row_pass<kDtype, kVecOk>(row, V, inv_t, [&](float s, int v) { f(s, v, desc_key(s)); });
  };

  // ---- pass 1: the maximum, faults. fl32(x inv_t) is non-decreasing in x,
  // so the maximum of s is the scaled maximum of x; s is NaN only where x
  // is (inv_t = inf aside: then every s is +-inf or NaN and the row is
  // left whole below either way), and +inf somewhere only if at the maximum.
  // With top-k on, the same pass counts tokens per first-level bin below R0,
  // the largest scaled logit of the row's first tile (bins relative to it
  // keep the order of s and spread clustered logits as the bins below the
  // maximum do).
  float mx = -INFINITY;
  bool nan = false;
  float R0x32 = 0.f;  // 32 R0
  bool spec = false;  // pass 1 also lists the tokens of bins up to gb
  uint32_t gb = 0;
  if (k_on) {
    // NaN shows as an absolute value above +inf's bits
    uint32_t amax = 0;
    Grp<kDtype> g0;
    load_grp<kDtype, kVecOk, true>(row, V, tile_elem(0), g0);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float x = gelem(g0, j);
      if (tile_elem(0) + j < V) {
        amax = max(amax, __float_as_uint(x) & 0x7fffffffu);
        mx = fmaxf(mx, x);
      }
    }
    for (int i = threadIdx.x; i < kNB1; i += kThreads) ts.cnt1[i] = 0;
    const float R0 = __fmul_rn(block_max_f(mx, ts), inv_t);  // (its barriers cover the zeroing)
    // any finite reference keeps the order; 32 R0 is exact unless it overflows
    R0x32 = (R0 > -1e37f && R0 < 1e37f) ? R0 * float(kRes) : 0.f;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
      if (tile_elem(0) + j < V)
        atomicAdd(&ts.cnt1[l1_bin_ref(__fmul_rn(gelem(g0, j), inv_t), R0x32)], 1u);
    // For a small top_k the pass, instead of counting every token, lists
    // every token down to the bin where the first tile's count reaches
    // F top_k times the tile's share of the row (F = 16, less for a larger
    // top_k, so that about half the list is expected to fill): if the list
    // holds at least top_k tokens it is complete without a second pass, and
    // no LDS atomic is spent on the tokens below it.
    const int F = min(16, kCand / (2 * top_k));
    spec = F >= 4;
    if (spec) {
      __syncthreads();
      const int n0 = V < kTile ? V : kTile;
      const uint64_t kk =
          (uint64_t(F) * uint64_t(top_k) * uint64_t(n0) + uint64_t(V) - 1) / uint64_t(V);
      uint64_t b0, b1;
      gb = uint32_t(select2(ts.cnt1, ts.cnt1, kNB1, kk < 1 ? 1 : kk, b0, b1, ts));
      if (threadIdx.x == 0) ts.ncand = 0;
      __syncthreads();
    }
    // l1_bin_ref(s) <= gb as one comparison of its argument (the bin is not
    // an index here): g < gb + 1, or every token when gb is the last bin
    const bool every_g = gb >= uint32_t(kNB1 - 1);
    const float lim_g = float(gb + 1);
    if (spec) {
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int v = tile_elem(0) + j;
        const float s = __fmul_rn(gelem(g0, j), inv_t);
        list_append(v < V && (every_g || l1_ref_g(s, R0x32) < lim_g), s, v, ts);
      }
      raw_pass<kDtype, kVecOk>(row, V, [&](float x, int v) {
        amax = max(amax, __float_as_uint(x) & 0x7fffffffu);
        mx = fmaxf(mx, x);
        const float s = __fmul_rn(x, inv_t);
        list_append(every_g || l1_ref_g(s, R0x32) < lim_g, s, v, ts);
      }, 1);
    } else {
      raw_pass<kDtype, kVecOk>(row, V, [&](float x, int) {
        amax = max(amax, __float_as_uint(x) & 0x7fffffffu);
        mx = fmaxf(mx, x);
        atomicAdd(&ts.cnt1[l1_bin_ref(__fmul_rn(x, inv_t), R0x32)], 1u);
      }, 1);
    }
    nan = amax > 0x7f800000u;
  } else {
    raw_pass<kDtype, kVecOk>(row, V, [&](float x, int) {
      nan |= (x != x);
      mx = fmaxf(mx, x);
    });
  }
  nan = __syncthreads_or(nan);
  const float M = __fmul_rn(block_max_f(mx, ts), inv_t);
  if (nan || !(M > -INFINITY && M < INFINITY)) {  // the rows kernel faults the row: leave it whole
    if (threadIdx.x == 0) *out = keep_all();
    return;
  }

  // list: top-k is on and every token down to the bin (below R0) where the
  // count reaches top_k fits the LDS list. One more pass gathers them (every
  // token that top-k keeps is among them) and the rest works on the list.
  bool list = false, listed = false;
  float limR = 0.f;
  bool everyR = false;
  if (k_on && spec) {
    // The list holds every token of the bins up to gb, all ranking above the
    // tokens it leaves out: with at least top_k of them it holds every token
    // that top-k keeps. Their own bin counts give top_k's bin.
    const uint32_t n = ts.ncand;
    listed = n >= uint32_t(top_k) && n <= uint32_t(kCand);
    if (listed) {
      __syncthreads();
      for (int i = threadIdx.x; i < kNB1; i += kThreads) ts.cnt1[i] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n; i += kThreads)
        atomicAdd(&ts.cnt1[l1_bin_ref(key_value(ts.ckey[i]), R0x32)], 1u);
      __syncthreads();
      uint64_t bc, bg;
      const int binR = select2(ts.cnt1, ts.cnt1, kNB1, uint64_t(top_k), bc, bg, ts);
      everyR = binR >= kNB1 - 1;
      limR = float(binR + 1);
      list = true;
    }
    // otherwise the bins are redone below M
  } else if (k_on) {
    uint64_t bc, bg;
    const int binR = select2(ts.cnt1, ts.cnt1, kNB1, uint64_t(top_k), bc, bg, ts);
    list = bc + ts.cnt1[binR] <= uint64_t(kCand);
    everyR = binR >= kNB1 - 1;
    limR = float(binR + 1);
  }
  // masses of the whole row into the first-level histogram
  auto mass_pass = [&]() {
    row_pass<kDtype, kVecOk>(row, V, inv_t, [&](float s, int) {
      atomicAdd(&ts.mass1[l1_bin(s, M)], (unsigned long long)fixed_mass(s, M, scale));
    });
    __syncthreads();
  };

  int binK = -1, binP = -1;
  uint64_t rankK = 0, W0 = 0, needP = 0, beforeP = 0;
  // all_in: top-k is on and every token of the bins down to top-k's own
  // fits the LDS list; it is gathered whole and the masses of those bins
  // come from it. Otherwise a mass pass fills the histogram for the row.
  bool all_in = false;
  if (list) {
    if (!listed) {
      if (threadIdx.x == 0) ts.ncand = 0;
      __syncthreads();
      gather_pass<kDtype, kVecOk>(
          row, V, inv_t, [&](float s) { return everyR || l1_ref_g(s, R0x32) < limR; }, ts);
      __syncthreads();
    }
    rankK = uint64_t(top_k);
  } else {
    // ---- pass 2: first-level histograms, token counts for top-k, masses for
    // top-p alone (with top-k on, top-p only looks at the tokens top-k keeps,
    // whose masses are taken from the gathered list below)
    for (int i = threadIdx.x; i < kNB1; i += kThreads) {
      ts.cnt1[i] = 0;
      ts.mass1[i] = 0;
    }
    __syncthreads();
    if (k_on) {
      row_pass<kDtype, kVecOk>(row, V, inv_t,
                               [&](float s, int) { atomicAdd(&ts.cnt1[l1_bin(s, M)], 1u); });
      __syncthreads();
    } else {
      mass_pass();
    }

    if (k_on) {
      uint64_t bc, bm;
      binK = select2(ts.cnt1, ts.mass1, kNB1, uint64_t(top_k), bc, bm, ts);
      rankK = uint64_t(top_k) - bc;
      all_in = bc + ts.cnt1[binK] <= uint64_t(kCand);
      if (!all_in) {
        mass_pass();
        W0 = sum_before(ts.mass1, kNB1, binK, ts);  // mass of the bins above top-k's own
        if (p_on) {
          // top-p's bin is settled now if even the most top-k can keep of its
          // own bin leaves the target above it, in one bin
          const uint64_t n_hi = top_p_need(top_p, W0 + ts.mass1[binK]);
          if (n_hi <= W0) {
            uint64_t b0, b1, c0, c1;
            const int lo_bin = select2(ts.mass1, ts.cnt1, kNB1, top_p_need(top_p, W0), b0, c0, ts);
            const int hi_bin = select2(ts.mass1, ts.cnt1, kNB1, n_hi, b1, c1, ts);
            if (lo_bin == hi_bin) binP = lo_bin;
          }
        }
      }
    } else {
      uint64_t W = 0;
      {
        uint64_t e0, e1, t1;
        uint64_t m = 0;
        for (int i = 0; i < kNB1 / kThreads; ++i) m += ts.mass1[threadIdx.x * (kNB1 / kThreads) + i];
        block_exscan2_u64(m, 0, e0, e1, W, t1, ts);
      }
      needP = top_p_need(top_p, W);
      uint64_t bc;
      binP = select2(ts.mass1, ts.cnt1, kNB1, needP, beforeP, bc, ts);
    }

    // ---- pass 3: gather the tokens of the open bins into LDS
    if (threadIdx.x == 0) ts.ncand = 0;
    __syncthreads();
    if (all_in) {
      const bool every = binK >= kNB1 - 1;  // the last bin also takes g >= kNB1 and -inf
      const float lim = float(binK + 1);
      gather_pass<kDtype, kVecOk>(row, V, inv_t,
                                  [&](float s) { return every || l1_at_most(s, M, lim); }, ts);
    } else {
      gather_pass<kDtype, kVecOk>(row, V, inv_t, [&](float s) {
        const int i = int(l1_bin(s, M));
        return i == binK || i == binP;
      }, ts);
    }
    __syncthreads();
  }
  uint32_t nc = ts.ncand;
  bool in_lds = nc <= uint32_t(kCand);
  __syncthreads();
  auto lds = [&](auto&& f) {
    for (uint32_t i = threadIdx.x; i < nc; i += kThreads) {
      const uint32_t d = ts.ckey[i];
      f(key_value(d), ts.cidx[i], d);
    }
  };
  if (all_in) {
    if (in_lds) {
      // the same masses, bins and exact sums as a pass over the row would
      // give (key_value(desc_key(s)) = s, up to the sign of zero)
      lds([&](float s, int, uint32_t) {
        const uint64_t m = fixed_mass(s, M, scale);
        if (m) atomicAdd(&ts.mass1[l1_bin(s, M)], (unsigned long long)m);
      });
      __syncthreads();
    } else {
      mass_pass();  // not reached: the list holds exactly the tokens counted
    }
    W0 = sum_before(ts.mass1, kNB1, binK, ts);
  }

  // ---- small lists: every listed token's rank among the list in (key, id)
  // order from comparisons with all the others, masses in rank order and
  // their prefix sums. The list holds every token ranking at or above the
  // top_k-th, so for those their rank in the list is their rank in the row.
  uint32_t keyK = 0xffffffffu;
  int idxK = INT_MAX;
  uint64_t WK = 0;  // mass of the tokens top-k keeps
  uint32_t key = keyK;
  int idx = idxK;
  uint64_t kept = WK;  // mass of the kept tokens
  bool ranked = false;
  uint32_t* rk = ts.vmin;                                // keys of the ranked tokens
  int32_t* ri = reinterpret_cast<int32_t*>(ts.vmax);     // their ids
  if (k_on && in_lds && (list || all_in)) {
    // the listed tokens of the bins down to top-k's own (a list pass 1 made
    // also holds lower bins), copied out
    if (threadIdx.x == 0) ts.nrank = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nc; i += kThreads) {
      const uint32_t d = ts.ckey[i];
      if (!listed || everyR || l1_ref_g(key_value(d), R0x32) < limR) {
        const uint32_t pos = atomicAdd(&ts.nrank, 1u);
        if (pos < uint32_t(kNB)) {
          rk[pos] = d;
          ri[pos] = ts.cidx[i];
        }
      }
    }
    __syncthreads();
    const uint32_t nr = ts.nrank;
    const uint32_t np = (nr + 7u) & ~7u;  // padded with keys above every real one
    ranked = np <= uint32_t(kRankMax) && uint32_t(top_k) <= nr;
    if (ranked && threadIdx.x < np - nr) {
      rk[nr + threadIdx.x] = 0xffffffffu;
      ri[nr + threadIdx.x] = INT_MAX;
    }
    __syncthreads();
    if (ranked) {
      for (uint32_t i = threadIdx.x; i < nr; i += kThreads) {
        const uint64_t ci = (uint64_t(rk[i]) << 32) | uint32_t(ri[i]);
        uint32_t r = 0;
        for (uint32_t j = 0; j < np; j += 8) {
          const uint4 ka = *reinterpret_cast<const uint4*>(rk + j);
          const uint4 kb = *reinterpret_cast<const uint4*>(rk + j + 4);
          const uint4 ia = *reinterpret_cast<const uint4*>(ri + j);
          const uint4 ib = *reinterpret_cast<const uint4*>(ri + j + 4);
          r += ((uint64_t(ka.x) << 32) | ia.x) < ci;
          r += ((uint64_t(ka.y) << 32) | ia.y) < ci;
          r += ((uint64_t(ka.z) << 32) | ia.z) < ci;
          r += ((uint64_t(ka.w) << 32) | ia.w) < ci;
          r += ((uint64_t(kb.x) << 32) | ib.x) < ci;
          r += ((uint64_t(kb.y) << 32) | ib.y) < ci;
          r += ((uint64_t(kb.z) << 32) | ib.z) < ci;
          r += ((uint64_t(kb.w) << 32) | ib.w) < ci;
        }
        if (r < uint32_t(top_k)) {
          ts.cnt[r] = i;
          ts.mass[r] = fixed_mass(key_value(rk[i]), M, scale);
        }
      }
    }
    __syncthreads();
  }
  if (ranked) {
    uint32_t* srt = ts.cnt;            // index of each rank below top_k
    unsigned long long* pm = ts.mass;  // mass of each rank, then inclusive sums
    constexpr int kPer = kNB / kThreads;
    uint64_t m[kPer], own = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int r = threadIdx.x * kPer + q;
      m[q] = r < top_k ? pm[r] : 0;
      own += m[q];
    }
    uint64_t ex, e1, tot, t1;
    block_exscan2_u64(own, 0, ex, e1, tot, t1, ts);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      ex += m[q];
      pm[threadIdx.x * kPer + q] = ex;
    }
    __syncthreads();
    WK = tot;
    keyK = rk[srt[top_k - 1]];
    idxK = ri[srt[top_k - 1]];
    key = keyK;
    idx = idxK;
    kept = WK;
    if (p_on) {
      // the first rank whose running mass reaches top_p times WK
      needP = top_p_need(top_p, WK);
      if (threadIdx.x == 0) ts.r32 = top_k - 1;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int r = threadIdx.x * kPer + q;
        if (r < top_k && pm[r] >= needP && (r == 0 || pm[r - 1] < needP)) ts.r32 = r;
      }
      __syncthreads();
      const int rp = ts.r32;
      key = rk[srt[rp]];
      idx = ri[srt[rp]];
      kept = pm[rp];
    }
  }

  // ---- top-k: the top_k-th token
  if (k_on && !ranked) {
    auto adm = [&](float s, int, uint32_t) { return list || int(l1_bin(s, M)) == binK; };
    uint32_t lo = 0, hi = 0xffffffffu;
    if (!in_lds) l1_key_range(uint32_t(binK), M, lo, hi);
    const Sel sk = in_lds ? select_value(lds, adm, false, false, true, rankK, lo, hi, M, scale, ts)
                          : select_value(hbm, adm, false, false, true, rankK, lo, hi, M, scale, ts);
    keyK = sk.val;
    const uint64_t nK = sk.rest;
    if (nK < sk.acnt) {
      if (in_lds) {
        auto tie = [&](float, int, uint32_t d) { return d == keyK; };
        idxK = int(select_value(lds, tie, true, false, false, nK, 0, uint32_t(V - 1), M, scale, ts).val);
      } else {
        idxK = nth_with_key<kDtype, kVecOk>(row, V, inv_t, keyK, nK, ts);
      }
    }
    WK = W0 + sk.bmass + nK * (sk.acnt ? sk.amass / sk.acnt : 0);
  }

  // ---- top-p over the top-k set
  if (!ranked) {
    key = keyK;
    idx = idxK;
    kept = WK;
  }
  if (p_on && !ranked) {
    if (k_on) {
      needP = top_p_need(top_p, WK);
      if (list) {
        beforeP = 0;
      } else if (needP > W0) {
        binP = binK;
        beforeP = W0;
      } else {
        if (binP < 0) {
          uint64_t bc;
          binP = select2(ts.mass1, ts.cnt1, kNB1, needP, beforeP, bc, ts);
          if (!all_in) {
            // not gathered yet: gather it alone
            if (threadIdx.x == 0) ts.ncand = 0;
            __syncthreads();
            gather_pass<kDtype, kVecOk>(row, V, inv_t,
                                        [&](float s) { return int(l1_bin(s, M)) == binP; }, ts);
            __syncthreads();
            nc = ts.ncand;
            in_lds = nc <= uint32_t(kCand);
            __syncthreads();
          }
        } else {
          beforeP = sum_before(ts.mass1, kNB1, binP, ts);
        }
      }
    }
    const uint64_t rem = needP - beforeP;
    auto adm = [&](float s, int v, uint32_t d) {
      return (list || int(l1_bin(s, M)) == binP) && (d < keyK || (d == keyK && v <= idxK));
    };
    uint32_t lo = 0, hi = 0xffffffffu;
    if (!in_lds) l1_key_range(uint32_t(binP), M, lo, hi);
    const Sel sp = in_lds ? select_value(lds, adm, false, true, true, rem, lo, hi, M, scale, ts)
                          : select_value(hbm, adm, false, true, true, rem, lo, hi, M, scale, ts);
    key = sp.val;
    // every token of one key has the same mass; the bucket reached holds
    // positive mass
    const uint64_t w = sp.acnt ? sp.amass / sp.acnt : 0;
    const uint64_t n = w ? (sp.rest + w - 1) / w : 1;
    kept = beforeP + sp.bmass + n * w;
    if (n < sp.acnt) {
      if (in_lds) {
        auto tie = [&](float, int v, uint32_t d) {
          return d == key && (d != keyK || v <= idxK);
        };
        idx = int(select_value(lds, tie, true, false, false, n, 0, uint32_t(V - 1), M, scale, ts).val);
      } else {
        // the admitted tokens of the key are its first ones in id order
        idx = nth_with_key<kDtype, kVecOk>(row, V, inv_t, key, n, ts);
      }
    } else {
      idx = (key == keyK) ? idxK : INT_MAX;
    }
  }
  if (!draft) {
    // the kept tokens' ids for the row kernel, when every one of them is in
    // the LDS list (top-k on: they are among the tokens gathered)
    int32_t* klen = &a.klen[target_row(a, b, k)];
    if (k_on && in_lds && (list || all_in)) {
      int32_t* dst = a.klist + size_t(target_row(a, b, k)) * kCand;
      __syncthreads();
      if (threadIdx.x == 0) ts.ncand = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < nc; i += kThreads) {
        const uint32_t d = ts.ckey[i];
        const int v = ts.cidx[i];
        if (d < key || (d == key && v <= idx)) {
          const uint32_t pos = atomicAdd(&ts.ncand, 1u);
          if (pos < uint32_t(kCand)) dst[pos] = v;
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) *klen = int32_t(min(ts.ncand, uint32_t(kCand)));
    } else if (threadIdx.x == 0) {
      *klen = 0;
    }
  }
  if (threadIdx.x == 0) {
    // kept mass in the row kernel's convention: sum 2^(s log2e - R) =
    // 2^(M log2e - R) sum e^(s - M), log2e as the kernels round it
    const float R = __fmul_rn(M, kL2E);
    const double L = (double)kept / (double)scale * exp2((double)M * (double)kL2E - (double)R);
    *out = KeepRow{key, idx, R, (float)L};
  }
}

template <int kDtype, bool kVecOk>
__global__ __launch_bounds__(kThreads) void trunc_rows(Args a) {
  trunc_body<kDtype, kVecOk>(a);
}

// ------------------------------------------------------------------ finalize

// Block-wide exclusive scan in fp64 (fixed order); `total` gets the sum.
__device__ __forceinline__ double block_exscan(double v, Shared& sh, double& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  __syncthreads();
  if (lane == kWave - 1) sh.d[wave] = inc;
  __syncthreads();
  double pre = 0.0;
  total = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) pre += sh.d[w];
    total += sh.d[w];
  }
  return pre + inc - v;
}

__device__ __forceinline__ int block_min(int v, Shared& sh) {
  v = wmin(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.i[threadIdx.x / kWave][0] = v;
  __syncthreads();
  int r = sh.i[0][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = min(r, sh.i[w][0]);
  return r;
}

// fp64 probability of token v under a row's (R, L), base-2 convention; 0 for
// a token the row's truncation drops.
template <int kDtype>
__device__ __forceinline__ double prob64(const void* row, int v, float inv_t, bool unit, float R,
                                         float L, const KeepRow& kr) {
  return prob64_of(load1<kDtype>(row, v), v, inv_t, unit, R, L, kr);
}

// Inverse-CDF choice of a chunk from the masses m[0..NC) at u * total: the
// first chunk of positive mass whose running sum passes the target (if
// rounding leaves none, the last chunk of positive mass). Returns the chunk
// and, in `rem`, the target minus the mass before it.
__device__ __forceinline__ int pick_chunk(const float* m, int NC, double u, Shared& sh,
                                          double& rem) {
  double total = 0.0;
  for (int c0 = 0; c0 < NC; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    double part;
    (void)block_exscan(c < NC ? (double)m[c] : 0.0, sh, part);
    total += part;
  }
  const double target = u * total;
  double base = 0.0;
  for (int c0 = 0; c0 < NC; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const double mc = c < NC ? (double)m[c] : 0.0;
    double part;
    const double exc = base + block_exscan(mc, sh, part);
    const int hit = block_min((mc > 0.0 && exc + mc > target) ? c : INT_MAX, sh);
    if (hit != INT_MAX) {
      if (c == hit) sh.d[0] = target - exc;
      __syncthreads();
      rem = sh.d[0];
      __syncthreads();
      return hit;
    }
    base += part;
  }
  int last = -1;
  for (int c0 = 0; c0 < NC; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const int mine = (c < NC && m[c] > 0.f) ? c : -1;
    last = max(last, -block_min(mine >= 0 ? -mine : INT_MAX, sh));
  }
  rem = INFINITY;
  return last >= 0 ? last : 0;
}

// pick_chunk for NC <= kThreads chunks in one block scan: thread c holds
// chunk c's mass. Returns -1 (every thread) when no chunk has positive mass.
__device__ __forceinline__ int pick_chunk_small(const float* m, int NC, double u, Shared& sh,
                                                double& rem) {
  const int c = threadIdx.x;
  const double mc = c < NC ? (double)m[c] : 0.0;
  double total;
  const double exc = block_exscan(mc, sh, total);
  const double target = u * total;
  const int hit = block_min((mc > 0.0 && exc + mc > target) ? c : INT_MAX, sh);
  if (hit != INT_MAX) {
    if (c == hit) sh.d[0] = target - exc;
    __syncthreads();
    rem = sh.d[0];
    __syncthreads();
    return hit;
  }
  // rounding left no chunk past the target: the last chunk of positive mass
  const int last = -block_min((c < NC && mc > 0.0) ? -c : INT_MAX, sh);
  rem = INFINITY;
  return last == -INT_MAX ? -1 : last;
}

// Token of chunk c at remaining mass `rem`: fp64 weights of the chunk's 512
// tokens (one per thread), rescaled so they sum to the chunk's mass `cmass`
// (the unit the chunk was chosen in); the first token whose running weight
// passes `rem`, else the last token of positive weight; -1 if no token of
// the chunk has positive weight.
template <int kDtype>
__device__ __forceinline__ int search_chunk(const void* trow, const void* drow, int V, int c,
                                            double rem, double cmass, float inv_t, bool unit,
                                            float Rt, float Lt, float Rd, float Ld,
                                            const KeepPair& kp, Shared& sh) {
  const int v = c * kChunk + (int)threadIdx.x;
  double w = 0.0;
  if (threadIdx.x < kChunk && v < V) {
    const double p = prob64<kDtype>(trow, v, inv_t, unit, Rt, Lt, kp.t);
    w = drow ? fmax(0.0, p - prob64<kDtype>(drow, v, inv_t, unit, Rd, Ld, kp.d)) : p;
  }
  double total;
  const double exc = block_exscan(w, sh, total);
  const double f = (total > 0.0 && cmass > 0.0) ? cmass / total : 1.0;
  int pick = block_min((w > 0.0 && (exc + w) * f > rem) ? v : INT_MAX, sh);
  if (pick == INT_MAX) {
    const int last = -block_min(w > 0.0 ? -v : INT_MAX, sh);
    pick = (last == -INT_MAX) ? -1 : last;
  }
  return pick;
}

// Masses of p per chunk over a whole row, written over `m` (used when a
// rejection meets an all-zero residual, p_j == q_j).
template <int kDtype>
__device__ __forceinline__ void p_chunk_masses(const void* trow, int V, int NC, float inv_t,
                                               bool unit, float Rt, float Lt, const KeepRow& kr,
                                               float* m) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  for (int c = wave; c < NC; c += kWaves) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = c * kChunk + lane * kVec + j;
      if (v < V)
        s += (float)prob64<kDtype>(trow, v, inv_t, unit, Rt, Lt, kr);
    }
    s = wsum(s);
    if (lane == 0) m[c] = s;
  }
  __syncthreads();
}

// A request's output slots: out_tokens [ntok] and alpha [nalpha] (padded:
// Kmax + 1 and Kmax; packed: K_b + 1 and K_b; none when the packed offsets
// are bad).
struct Slots {
  int32_t* tok;
  float* alpha;
  int ntok, nalpha;
};

__device__ __forceinline__ void write_fault(const Args& a, int b, int status, const Slots& o) {
  for (int k = threadIdx.x; k < o.ntok; k += kThreads) o.tok[k] = -1;
  for (int k = threadIdx.x; k < o.nalpha; k += kThreads) o.alpha[k] = 0.f;
  if (threadIdx.x == 0) {
    a.status[b] = status;
    a.acc_len[b] = -1;
  }
}

struct FinShared {
  Shared red;
  double ratio[LVTV_MAX_K];
  double uacc[LVTV_MAX_K];
  int j;
  RowOut rc[LVTV_MAX_K + 1];  // the request's row records, read once
};

template <int kDtype>
__device__ __forceinline__ void finalize_body(const Args& a) {
  __shared__ FinShared fs;
  Shared& sh = fs.red;
  const int b = blockIdx.x;
  const float T = a.temp[b];
  const int Kmax = a.Kmax;
  int kb;
  Slots o;
  if (a.toff) {
    if (*a.packed_ok) {
      kb = a.toff[b + 1] - a.toff[b] - 1;
      o = Slots{a.out_tokens + a.toff[b], a.alpha + (a.toff[b] - b), kb + 1, kb};
    } else {
      kb = -1;
      o = Slots{a.out_tokens, a.alpha, 0, 0};
    }
  } else {
    kb = a.kreq[b];
    o = Slots{a.out_tokens + size_t(b) * (Kmax + 1), a.alpha + size_t(b) * Kmax, Kmax + 1, Kmax};
  }
  // faults: the draft tokens are checked whenever K_b is valid, the rows
  // only when the temperature is valid too (they are not computed otherwise)
  const bool k_ok = kb >= 0 && kb <= Kmax, t_ok = temperature_ok(T);
  const bool greedy = (T == 0.f);
  const int32_t* y = a.tokens + draft_row(a, b, 0);
  const RowOut* rows = a.rows + target_row(a, b, 0);
  int bad = 0, fault = 0;
  if (k_ok) {
    for (int k = threadIdx.x; k <= kb; k += kThreads) {
      if (k < kb) bad |= (y[k] < 0 || y[k] >= a.V);
      if (!t_ok) continue;
      const RowOut r = rows[k];
      fs.rc[k] = r;
      if (greedy) {
        fault |= (r.nan & 1) || !isfinite(r.Rt);
        if (k < kb) fault |= (r.nan & 2) || !isfinite(r.Rd);
      } else {
        fault |= !isfinite(r.Rt) || !isfinite(r.Lt) || !(r.Lt > 0.f);
        if (k < kb) fault |= !isfinite(r.Rd) || !isfinite(r.Ld) || !(r.Ld > 0.f);
      }
    }
  }
  const int status = (k_ok ? 0 : LVTV_STATUS_BAD_K) | (t_ok ? 0 : LVTV_STATUS_BAD_TEMPERATURE) |
                     ((a.top_p && !(a.top_p[b] > 0.f)) ? LVTV_STATUS_BAD_TRUNCATION : 0) |
                     (__syncthreads_or(bad) ? LVTV_STATUS_BAD_TOKEN : 0) |
                     (__syncthreads_or(fault) ? LVTV_STATUS_NONFINITE : 0);
  if (status) {
    write_fault(a, b, status, o);
    return;
  }
  int32_t* out_tok = o.tok;
  float* out_alpha = o.alpha;

  if (greedy) {
    if (threadIdx.x == 0) {
      int j = kb;
      for (int k = 0; k < kb; ++k)
        if (y[k] != rows[k].arg_t) {
          j = k;
          break;
        }
      for (int k = 0; k < o.nalpha; ++k)
        out_alpha[k] = (k < kb) ? (rows[k].arg_t == rows[k].arg_d ? 1.f : 0.f) : 0.f;
      for (int k = 0; k < o.ntok; ++k) out_tok[k] = k < j ? y[k] : (k == j ? rows[j].arg_t : -1);
      a.acc_len[b] = j;
      a.status[b] = 0;
    }
    return;
  }

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  // accept inputs for every position in parallel: u_k, and p(y_k)/q(y_k)
  // as the row kernel evaluated it (prob64_of with the row's statistics)
  if (int(threadIdx.x) < kb) {
    const int k = threadIdx.x;
    double u, u2;
    verify_uniforms(a.seed[b], uint64_t(b), uint64_t(k), u, u2);
    fs.uacc[k] = u;
    fs.ratio[k] = get_ratio(fs.rc[k]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 0; k < o.nalpha; ++k) out_alpha[k] = k < kb ? fs.rc[k].alpha : 0.f;
    int j = kb;
    for (int k = 0; k < kb; ++k)
      if (!(fs.uacc[k] < fs.ratio[k])) {
        j = k;
        break;
      }
    fs.j = j;
  }
  __syncthreads();
  const int j = fs.j;

  // the draw at position j
  double u_acc, u_draw;
  verify_uniforms(a.seed[b], uint64_t(b), uint64_t(j), u_acc, u_draw);
  const bool residual = j < kb;
  const RowOut r = fs.rc[j];
  const void* trow = row_ptr<kDtype>(a, b, true, j);
  const void* drow = residual ? row_ptr<kDtype>(a, b, false, j) : nullptr;
  float* m = a.chunk + size_t(target_row(a, b, j)) * a.NC;
  const int NC = a.NC;
  const KeepPair kp = a.keep ? a.keep[target_row(a, b, j)] : KeepPair{keep_all(), keep_all()};
  double rem;
  int c;
  if (NC <= kThreads) {
    // one block scan of the chunk masses gives the total and every chunk's
    // running mass
    c = pick_chunk_small(m, NC, u_draw, sh, rem);
    if (c < 0 && residual) {
      // residual zero everywhere: draw from p_j
      p_chunk_masses<kDtype>(trow, a.V, NC, inv_t, unit, r.Rt, r.Lt, kp.t, m);
      drow = nullptr;
      c = pick_chunk_small(m, NC, u_draw, sh, rem);
    }
    if (c < 0) c = 0;
  } else {
    int any = 0;
    for (int cc = threadIdx.x; cc < NC; cc += kThreads) any |= m[cc] > 0.f;
    if (residual && !__syncthreads_or(any)) {
      // residual zero everywhere: draw from p_j
      p_chunk_masses<kDtype>(trow, a.V, NC, inv_t, unit, r.Rt, r.Lt, kp.t, m);
      drow = nullptr;
    }
    c = pick_chunk(m, NC, u_draw, sh, rem);
  }
  const double cmass = (double)m[c];
  int v = search_chunk<kDtype>(trow, drow, a.V, c, rem, cmass, inv_t, unit, r.Rt, r.Lt, r.Rd,
                               r.Ld, kp, sh);
  if (v < 0 && drow) {
    // The chunk's residual mass was rounding noise (p_j and q_j agree to
    // within it, as when both are truncated to one token): the residual is
    // zero, draw from p_j.
    p_chunk_masses<kDtype>(trow, a.V, NC, inv_t, unit, r.Rt, r.Lt, kp.t, m);
    const int c2 = pick_chunk(m, NC, u_draw, sh, rem);
    v = search_chunk<kDtype>(trow, nullptr, a.V, c2, rem, (double)m[c2], inv_t, unit, r.Rt, r.Lt,
                             r.Rd, r.Ld, kp, sh);
  }
  if (v < 0 || v >= a.V) v = a.V - 1;  // unreachable: the chosen chunk has positive mass
  if (threadIdx.x == 0) {
    for (int k = 0; k < o.ntok; ++k) out_tok[k] = k < j ? y[k] : (k == j ? v : -1);
    a.acc_len[b] = j;
    a.status[b] = 0;
  }
}

template <int kDtype>
__global__ __launch_bounds__(kThreads) void verify_finalize(Args a) {
  finalize_body<kDtype>(a);
}

// ------------------------------------------------------------------ host side

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  int n_tiles, NC;
  size_t off_rows, off_chunk, off_map, off_keep, off_klen, off_klist, total;
};

// `rows` target rows (B (Kmax + 1) padded, total_rows packed); the row map
// and its validity flag only for the packed layout, the keep records only
// with truncation.
Layout make_layout(size_t rows, int V, bool packed, bool trunc = false) {
  Layout L;
  L.n_tiles = (V + kTile - 1) / kTile;
  L.NC = L.n_tiles * kWaves;
  size_t off = kReservedBytes;
  L.off_rows = off;
  off = align256(off + sizeof(RowOut) * rows);
  L.off_chunk = off;
  off = align256(off + sizeof(float) * rows * L.NC);
  L.off_map = off;
  if (packed) off = align256(off + sizeof(int32_t) * (rows + 1));
  L.off_keep = off;
  if (trunc) off = align256(off + sizeof(KeepPair) * rows);
  L.off_klen = off;
  if (trunc) off = align256(off + sizeof(int32_t) * rows);
  L.off_klist = off;
  if (trunc) off = align256(off + sizeof(int32_t) * rows * kCand);
  L.total = off;
  return L;
}

bool sizes_ok(int32_t B, int32_t Kmax, int32_t V) {
  return B >= 1 && B <= LVTV_MAX_B && Kmax >= 0 && Kmax <= LVTV_MAX_K && V >= 1 && V <= LVTV_MAX_V;
}

bool packed_sizes_ok(int32_t B, int32_t total_rows, int32_t V) {
  return B >= 1 && B <= LVTV_MAX_B && total_rows >= B && total_rows <= B * (LVTV_MAX_K + 1) &&
         V >= 1 && V <= LVTV_MAX_V;
}

// Checks the packed offsets (toff[0] = 0, toff[B] = total_rows, 1 to
// LVTV_MAX_K + 1 target rows per request, so the requests tile the rows
// exactly) and writes the request of every target row, or -1 everywhere if
// the offsets are bad. One workgroup.
__global__ __launch_bounds__(1024) void packed_map(const int32_t* toff, int B, int total_rows,
                                                   int32_t* rowmap, int32_t* ok) {
  int bad = 0;
  for (int b = threadIdx.x; b < B; b += 1024) {
    const int n = toff[b + 1] - toff[b];
    bad |= !(n >= 1 && n <= LVTV_MAX_K + 1);
  }
  if (threadIdx.x == 0) bad |= (toff[0] != 0) || (toff[B] != total_rows);
  const bool good = !__syncthreads_or(bad);
  if (good) {
    for (int b = threadIdx.x; b < B; b += 1024)
      for (int g = toff[b]; g < toff[b + 1]; ++g) rowmap[g] = b;
  } else {
    for (int g = threadIdx.x; g < total_rows; g += 1024) rowmap[g] = -1;
  }
  if (threadIdx.x == 0) *ok = good ? 1 : 0;
}

template <int kDtype, bool kVecOk>
hipError_t launch(const Args& a, hipStream_t stream) {
  if (a.toff) {
    hipLaunchKernelGGL(packed_map, dim3(1), dim3(1024), 0, stream, a.toff, a.B, a.total_rows,
                       const_cast<int32_t*>(a.rowmap), const_cast<int32_t*>(a.packed_ok));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid =
      a.toff ? unsigned(a.total_rows) : unsigned(a.B) * unsigned(a.Kmax + 1);
  if (a.keep) {
    hipLaunchKernelGGL((trunc_rows<kDtype, kVecOk>), dim3(2 * grid), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (kDtype == 1)
      hipLaunchKernelGGL((verify_rows_bf16<kVecOk, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((verify_rows_f32<kVecOk, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if constexpr (kDtype == 1)
      hipLaunchKernelGGL((verify_rows_bf16<kVecOk, false>), dim3(grid), dim3(kThreads), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((verify_rows_f32<kVecOk, false>), dim3(grid), dim3(kThreads), 0, stream,
                         a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_finalize<kDtype>, dim3(unsigned(a.B)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// The padded-layout verify, with top-k / top-p truncation when top_k and
// top_p are given.
int verify_padded(const void* target_logits, const void* draft_logits, int dtype,
                  const int32_t* draft_tokens, const int32_t* k_per_req, const float* temperature,
                  const uint64_t* seed, const int32_t* top_k, const float* top_p, int32_t B,
                  int32_t Kmax, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                  float* alpha, int32_t* status, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (dtype != LVTV_F32 && dtype != LVTV_BF16) return LVTV_ERR_DTYPE;
  if (!sizes_ok(B, Kmax, V)) return LVTV_ERR_SHAPE;
  if (!target_logits || !k_per_req || !temperature || !seed || !accepted_len || !out_tokens ||
      !status)
    return LVTV_ERR_NULL;
  if (Kmax > 0 && (!draft_logits || !draft_tokens || !alpha)) return LVTV_ERR_NULL;
  const bool trunc = top_k || top_p;
  if (trunc && !(top_k && top_p)) return LVTV_ERR_NULL;
  const Layout L = make_layout(size_t(B) * (Kmax + 1), V, false, trunc);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LVTV_ERR_WORKSPACE;
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
  a.n_tiles = L.n_tiles;
  a.NC = L.NC;
  a.acc_len = accepted_len;
  a.out_tokens = out_tokens;
  a.alpha = alpha;
  a.status = status;
  char* ws = static_cast<char*>(workspace);
  a.rows = reinterpret_cast<RowOut*>(ws + L.off_rows);
  a.chunk = reinterpret_cast<float*>(ws + L.off_chunk);
  a.toff = nullptr;
  a.rowmap = nullptr;
  a.packed_ok = nullptr;
  a.total_rows = B * (Kmax + 1);
  a.top_k = top_k;
  a.top_p = top_p;
  a.keep = trunc ? reinterpret_cast<KeepPair*>(ws + L.off_keep) : nullptr;
  a.klen = trunc ? reinterpret_cast<int32_t*>(ws + L.off_klen) : nullptr;
  a.klist = trunc ? reinterpret_cast<int32_t*>(ws + L.off_klist) : nullptr;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(target_logits) |
                        reinterpret_cast<uintptr_t>(draft_logits);
  const bool vec_ok = (V % kVec == 0) && ((mis & 15) == 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == LVTV_BF16)
    e = vec_ok ? launch<1, true>(a, s) : launch<1, false>(a, s);
  else
    e = vec_ok ? launch<0, true>(a, s) : launch<0, false>(a, s);
  return e == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}

}  // namespace
}  // namespace vr
}  // namespace lvtv

// ------------------------------------------------------------------ no-allocation entry

namespace lvtv {
namespace vr {
namespace {

// The verify step's scratch for callers that cannot allocate: one array per
// GPU in the library's own device memory, held until the process ends. Host
// code never uses the array's name as an address (on the host it is only a
// stand-in): each device's address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kNoAllocBytes = LVTV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (nullptr on a HIP error).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace vr
}  // namespace lvtv

extern "C" int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                                   int dtype, const int32_t* draft_tokens,
                                   const int32_t* k_per_req, const float* temperature,
                                   const uint64_t* seed, int32_t B, int32_t Kmax, int32_t V,
                                   int32_t* accepted_len, int32_t* out_tokens, float* alpha,
                                   int32_t* status, void* stream) {
  using namespace lvtv::vr;
  if (dtype != LVTV_F32 && dtype != LVTV_BF16) return LVTV_ERR_DTYPE;
  if (!sizes_ok(B, Kmax, V)) return LVTV_ERR_SHAPE;
  if (make_layout(size_t(B) * (Kmax + 1), V, false).total > kNoAllocBytes)
    return LVTV_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return LVTV_ERR_LAUNCH;
  return verify_padded(target_logits, draft_logits, dtype, draft_tokens, k_per_req, temperature,
                       seed, nullptr, nullptr, B, Kmax, V, accepted_len, out_tokens, alpha,
                       status, ws, kNoAllocBytes, stream);
}

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t Kmax, int32_t V, int dtype) {
  if (!lvtv::vr::sizes_ok(B, Kmax, V) || (dtype != LVTV_F32 && dtype != LVTV_BF16)) return 0;
  return lvtv::vr::make_layout(size_t(B) * (Kmax + 1), V, false).total;
}

extern "C" size_t spec_verify_packed_workspace_bytes(int32_t B, int32_t total_rows, int32_t V,
                                                      int dtype) {
  if (!lvtv::vr::packed_sizes_ok(B, total_rows, V) || (dtype != LVTV_F32 && dtype != LVTV_BF16))
    return 0;
  return lvtv::vr::make_layout(size_t(total_rows), V, true).total;
}

extern "C" int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                           const int32_t* draft_tokens, const int32_t* k_per_req,
                           const float* temperature, const uint64_t* seed, int32_t B,
                           int32_t Kmax, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                           float* alpha, int32_t* status, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return lvtv::vr::verify_padded(target_logits, draft_logits, dtype, draft_tokens, k_per_req,
                                 temperature, seed, nullptr, nullptr, B, Kmax, V, accepted_len,
                                 out_tokens, alpha, status, workspace, workspace_bytes, stream);
}

extern "C" size_t spec_verify_topkp_workspace_bytes(int32_t B, int32_t Kmax, int32_t V,
                                                     int dtype) {
  if (!lvtv::vr::sizes_ok(B, Kmax, V) || (dtype != LVTV_F32 && dtype != LVTV_BF16)) return 0;
  return lvtv::vr::make_layout(size_t(B) * (Kmax + 1), V, false, true).total;
}

extern "C" int spec_verify_topkp(const void* target_logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const int32_t* k_per_req,
                                 const float* temperature, const uint64_t* seed,
                                 const int32_t* top_k, const float* top_p, int32_t B,
                                 int32_t Kmax, int32_t V, int32_t* accepted_len,
                                 int32_t* out_tokens, float* alpha, int32_t* status,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!top_k || !top_p) return LVTV_ERR_NULL;
  return lvtv::vr::verify_padded(target_logits, draft_logits, dtype, draft_tokens, k_per_req,
                                 temperature, seed, top_k, top_p, B, Kmax, V, accepted_len,
                                 out_tokens, alpha, status, workspace, workspace_bytes, stream);
}

extern "C" int spec_verify_packed(const void* target_logits, const void* draft_logits, int dtype,
                                  const int32_t* draft_tokens, const int32_t* row_offsets,
                                  const float* temperature, const uint64_t* seed, int32_t B,
                                  int32_t total_rows, int32_t V, int32_t* accepted_len,
                                  int32_t* out_tokens, float* alpha, int32_t* status,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  using namespace lvtv;
  using namespace lvtv::vr;
  if (dtype != LVTV_F32 && dtype != LVTV_BF16) return LVTV_ERR_DTYPE;
  if (!packed_sizes_ok(B, total_rows, V)) return LVTV_ERR_SHAPE;
  if (!target_logits || !row_offsets || !temperature || !seed || !accepted_len || !out_tokens ||
      !status)
    return LVTV_ERR_NULL;
  if (total_rows > B && (!draft_logits || !draft_tokens || !alpha)) return LVTV_ERR_NULL;
  const Layout L = make_layout(size_t(total_rows), V, true);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LVTV_ERR_WORKSPACE;
  Args a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.kreq = nullptr;
  a.temp = temperature;
  a.seed = seed;
  a.B = B;
  a.Kmax = LVTV_MAX_K;
  a.V = V;
  a.n_tiles = L.n_tiles;
  a.NC = L.NC;
  a.acc_len = accepted_len;
  a.out_tokens = out_tokens;
  a.alpha = alpha;
  a.status = status;
  char* ws = static_cast<char*>(workspace);
  a.rows = reinterpret_cast<RowOut*>(ws + L.off_rows);
  a.chunk = reinterpret_cast<float*>(ws + L.off_chunk);
  a.toff = row_offsets;
  a.rowmap = reinterpret_cast<int32_t*>(ws + L.off_map);
  a.packed_ok = reinterpret_cast<int32_t*>(ws + L.off_map) + total_rows;
  a.total_rows = total_rows;
  a.top_k = nullptr;
  a.top_p = nullptr;
  a.keep = nullptr;
  a.klen = nullptr;
  a.klist = nullptr;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(target_logits) |
                        reinterpret_cast<uintptr_t>(draft_logits);
  const bool vec_ok = (V % kVec == 0) && ((mis & 15) == 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == LVTV_BF16)
    e = vec_ok ? launch<1, true>(a, s) : launch<1, false>(a, s);
  else
    e = vec_ok ? launch<0, true>(a, s) : launch<0, false>(a, s);
  return e == hipSuccess ? LVTV_OK : LVTV_ERR_LAUNCH;
}
