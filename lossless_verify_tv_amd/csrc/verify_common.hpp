// Shared pieces of the verify step's kernels (gfx950): tile and chunk
// geometry, the per-row record, argument block, groups of 8 tokens and
// their loads, block reductions and the fp64 probability of one token.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

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
  } else if (e + kVec <= V) {
    // a group wholly inside a row that is not 16-byte aligned: unaligned
    // vector loads
    const char* p = static_cast<const char*>(row) + int64_t(e) * (kDtype == 1 ? 2 : 4);
    g.q[0] = kNt ? ld_nt16_u(p) : ld16_u(p);
    if constexpr (kDtype == 0) g.q[1] = kNt ? ld_nt16_u(p + 16) : ld16_u(p + 16);
  } else if constexpr (kDtype == 1) {
    // the row's last group: token by token
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

}  // namespace
}  // namespace vr
}  // namespace lvtv
