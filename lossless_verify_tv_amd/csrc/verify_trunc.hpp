// Top-k / top-p selection for spec_verify_topkp (gfx950).
#pragma once

#include "verify_common.hpp"

namespace lvtv {
namespace vr {
namespace {

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
  static_assert(kVec <= 8, "a tile's tokens of one thread fit 8 mask bits");
  if (threadIdx.x == 0) ts.r32 = INT_MAX;
  const int nt = (V + kTile - 1) / kTile;
  uint64_t run = 0;  // matches in the tiles before t
  for (int t = 0; t < nt && run < n; t += 4) {
    Grp<kDtype> g[4];
    uint64_t mine = 0;   // this thread's matches per tile, 16 bits each
    uint32_t masks = 0;  // which of its kVec tokens match, 8 bits a tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t + i < nt)
        load_grp<kDtype, kVecOk, true>(row, V, tile_elem(t + i), g[i]);
      else
        fill_grp(g[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t mk = 0;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int v = tile_elem(t + i) + j;
        mk |= uint32_t(t + i < nt && v < V &&
                       desc_key(__fmul_rn(gelem(g[i], j), inv_t)) == key) << j;
      }
      masks |= mk << (8 * i);
      mine |= uint64_t(__popc(mk)) << (16 * i);
    }
    uint64_t exc, e1, total, t1;
    block_exscan2_u64(mine, 0, exc, e1, total, t1, ts);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t before = run + ((exc >> (16 * i)) & 0xffff);
      const uint64_t c = (mine >> (16 * i)) & 0xffff;
      if (before < n && n <= before + c) {
        // the (n - before)-th set bit of the tile's mask
        const uint32_t mk = (masks >> (8 * i)) & 0xffu;
        uint32_t left = uint32_t(n - before);
        int hit = 0;
        for (int j = 0; j < kVec; ++j) {
          if (((mk >> j) & 1u) && --left == 0) {
            hit = j;
            break;
          }
        }
        ts.r32 = tile_elem(t + i) + hit;
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

}  // namespace
}  // namespace vr
}  // namespace lvtv
