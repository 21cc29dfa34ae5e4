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
#include "verify_common.hpp"


namespace lvtv {
namespace vr {
namespace {

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

// A truncated row's keep rule on the raw logits. The scaled logit
// s(x) = scale_logit(x) never decreases as x grows, so "s > sk" is "x > xa"
// with xa the largest input value whose s is at most sk, and "s == sk" is
// "xe <= x <= xa" with xe the smallest whose s is at least sk: a token is
// kept iff x > xa, or x >= xe and its id is at most idx. The bounds are
// found by bisection over the input format's values in order (16 steps for
// bf16, 32 for fp32; s itself at T = 1).
struct KeepCut {
  float xa, xe;
  int idx;
};

__device__ __forceinline__ uint32_t asc_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float asc_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The input format's values in ascending order, by position.
template <int kDtype>
__device__ __forceinline__ uint32_t fmt_pos(float x) {
  return kDtype == 1 ? asc_key(x) >> 16 : asc_key(x);
}

template <int kDtype>
__device__ __forceinline__ float fmt_at(uint32_t i) {
  if constexpr (kDtype == 1)
    return asc_value((i << 16) | ((i & 0x8000u) ? 0u : 0xffffu));
  else
    return asc_value(i);
}

template <int kDtype>
__device__ __forceinline__ KeepCut keep_cut(const KeepRow& kr, float inv_t, bool unit) {
  const float sk = key_value(kr.key);
  KeepCut k{sk, sk, kr.idx};
  if (unit) return k;
  // largest position with s <= sk: s(-inf) = -inf <= sk, s(+inf) = +inf > sk
  uint32_t lo = fmt_pos<kDtype>(-INFINITY), hi = fmt_pos<kDtype>(INFINITY);
  while (hi - lo > 1) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (scale_logit(fmt_at<kDtype>(mid), inv_t, false) <= sk)
      lo = mid;
    else
      hi = mid;
  }
  k.xa = fmt_at<kDtype>(lo);
  // smallest position with s >= sk
  if (sk == -INFINITY) {
    k.xe = -INFINITY;
  } else {
    lo = fmt_pos<kDtype>(-INFINITY);
    hi = fmt_pos<kDtype>(INFINITY);
    while (hi - lo > 1) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (scale_logit(fmt_at<kDtype>(mid), inv_t, false) >= sk)
        hi = mid;
      else
        lo = mid;
    }
    k.xe = fmt_at<kDtype>(hi);
  }
  return k;
}

// overlap_tile over a pair whose rows are both truncated: a dropped token
// has p (q) = 0, the value its -inf logit would give.
template <int kDtype, bool kPair>
__device__ __forceinline__ void overlap_tile_cut(const Grp<kDtype>& gt, const Grp<kDtype>& gd,
                                                 int e, float c, float nrt, float nrd,
                                                 const KeepCut& kt, const KeepCut& kd, float& sa,
                                                 float* chunk_row, int t) {
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float xt = gelem(gt, j);
    const bool keep_t = (xt > kt.xa) | ((xt >= kt.xe) & (e + j <= kt.idx));
    const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(xt, c, nrt));
    const float p = keep_t ? pe : 0.f;
    if constexpr (kPair) {
      const float xd = gelem(gd, j);
      const bool keep_d = (xd > kd.xa) | ((xd >= kd.xe) & (e + j <= kd.idx));
      const float qe = __builtin_amdgcn_exp2f(__builtin_fmaf(xd, c, nrd));
      const float q = keep_d ? qe : 0.f;
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
      // one pass, the keep rule applied on the raw logits
      const KeepCut ct = keep_cut<kDtype>(kp.t, inv_t, unit);
      const KeepCut cd = kPair ? keep_cut<kDtype>(kp.d, inv_t, unit) : ct;
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
        for (int n = 0; n < kBatch; ++n)
          overlap_tile_cut<kDtype, kPair>(gt[n], gd[n], tile_elem(t + n), c, nrt, nrd, ct, cd, sa,
                                          chunk_row, t + n);
      }
      for (; t < nfull; ++t) {
        Grp<kDtype> gt, gd;
        load_grp<kDtype, kVecOk, true>(trow, V, tile_elem(t), gt);
        if constexpr (kPair) load_grp<kDtype, kVecOk, true>(drow, V, tile_elem(t), gd);
        overlap_tile_cut<kDtype, kPair>(gt, gd, tile_elem(t), c, nrt, nrd, ct, cd, sa, chunk_row,
                                        t);
      }
      if (tail) {
        Grp<kDtype> gt, gd;
        load_tail<kDtype, kVecOk>(trow, V, nfull, gt);
        if constexpr (kPair) load_tail<kDtype, kVecOk>(drow, V, nfull, gd);
        overlap_tile_cut<kDtype, kPair>(gt, gd, tile_elem(nfull), c, nrt, nrd, ct, cd, sa,
                                        chunk_row, nfull);
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

}  // namespace
}  // namespace vr
}  // namespace lvtv

#include "verify_trunc.hpp"

namespace lvtv {
namespace vr {
namespace {

// ------------------------------------------------------------------ finalize

// One DPP move of an fp64 value (both halves with the same control); lanes
// without a source, or in rows the row mask leaves out, read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b)), kCtrl, kRowMask,
                                                           0xf, true));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), kCtrl,
                                                           kRowMask, 0xf, true));
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

// Block-wide exclusive scan in fp64 (fixed order); `total` gets the sum.
// Within a wave: an inclusive scan of each 16-lane row by row shifts of 1,
// 2, 4 and 8 lanes, then rows 1 and 3 add the last lane of the row before
// them and rows 2 and 3 the last lane of row 1 (row broadcasts 15 and 31).
__device__ __forceinline__ double block_exscan(double v, Shared& sh, double& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double inc = v;
  inc += dpp_f64<0x111, 0xf>(inc);  // row_shr:1
  inc += dpp_f64<0x112, 0xf>(inc);  // row_shr:2
  inc += dpp_f64<0x114, 0xf>(inc);  // row_shr:4
  inc += dpp_f64<0x118, 0xf>(inc);  // row_shr:8
  inc += dpp_f64<0x142, 0xa>(inc);  // row_bcast:15 into rows 1 and 3
  inc += dpp_f64<0x143, 0xc>(inc);  // row_bcast:31 into rows 2 and 3
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
// chunk c's mass mc (0 past NC). Returns -1 (every thread) when no chunk has
// positive mass.
__device__ __forceinline__ int pick_chunk_small(double mc, int NC, double u, Shared& sh,
                                                double& rem) {
  const int c = threadIdx.x;
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

__device__ __forceinline__ int pick_chunk_small(const float* m, int NC, double u, Shared& sh,
                                                double& rem) {
  const int c = threadIdx.x;
  return pick_chunk_small(c < NC ? (double)m[c] : 0.0, NC, u, sh, rem);
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
  double udraw[LVTV_MAX_K + 1];  // word 1 of each position's Philox block
  double cmass;                  // the chosen chunk's mass
  int j;
  RowOut rc[LVTV_MAX_K + 1];  // the request's row records, read once
  int32_t y[LVTV_MAX_K];      // its draft tokens, read once
};

template <int kDtype>
__device__ __forceinline__ void finalize_body(const Args& a) {
  __shared__ FinShared fs;
  Shared& sh = fs.red;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float T = a.temp[b];
  const int Kmax = a.Kmax;
  const int NC = a.NC;
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
  // kb <= LVTV_MAX_K < kThreads: thread k takes position k, and the draft
  // tokens and row records go to LDS for the serial steps below
  if (k_ok && tid <= kb) {
    const int k = tid;
    if (k < kb) {
      const int32_t yv = y[k];
      fs.y[k] = yv;
      bad |= (yv < 0 || yv >= a.V);
    }
    if (t_ok) {
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
        if (fs.y[k] != fs.rc[k].arg_t) {
          j = k;
          break;
        }
      for (int k = 0; k < o.nalpha; ++k)
        out_alpha[k] = (k < kb) ? (fs.rc[k].arg_t == fs.rc[k].arg_d ? 1.f : 0.f) : 0.f;
      for (int k = 0; k < o.ntok; ++k)
        out_tok[k] = k < j ? fs.y[k] : (k == j ? fs.rc[j].arg_t : -1);
      a.acc_len[b] = j;
      a.status[b] = 0;
    }
    return;
  }

  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  // accept inputs for every position in parallel: u_k, and p(y_k)/q(y_k)
  // as the row kernel evaluated it (prob64_of with the row's statistics)
  if (tid <= kb) {
    const int k = tid;
    double u, u2;
    verify_uniforms(a.seed[b], uint64_t(b), uint64_t(k), u, u2);
    fs.udraw[k] = u2;
    if (k < kb) {
      fs.uacc[k] = u;
      fs.ratio[k] = get_ratio(fs.rc[k]);
    }
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
  const double u_draw = fs.udraw[j];
  const bool residual = j < kb;
  const RowOut r = fs.rc[j];
  const void* trow = row_ptr<kDtype>(a, b, true, j);
  const void* drow = residual ? row_ptr<kDtype>(a, b, false, j) : nullptr;
  float* m = a.chunk + size_t(target_row(a, b, j)) * NC;
  const KeepPair kp = a.keep ? a.keep[target_row(a, b, j)] : KeepPair{keep_all(), keep_all()};
  double rem;
  int c;
  double cmass;
  if (NC <= kThreads) {
    // one block scan of the chunk masses gives the total and every chunk's
    // running mass
    double mc = tid < NC ? (double)m[tid] : 0.0;
    c = pick_chunk_small(mc, NC, u_draw, sh, rem);
    if (c < 0 && residual) {
      // residual zero everywhere: draw from p_j
      p_chunk_masses<kDtype>(trow, a.V, NC, inv_t, unit, r.Rt, r.Lt, kp.t, m);
      drow = nullptr;
      mc = tid < NC ? (double)m[tid] : 0.0;
      c = pick_chunk_small(mc, NC, u_draw, sh, rem);
    }
    if (c < 0) c = 0;
    if (tid == c) fs.cmass = mc;
    __syncthreads();
    cmass = fs.cmass;
  } else {
    int any = 0;
    for (int cc = threadIdx.x; cc < NC; cc += kThreads) any |= m[cc] > 0.f;
    if (residual && !__syncthreads_or(any)) {
      // residual zero everywhere: draw from p_j
      p_chunk_masses<kDtype>(trow, a.V, NC, inv_t, unit, r.Rt, r.Lt, kp.t, m);
      drow = nullptr;
    }
    c = pick_chunk(m, NC, u_draw, sh, rem);
    cmass = (double)m[c];
  }
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
    for (int k = 0; k < o.ntok; ++k) out_tok[k] = k < j ? fs.y[k] : (k == j ? v : -1);
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
