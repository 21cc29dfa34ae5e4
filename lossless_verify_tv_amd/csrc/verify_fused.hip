// spec_verify, single-read kernel (one launch) for gfx950.
//
// Each 512-thread workgroup owns one slice of 16384 tokens of one (request b,
// position k) pair of rows: target row k and, for k < K_b, draft row k
// (k = K_b is the bonus row, target only). It streams its slice from HBM
// once, keeping the raw logits in registers (bf16 stays packed, two tokens
// per register), then:
//   1. computes the slice's softmax statistics for both rows (max, sum of
//      exp), publishes them as tagged words and collects those of the other
//      slices of the same rows (bounded wait, see fused_common.hpp);
//   2. with the row statistics, recomputes the exponentials from the
//      registers into p and q and accumulates alpha = sum min(p, q) over the
//      slice and, per 2048-token chunk (one wave's contiguous span), the
//      residual mass sum max(0, p - q); for the bonus row, the mass of p;
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

constexpr int kThreads = 512;                       // threads per workgroup
constexpr int kWaves = kThreads / kWave;            // 8
constexpr int kSteps = 4;                           // 8-token groups per thread per row
constexpr int kSlice = kThreads * kVec * kSteps;    // 16384 tokens per workgroup
constexpr int kSpan = kWave * kVec * kSteps;        // 2048 tokens per wave = one chunk
constexpr int kStepStride = kWave * kVec;           // 512
constexpr int kRowsMax = 2 * LVTV_MAX_K + 1;
constexpr float kL2E = 1.44269504088896340736f;
static_assert(kSlice * kMaxSlices >= 524288, "slice count limit covers V <= 524288");

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

// ------------------------------------------------------------------ reductions (8 waves)

template <int N>
struct Red {
  float v[kWaves][N];
};

__device__ __forceinline__ void bmax2(float& a, float& b, Red<2>& sh) {
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
  for (int w = 1; w < kWaves; ++w) {
    a = fmaxf(a, sh.v[w][0]);
    b = fmaxf(b, sh.v[w][1]);
  }
}

__device__ __forceinline__ void bsum2(float& a, float& b, Red<2>& sh) {
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
  for (int w = 1; w < kWaves; ++w) {
    a += sh.v[w][0];
    b += sh.v[w][1];
  }
}

__device__ __forceinline__ ArgMax bargmax(ArgMax x, ArgMax* sh) {
  x = wave_argmax(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = x;
  __syncthreads();
  ArgMax r = sh[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = argmax_combine(r, sh[w]);
  return r;
}

__device__ __forceinline__ double bexscan(double v, double* sh, double& total) {
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
  for (int w = 0; w < kWaves; ++w) total += sh[w];
  return pre + inc - v;
}

__device__ __forceinline__ int bmin_i(int v, int* sh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = sh[0];
  for (int w = 1; w < kWaves; ++w) r = min(r, sh[w]);
  return r;
}

// Block-wide poll of up to two ranges of tagged words into dst / have
// (concatenated). Returns true when every word was seen fresh.
struct Ranges {
  uint64_t* src0;
  uint64_t* src1;
  int n0, n1;
};

__device__ __forceinline__ bool poll(const Ranges& r, uint32_t tag, uint32_t* dst, uint8_t* have,
                                     int spin_limit) {
  const int n0 = r.n0;
  const int n = n0 + r.n1;
  for (int i = threadIdx.x; i < n; i += kThreads) have[i] = 0;
  __syncthreads();
  int round = 0;
  while (true) {
    int missing = 0;
    for (int i = threadIdx.x; i < n; i += kThreads) {
      if (!have[i]) {
        uint64_t* p = i < n0 ? r.src0 + i : r.src1 + (i - n0);
        const uint64_t w = tag_load(p);
        if (uint32_t(w >> 32) == tag) {
          dst[i] = uint32_t(w);
          have[i] = 1;
        } else {
          missing = 1;
        }
      }
    }
    if (!__syncthreads_or(missing)) return true;
    if (++round > spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ bool have4(const uint8_t* have, int e) {
  return have[4 * e] && have[4 * e + 1] && have[4 * e + 2] && have[4 * e + 3];
}

// ------------------------------------------------------------------ raw slices in registers

// A thread's share of one row slice: kSteps groups of 8 tokens, bf16 kept
// packed (one 16-byte register quad per group), fp32 as two quads.
template <int kDtype>
struct Raw {
  u32x4 q[kSteps][kDtype == 1 ? 1 : 2];
};

template <int kDtype>
__device__ __forceinline__ float elem(const Raw<kDtype>& r, int i, int j) {
  if constexpr (kDtype == 1) {
    const uint32_t w = r.q[i][0][j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(r.q[i][j >> 2][j & 3]);
  }
}

// Makes the compiler treat the raw registers as rewritten, so pass 2
// recomputes the exponentials from them instead of keeping pass 1's
// unpacked values and exponentials alive across the exchange (that would
// need four times the registers).
template <int kDtype>
__device__ __forceinline__ void launder(Raw<kDtype>& r) {
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int q = 0; q < (kDtype == 1 ? 1 : 2); ++q) asm volatile("" : "+v"(r.q[i][q]));
}

__device__ __forceinline__ int64_t elem_base(int s) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  return int64_t(s) * kSlice + wave * kSpan + lane * kVec;
}

// Streaming loads of a slice; tokens at or beyond V read as -inf. With
// kVecOk (16-byte aligned rows, V % 8 == 0) a group of 8 is either wholly
// inside the row or wholly past its end.
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void load_raw(const void* row, int64_t V, int s, Raw<kDtype>& r) {
  const int64_t base = elem_base(s);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int64_t e = base + i * kStepStride;
    if constexpr (kVecOk) {
      if (e < V) {
        if constexpr (kDtype == 1) {
          r.q[i][0] = ld_nt16(static_cast<const uint16_t*>(row) + e);
        } else {
          r.q[i][0] = ld_nt16(static_cast<const float*>(row) + e);
          r.q[i][1] = ld_nt16(static_cast<const float*>(row) + e + 4);
        }
      } else if constexpr (kDtype == 1) {
        r.q[i][0] = u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
      } else {
        r.q[i][0] = u32x4{0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
        r.q[i][1] = r.q[i][0];
      }
    } else {
      if constexpr (kDtype == 1) {
        const uint16_t* p = static_cast<const uint16_t*>(row);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t lo = (e + 2 * h < V) ? p[e + 2 * h] : 0xff80u;
          const uint32_t hi = (e + 2 * h + 1 < V) ? p[e + 2 * h + 1] : 0xff80u;
          r.q[i][0][h] = lo | (hi << 16);
        }
      } else {
        const uint32_t* p = static_cast<const uint32_t*>(row);
#pragma unroll
        for (int h = 0; h < 8; ++h) r.q[i][h >> 2][h & 3] = (e + h < V) ? p[e + h] : 0xff800000u;
      }
    }
  }
}

// Maximum of the raw logits a thread holds. Each token is unpacked exactly:
// a packed bf16 word read as one float can be a signalling-NaN pattern (two
// -inf padding tokens are), which the hardware maximum propagates. A NaN
// token may or may not surface here; it always surfaces through its
// exponential (the slice sum turns NaN).
template <int kDtype>
__device__ __forceinline__ float raw_max(const Raw<kDtype>& r) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) m = fmaxf(m, elem(r, i, j));
  return m;
}

struct SliceStats {
  float R;     // log2-domain reference fl32(m * L2E) (-inf for an all -inf slice)
  float l;     // sum of 2^(s L2E - R) over the slice
  float wsum;  // this wave's part of l (its chunk)
};

// Exponent offset for a slice reference R (0 for an all -inf slice, so its
// -inf tokens still give 0 and a NaN still gives NaN).
__device__ __forceinline__ float neg_ref(float R) { return R == -INFINITY ? 0.f : -R; }

__device__ __forceinline__ float ex(float x, float inv_t, bool unit, float nr) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(scale_logit(x, inv_t, unit), kL2E, nr));
}

// Softmax statistics of the target slice and, with kTwo, of the draft slice.
// Every thread of the block must call it.
template <int kDtype, bool kTwo>
__device__ __forceinline__ void slice_stats(Raw<kDtype>& rt, Raw<kDtype>& rd, float inv_t,
                                            bool unit, Red<2>& sh, SliceStats& st,
                                            SliceStats& sd) {
  float mt = raw_max(rt), md = kTwo ? raw_max(rd) : -INFINITY;
  launder(rt);
  if constexpr (kTwo) launder(rd);
  bmax2(mt, md, sh);
  mt = scale_logit(mt, inv_t, unit);
  md = scale_logit(md, inv_t, unit);
  const float rtf = (mt == -INFINITY) ? -INFINITY : mt * kL2E;
  const float rdf = (md == -INFINITY) ? -INFINITY : md * kL2E;
  const float nt = neg_ref(rtf), nd = neg_ref(rdf);
  float lt = 0.f, ld = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      lt += ex(elem(rt, i, j), inv_t, unit, nt);
      if constexpr (kTwo) ld += ex(elem(rd, i, j), inv_t, unit, nd);
    }
  const float wt = wave_sum(lt), wd = wave_sum(ld);
  float bt = lt, bd = ld;
  bsum2(bt, bd, sh);
  st = SliceStats{rtf, bt, wt};
  sd = SliceStats{rdf, bd, wd};
}

// Pass 2 of a pair slice: the exponentials are recomputed from the
// registers exactly as in slice_stats, scaled into p and q; alpha over the
// slice and the residual mass of this wave's chunk.
template <int kDtype>
__device__ __forceinline__ void pair_overlap(const Raw<kDtype>& rt, const Raw<kDtype>& rd,
                                             float inv_t, bool unit, float nt, float nd, float at,
                                             float ad, Red<2>& sh, float& alpha_slice,
                                             float& chunk_mass) {
  float sa = 0.f, sr = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float p = ex(elem(rt, i, j), inv_t, unit, nt) * at;
      const float q = ex(elem(rd, i, j), inv_t, unit, nd) * ad;
      const float mn = fminf(p, q);
      sa += mn;
      sr += p - mn;
    }
  chunk_mass = wave_sum(sr);
  float unused = 0.f;
  bsum2(sa, unused, sh);
  alpha_slice = sa;
}

// Argmax of one slice of raw logits (lowest index among equal values; NaN
// flagged).
template <int kDtype, bool kVecOk>
__device__ __forceinline__ ArgMax slice_argmax(const void* row, int64_t V, int s, ArgMax* sh) {
  Raw<kDtype> r;
  load_raw<kDtype, kVecOk>(row, V, s, r);
  const int64_t base = elem_base(s);
  ArgMax best{-INFINITY, INT_MAX, 0};
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int64_t idx = base + i * kStepStride + j;
      const float v = elem(r, i, j);
      if (idx < V) {
        if (isnan(v)) best.nan = 1;
        else if (v > best.v || (v == best.v && idx < best.i)) {
          best.v = v;
          best.i = int32_t(idx);
        }
      }
    }
  return bargmax(best, sh);
}

// ------------------------------------------------------------------ shared memory

constexpr int kFinWords = 4 * kMaxSlices * (LVTV_MAX_K + 1) + kMaxSlices * LVTV_MAX_K;

struct Shared {
  Red<2> red;
  ArgMax am[kWaves];
  double redd[kWaves];
  int redi[kWaves];
  float cm8[kWaves];
  // item exchange
  uint32_t words[4 * kMaxSlices];
  uint8_t have[4 * kMaxSlices];
  float at, ad;
  float Rt, Rd;
  double Lt, Ld;
  int last;
  // finalize
  uint32_t fwords[kFinWords];
  uint8_t fhave[kFinWords];
  float R[kRowsMax];
  double L[kRowsMax];
  int32_t arg[kRowsMax];
  double alpha[LVTV_MAX_K];
  double ratio[LVTV_MAX_K];
  double uacc[LVTV_MAX_K];
  float cm[kWaves * kMaxSlices];
  int j;
  int pick;
  double before;
  double scale;
};

// ------------------------------------------------------------------ recomputation

// The four statistics words a (b, k, s) workgroup publishes, recomputed from
// the inputs (bit-identical to what it publishes).
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void recompute_stat_words(const Args& a, int b, int k, int s, int kb,
                                                     float T, uint32_t (&w)[4], Shared& sh) {
  const int64_t V = a.V;
  const bool pair = k < kb;
  if (T == 0.f) {
    const ArgMax at = slice_argmax<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, sh.am);
    ArgMax ad{-INFINITY, INT_MAX, 0};
    if (pair) ad = slice_argmax<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, sh.am);
    w[0] = __float_as_uint(at.nan ? NAN : at.v);
    w[1] = uint32_t(at.i);
    w[2] = __float_as_uint(ad.nan ? NAN : ad.v);
    w[3] = uint32_t(ad.i);
    return;
  }
  const float inv_t = __fdiv_rn(1.f, T);
  const bool unit = T == 1.f;
  Raw<kDtype> rt, rd;
  SliceStats st, sd;
  load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, rt);
  if (pair) {
    load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, rd);
    slice_stats<kDtype, true>(rt, rd, inv_t, unit, sh.red, st, sd);
  } else {
    slice_stats<kDtype, false>(rt, rd, inv_t, unit, sh.red, st, sd);
  }
  w[0] = __float_as_uint(st.R);
  w[1] = __float_as_uint(st.l);
  w[2] = __float_as_uint(pair ? sd.R : 0.f);
  w[3] = __float_as_uint(pair ? sd.l : 1.f);
}

// Slice alpha and the slice's chunk masses (cm8[wave]) of (b, k, s),
// recomputed from the inputs given the row statistics.
template <int kDtype, bool kVecOk>
__device__ __forceinline__ void recompute_overlap(const Args& a, int b, int k, int s, int kb,
                                                  float T, float Rt, double Lt, float Rd,
                                                  double Ld, float& alpha_slice, Shared& sh) {
  const int64_t V = a.V;
  const bool pair = k < kb;
  const float inv_t = __fdiv_rn(1.f, T);
  const bool unit = T == 1.f;
  Raw<kDtype> rt, rd;
  SliceStats st, sd;
  float cmass;
  load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, rt);
  if (pair) {
    load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, rd);
    slice_stats<kDtype, true>(rt, rd, inv_t, unit, sh.red, st, sd);
    launder(rt);
    launder(rd);
    const float at = float(exp2((double)st.R - (double)Rt) / Lt);
    const float ad = float(exp2((double)sd.R - (double)Rd) / Ld);
    pair_overlap<kDtype>(rt, rd, inv_t, unit, neg_ref(st.R), neg_ref(sd.R), at, ad, sh.red,
                         alpha_slice, cmass);
  } else {
    slice_stats<kDtype, false>(rt, rd, inv_t, unit, sh.red, st, sd);
    const float at = float(exp2((double)st.R - (double)Rt) / Lt);
    alpha_slice = 0.f;
    cmass = st.wsum * at;
  }
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh.cm8[threadIdx.x / kWave] = cmass;
  __syncthreads();
}

// Row statistics from per-slice (R, l) words (4 words per slice, R at offset
// offR, l at offL), combined by one wave, one slice per lane: R_max = max R_s
// and L = sum_s l_s 2^(R_s - R_max) in fp64 (fixed butterfly order). Slices
// that are entirely -inf weigh 0 (their l is 0, or NaN when a NaN was
// present, which must propagate). All lanes of the wave get the result.
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
  for (int k = threadIdx.x; k <= a.Kmax; k += kThreads) out_tok[k] = -1;
  for (int k = threadIdx.x; k < a.Kmax; k += kThreads) out_alpha[k] = 0.f;
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

constexpr int kPerThread = kSpan / kThreads;  // 4 tokens of a chunk per thread

// Weights of the draw inside chunk c (fp64, from the inputs).
template <int kDtype>
__device__ __forceinline__ void chunk_weights(const void* trow, const void* drow, int64_t V,
                                              int c, float inv_t, bool unit, float Rt, double Lt,
                                              float Rd, double Ld, bool residual,
                                              double (&w)[kPerThread], int64_t& v0) {
  v0 = int64_t(c) * kSpan + threadIdx.x * kPerThread;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t v = v0 + i;
    double x = 0.0;
    if (v < V) {
      const double p = prob64<kDtype>(trow, v, inv_t, unit, Rt, Lt);
      x = residual ? fmax(0.0, p - prob64<kDtype>(drow, v, inv_t, unit, Rd, Ld)) : p;
    }
    w[i] = x;
  }
}

// Smallest token of chunk c whose cumulative weight passes `rem`. The fp64
// weights are rescaled to sum to the chunk's mass `cmass` (the unit the
// chunk was chosen in); when rounding leaves `rem` at or above that, the
// last positive-weight token of the chunk is taken.
template <int kDtype>
__device__ __forceinline__ int search_chunk(const void* trow, const void* drow, int64_t V, int c,
                                            double rem, double cmass, float inv_t, bool unit,
                                            float Rt, double Lt, float Rd, double Ld,
                                            bool residual, Shared& sh) {
  double w[kPerThread];
  int64_t v0;
  chunk_weights<kDtype>(trow, drow, V, c, inv_t, unit, Rt, Lt, Rd, Ld, residual, w, v0);
  double mine = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) mine += w[i];
  double total;
  const double exc = bexscan(mine, sh.redd, total);
  const double f = (total > 0.0 && cmass > 0.0) ? cmass / total : 1.0;
  int pick = INT_MAX, last = -1;
  double run = exc;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    run += w[i];
    if (w[i] > 0.0) {
      last = int(v0 + i);
      if (pick == INT_MAX && run * f > rem) pick = int(v0 + i);
    }
  }
  int v = bmin_i(pick, sh.redi);
  if (v == INT_MAX) {
    v = -bmin_i(last >= 0 ? -last : INT_MAX, sh.redi);
    if (v == -INT_MAX) v = int(int64_t(c) * kSpan);
  }
  return v;
}

// Inverse-CDF draw from the per-chunk masses sh.cm[0..NC).
template <int kDtype>
__device__ __forceinline__ int draw_from_masses(int NC, double u, const void* trow,
                                                const void* drow, int64_t V, float inv_t,
                                                bool unit, float Rt, double Lt, float Rd,
                                                double Ld, bool residual, Shared& sh) {
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int c = 0; c < NC; ++c) total += (double)sh.cm[c];
    const double target = u * total;
    double run = 0.0;
    int pick = -1;
    for (int c = 0; c < NC; ++c) {
      const double nxt = run + (double)sh.cm[c];
      if (nxt > target && sh.cm[c] > 0.f) {
        pick = c;
        break;
      }
      run = nxt;
    }
    if (pick < 0) {  // rounding put the target at or past the last sum
      for (int c = NC - 1; c >= 0; --c)
        if (sh.cm[c] > 0.f) {
          pick = c;
          break;
        }
      if (pick < 0) pick = 0;
      sh.before = INFINITY;
    } else {
      sh.before = target - run;
    }
    sh.pick = pick;
    sh.scale = (double)sh.cm[pick];
  }
  __syncthreads();
  const int c = sh.pick;
  const double rem = sh.before;
  const double cmass = sh.scale;
  __syncthreads();
  return search_chunk<kDtype>(trow, drow, V, c, rem, cmass, inv_t, unit, Rt, Lt, Rd, Ld,
                              residual, sh);
}

// Draw from p over the whole row when there are no chunk masses for it (a
// rejection where the residual is zero everywhere, p_j == q_j): masses of p
// per chunk in fp64 first, then the same search.
template <int kDtype>
__device__ __forceinline__ int draw_full_row(int NC, double u, const void* trow, int64_t V,
                                             float inv_t, bool unit, float Rt, double Lt,
                                             Shared& sh) {
  for (int c = 0; c < NC; ++c) {
    double w[kPerThread];
    int64_t v0;
    chunk_weights<kDtype>(trow, nullptr, V, c, inv_t, unit, Rt, Lt, 0.f, 1.0, false, w, v0);
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) mine += w[i];
    double total;
    (void)bexscan(mine, sh.redd, total);
    if (threadIdx.x == 0) sh.cm[c] = float(total);
    __syncthreads();
  }
  return draw_from_masses<kDtype>(NC, u, trow, nullptr, V, inv_t, unit, Rt, Lt, 0.f, 1.0, false,
                                  sh);
}

// ------------------------------------------------------------------ finalize

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void finalize(const Args& a, int b, int kb, float T, uint32_t epoch,
                                         Shared& sh) {
  const uint32_t tag = tag_from_epoch(epoch);
  const int S = a.S;
  const int Kmax = a.Kmax;
  const bool greedy = (T == 0.f);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int32_t* y = a.tokens + size_t(b) * Kmax;

  // draft tokens of this request
  int bad = 0;
  for (int k = threadIdx.x; k < kb; k += kThreads) bad |= (y[k] < 0 || y[k] >= a.V);
  const int status_tok = __syncthreads_or(bad) ? LVTV_STATUS_BAD_TOKEN : 0;

  // statistics words of every row ([k][s][4], k = 0..kb) and, for sampling
  // requests, the slice alphas ([k][s], k < kb), in one poll
  const int nstat = (kb + 1) * S * 4;
  Ranges rg;
  rg.src0 = a.stat + stat_idx(a, b, 0, 0);
  rg.n0 = nstat;
  rg.src1 = a.apart + apart_idx(a, b, 0, 0);
  rg.n1 = greedy ? 0 : kb * S;
  const bool all = poll(rg, tag, sh.fwords, sh.fhave, a.spin_limit);
  if (!all) {
    for (int e = 0; e < (kb + 1) * S; ++e)
      if (!have4(sh.fhave, e)) {
        uint32_t w[4];
        recompute_stat_words<kDtype, kVecOk>(a, b, e / S, e % S, kb, T, w, sh);
        __syncthreads();
        if (threadIdx.x == 0)
          for (int i = 0; i < 4; ++i) sh.fwords[4 * e + i] = w[i];
        __syncthreads();
      }
  }

  // per-row statistics; rows r = k (target, k <= kb) and r = kb + 1 + k
  // (draft, k < kb); wave w takes rows w, w + 8, ...
  int fault = 0;
  for (int r = wave; r < 2 * kb + 1; r += kWaves) {
    const bool tgt = r <= kb;
    const int k = tgt ? r : r - kb - 1;
    const int off = tgt ? 0 : 2;
    const uint32_t* words = sh.fwords + size_t(k) * S * 4;
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

  // slice alphas that did not arrive, then alpha_k
  const uint8_t* ahave = sh.fhave + nstat;
  uint32_t* awords = sh.fwords + nstat;
  if (!all) {
    for (int e = 0; e < kb * S; ++e)
      if (!ahave[e]) {
        const int k = e / S;
        float al;
        recompute_overlap<kDtype, kVecOk>(a, b, k, e % S, kb, T, sh.R[k], sh.L[k],
                                          sh.R[kb + 1 + k], sh.L[kb + 1 + k], al, sh);
        if (threadIdx.x == 0) awords[e] = __float_as_uint(al);
        __syncthreads();
      }
  }
  // accept inputs for every position in parallel: u_k and p(y_k)/q(y_k)
  if (threadIdx.x < kb) {
    const int k = threadIdx.x;
    double al = 0.0;
    for (int s = 0; s < S; ++s) al += (double)__uint_as_float(awords[k * S + s]);
    sh.alpha[k] = al;
    double u, u2;
    verify_uniforms(a.seed[b], uint64_t(b), uint64_t(k), u, u2);
    sh.uacc[k] = u;
    const int yk = y[k];
    const double p = prob64<kDtype>(row_ptr<kDtype>(a, b, true, k), yk, inv_t, unit, sh.R[k],
                                    sh.L[k]);
    const double q = prob64<kDtype>(row_ptr<kDtype>(a, b, false, k), yk, inv_t, unit,
                                    sh.R[kb + 1 + k], sh.L[kb + 1 + k]);
    // q == 0: accept iff p > 0, encoded as an infinite or zero ratio
    sh.ratio[k] = (q == 0.0) ? (p > 0.0 ? INFINITY : 0.0) : p / q;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 0; k < Kmax; ++k) out_alpha[k] = k < kb ? float(sh.alpha[k]) : 0.f;
    int j = kb;
    for (int k = 0; k < kb; ++k)
      if (!(sh.uacc[k] < sh.ratio[k])) {
        j = k;
        break;
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
  Ranges rc;
  rc.src0 = a.chunk + chunk_idx(a, b, j, 0);
  rc.n0 = NC;
  rc.src1 = a.chunk;
  rc.n1 = 0;
  if (!poll(rc, tag, sh.fwords, sh.fhave, a.spin_limit)) {
    for (int s = 0; s < S; ++s) {
      bool miss = false;
      for (int w = 0; w < kWaves; ++w) miss |= !sh.fhave[kWaves * s + w];
      if (miss) {
        float al;
        recompute_overlap<kDtype, kVecOk>(a, b, j, s, kb, T, Rt, Lt, Rd, Ld, al, sh);
        if (threadIdx.x < kWaves)
          sh.fwords[kWaves * s + threadIdx.x] = __float_as_uint(sh.cm8[threadIdx.x]);
        __syncthreads();
      }
    }
  }
  int has_mass = 0;
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    sh.cm[c] = __uint_as_float(sh.fwords[c]);
    has_mass |= sh.cm[c] > 0.f;
  }
  const bool any_mass = __syncthreads_or(has_mass);
  int v;
  if (residual && !any_mass) {
    v = draw_full_row<kDtype>(NC, u_draw, trow, V, inv_t, unit, Rt, Lt, sh);
  } else {
    v = draw_from_masses<kDtype>(NC, u_draw, trow, drow, V, inv_t, unit, Rt, Lt, Rd, Ld,
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
__device__ __forceinline__ void stochastic_item(const Args& a, int b, int k, int s, int kb,
                                                float T, uint32_t& epoch, Shared& sh) {
  const int S = a.S;
  const int64_t V = a.V;
  const bool unit = (T == 1.f);
  const float inv_t = __fdiv_rn(1.f, T);
  Raw<kDtype> rt, rd;
  load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, true, k), V, s, rt);
  if constexpr (kPair) load_raw<kDtype, kVecOk>(row_ptr<kDtype>(a, b, false, k), V, s, rd);
  epoch = read_epoch(a.ctl);
  const uint32_t tag = tag_from_epoch(epoch);
  SliceStats st, sd;
  slice_stats<kDtype, kPair>(rt, rd, inv_t, unit, sh.red, st, sd);
  launder(rt);
  if constexpr (kPair) launder(rd);
  if (threadIdx.x == 0) {
    uint64_t* w = a.stat + stat_idx(a, b, k, s);
    tag_store(w + 0, tag, __float_as_uint(st.R));
    tag_store(w + 1, tag, __float_as_uint(st.l));
    tag_store(w + 2, tag, __float_as_uint(kPair ? sd.R : 0.f));
    tag_store(w + 3, tag, __float_as_uint(kPair ? sd.l : 1.f));
  }
  // collect the statistics of every slice of these rows
  Ranges rg;
  rg.src0 = a.stat + stat_idx(a, b, k, 0);
  rg.n0 = 4 * S;
  rg.src1 = a.stat;
  rg.n1 = 0;
  const bool fresh = poll(rg, tag, sh.words, sh.have, a.spin_limit);
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
      pair_overlap<kDtype>(rt, rd, inv_t, unit, neg_ref(st.R), neg_ref(sd.R), sh.at, sh.ad,
                           sh.red, alpha_slice, cmass);
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
        recompute_stat_words<kDtype, kVecOk>(a, b, k, s2, kb, T, w, sh);
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
                                      sh);
    cmass = sh.cm8[threadIdx.x / kWave];
    __syncthreads();
  }
  if ((threadIdx.x & (kWave - 1)) == 0)
    tag_store(a.chunk + chunk_idx(a, b, k, kWaves * s + threadIdx.x / kWave), tag,
              __float_as_uint(cmass));
  if (kPair && threadIdx.x == 0)
    tag_store(a.apart + apart_idx(a, b, k, s), tag, __float_as_uint(alpha_slice));
}

template <int kDtype, bool kVecOk>
__device__ __forceinline__ void verify_body(const Args& a) {
  __shared__ Shared sh;
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
    recompute_stat_words<kDtype, kVecOk>(a, b, k, s, kb, T, w, sh);
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
    stochastic_item<kDtype, kVecOk, true>(a, b, k, s, kb, T, epoch, sh);
  } else {
    stochastic_item<kDtype, kVecOk, false>(a, b, k, s, kb, T, epoch, sh);
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
  finalize<kDtype, kVecOk>(a, b, kb, T, epoch, sh);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(a.req + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    complete_unit(a, epoch);
  }
}

// bf16 rows fit the item path in 128 registers: four waves per SIMD, two
// workgroups per compute unit.
template <bool kVecOk>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
verify_fused_bf16(Args a) {
  verify_body<1, kVecOk>(a);
}

template <bool kVecOk>
__global__ __launch_bounds__(kThreads) void verify_fused_f32(Args a) {
  verify_body<0, kVecOk>(a);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  int S, NC;
  size_t off_stat, off_apart, off_chunk, total;
};

Layout make_layout(int B, int Kmax, int V) {
  Layout L;
  L.S = (V + kSlice - 1) / kSlice;
  L.NC = L.S * kWaves;
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
  if constexpr (kDtype == 1)
    hipLaunchKernelGGL((verify_fused_bf16<kVecOk>), dim3(unsigned(grid)), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((verify_fused_f32<kVecOk>), dim3(unsigned(grid)), dim3(kThreads), 0,
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
