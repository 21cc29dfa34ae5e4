// Single-read verify kernel for gfx950 (bf16 logits): a persistent grid that
// streams every used row pair once, holding it on chip between the row
// statistics and the overlap pass.
//
// A row (or row pair: target row k and draft row k of one request) is cut
// into S slices of two 4096-token tiles. One item is one slice of one used
// row: 16 KB of each row, one 8-token group per row for each of a
// workgroup's 1024 threads (thread T takes tile 2 s + T / 512, group
// T mod 512). A preparation kernel lists the used rows as 16-byte records
// (and clears the exchange words); items are numbered row by row in that
// list, and workgroup w of the G resident ones (one per compute unit) takes
// items w, w + G, w + 2 G, ..., so the slices of one row are in flight at the
// same time on different compute units.
//
// Each workgroup keeps three items in flight in four register slots and
// holds a sampling item's groups in an LDS ring from its statistics to its
// overlap pass, two iterations later. Iteration j
//   1. polls the tagged words of item j - 1's row (wave 0),
//   2. issues item j + 3's loads (every iteration issues the same loads:
//      past the row's end, for the draft row of a bonus row and for items
//      past the end they read addresses the batch reads anyway),
//   3. combines the slice statistics of item j - 2's row from the words
//      polled one iteration earlier (wave 0, fixed lane order) into the
//      row's R and L,
//   4. computes item j's slice statistics (per row: maximum raw logit M_s
//      and L_s = sum 2^(x c - M_s c)) and publishes them as tagged words, or
//      for greedy rows the slice's argmax of both rows as a plain record,
//   5. runs item j - 2's overlap pass from the ring: p, q, the slice's part
//      of alpha and the residual mass of each of its 512-token chunks.
// Vector memory operations complete in issue order; the waits of steps 3
// and 4 are for the words polled in iteration j - 1 and item j's loads, so
// items j + 1 .. j + 3 stay in flight through the iteration. The barriers
// wait for LDS only.
//
// In iteration j a workgroup waits only for the row of item j - 2, whose
// slices the other workgroups publish in their iterations j - 3 .. j - 1
// (the row straddles at most two rounds of the grid), each before its own
// wait of that iteration; so with every workgroup resident no wait can be
// circular. Each wait is still bounded: past the spin limit the row is
// marked unfinished and the finalize recomputes it from memory with the
// same functions and the same reduction order, which gives the same bits.
//
// Arithmetic per row as the row kernel's (base-2 exponentials, R = fl32(M c),
// p = 2^(x c - R - log2 L)); the row's L is the fp64 sum over slices, in
// slice order, of L_s 2^(fl32(M_s c) - fl32(M c)).
#pragma once

#include "verify_common.hpp"

namespace lvtv {
namespace vr {
namespace {

constexpr int kSThreads = 1024;                 // threads of a stream workgroup
constexpr int kSWaves = kSThreads / kWave;      // 16
constexpr int kSTiles = kSThreads / kThreads;   // 2 tiles per item
constexpr int kPollWords = 2;                   // tagged words a lane polls
constexpr int kMaxSlices = 16 * kPollWords;     // 4 words per slice, 64 lanes
constexpr int kSlots = 4;                       // register slots: the item worked on, three in flight
constexpr uint32_t kStreamTag = 1u;             // the words are cleared at the start of every call

enum : int { kNone = 0, kPairS = 1, kBonusS = 2, kPairG = 3, kBonusG = 4 };

__device__ __forceinline__ bool is_pair(int kind) { return kind == kPairS || kind == kPairG; }
__device__ __forceinline__ bool is_sampling(int kind) { return kind == kPairS || kind == kBonusS; }

struct Item {
  int r, s;  // target row and slice
  int dr;    // draft row
  int kind;  // kNone past the end
  float T;
};

struct StreamShared {
  float st[kSWaves][2];   // slice statistics: wave maxima, then wave sums
  float st2[kSWaves][2];
  float al[kSWaves];      // wave parts of alpha
  float ga_v[kSWaves][2];
  int ga_i[kSWaves][2];
  int ga_n[kSWaves][2];
  float row[4];           // combined row statistics: Rt, Lt, Rd, Ld
  float nr[2];            // references of the overlap pass: nr_t, nr_d
  int row_ok;
};

// LDS barrier that does not wait for vector memory: outstanding global loads
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Read-only input that every lane reads at the same address: a scalar load
// (the inputs are not written while the kernel runs).
template <class T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ Item item_at(const Args& a, int i, int n_items) {
  i = uni(i);
  Item it{0, 0, 0, kNone, 0.f};
  if (i >= n_items) return it;
  const int u = uni(i / a.S);
  const int32_t* rec = reinterpret_cast<const int32_t*>(a.recs) + 4 * u;
  it.r = uni(sload(rec));
  it.s = uni(i - u * a.S);
  it.dr = uni(sload(rec + 1));
  it.kind = uni(sload(rec + 2));
  it.T = __int_as_float(uni(sload(rec + 3)));
  return it;
}

// Exponent scale c = fl32(log2(e) fl32(1/T)) (log2(e) itself at T = 1).
__device__ __forceinline__ float exp_scale(float T) {
  return (T == 1.f) ? kL2E : __fmul_rn(kL2E, __fdiv_rn(1.f, T));
}

// First token of group t (0 .. 511) of tile gt.
__device__ __forceinline__ int grp_elem(int gt, int t) { return gt * kTile + t * kVec; }

// ------------------------------------------------------------------ loads

// One row's group of an item: the rows hold whole groups (V is a multiple
// of 8, rows 16-byte aligned), a tile past the row's last one reads the last
// tile and a group past the row's end its last group; masked on arrival.
__device__ __forceinline__ void stream_grp(const void* row, int V, int n_tiles, int gt, int t,
                                           Grp<1>& g) {
  const int e = grp_elem(min(gt, n_tiles - 1), t);
  const int ee = e < V ? e : V - kVec;
  g.q[0] = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + size_t(ee) * 2));
}

struct Slot {
  Grp<1> t, d;
};

// An item's loads for group t of sub-tile sub, the same for every item: the
// draft group of a bonus row reads the target row, an item past the end
// (kind kNone) the first tiles of target row 0.
__device__ __forceinline__ void item_load(const Args& a, const Item& it, int sub, int t, Slot& sl) {
  const bool real = it.kind != kNone;
  const char* trow = static_cast<const char*>(a.target) +
                     (real ? int64_t(it.r) * int64_t(a.V) * 2 : int64_t(0));
  const char* drow = is_pair(it.kind)
                         ? static_cast<const char*>(a.draft) + int64_t(it.dr) * int64_t(a.V) * 2
                         : trow;
  const int gt = (real ? it.s * kSTiles : 0) + sub;
  stream_grp(trow, a.V, a.n_tiles, gt, t, sl.t);
  stream_grp(drow, a.V, a.n_tiles, gt, t, sl.d);
}

// Tokens past the row (and every token of a tile past the last one) read as
// -inf; the draft group of a bonus row too. Selects, not branches.
__device__ __forceinline__ void select_grp(Grp<1>& g, bool keep) {
#pragma unroll
  for (int i = 0; i < 4; ++i) g.q[0][i] = keep ? g.q[0][i] : 0xff80ff80u;
}

__device__ __forceinline__ void item_mask(const Args& a, const Item& it, int sub, int t, Slot& sl) {
  const int gt = it.s * kSTiles + sub;
  const bool in = gt < a.n_tiles && grp_elem(gt, t) < a.V;
  select_grp(sl.t, in);
  select_grp(sl.d, in && is_pair(it.kind));
}

// Makes the slot's loads complete here (no code: the registers are inputs).
__device__ __forceinline__ void touch(const Slot& s) {
  asm volatile("" ::"v"(s.t.q[0]), "v"(s.d.q[0]));
}

// ------------------------------------------------------------------ slice statistics

// A thread's maximum m of the raw logits of one group and
// l = sum 2^(x c - fl32(m c)) (0 while m = -inf).
__device__ __forceinline__ void grp_ml(const Grp<1>& g, float c, float& m, float& l) {
  float x[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) x[j] = gelem(g, j);
  m = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  const float nr = (m == -INFINITY) ? 0.f : -(m * c);
  float e[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, nr));
  l = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// Weight of a thread's sum under the slice maximum M: l 2^(fl32(m c) - fl32(M c)).
__device__ __forceinline__ float grp_weight(float m, float l, float M, float c) {
  return (m == -INFINITY) ? l * 0.f : l * __builtin_amdgcn_exp2f(m * c - M * c);
}

// Slice statistics out = {M_t, L_t, M_d, L_d} from the per-thread values of
// the 16 waves (wave w of the stream workgroup: sub-tile w / 8, wave w mod 8
// of the tile): the block maximum, then L_s = the fp32 sum over waves, in
// wave order, of the wave sums of the threads' weights. Every thread of the
// stream kernel calls it with its own values.
__device__ __forceinline__ void slice_stats(float mt, float lt, float md, float ld, float c,
                                            StreamShared& sh, float (&out)[4]) {
  const int wave = threadIdx.x / kWave;
  const float Mtw = wmax(mt), Mdw = wmax(md);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.st[wave][0] = Mtw;
    sh.st[wave][1] = Mdw;
  }
  lds_barrier();
  float Mt = sh.st[0][0], Md = sh.st[0][1];
#pragma unroll
  for (int w = 1; w < kSWaves; ++w) {
    Mt = fmaxf(Mt, sh.st[w][0]);
    Md = fmaxf(Md, sh.st[w][1]);
  }
  const float Stw = wsum(grp_weight(mt, lt, Mt, c)), Sdw = wsum(grp_weight(md, ld, Md, c));
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.st2[wave][0] = Stw;
    sh.st2[wave][1] = Sdw;
  }
  lds_barrier();
  float St = sh.st2[0][0], Sd = sh.st2[0][1];
#pragma unroll
  for (int w = 1; w < kSWaves; ++w) {
    St += sh.st2[w][0];
    Sd += sh.st2[w][1];
  }
  out[0] = Mt;
  out[1] = St;
  out[2] = Md;
  out[3] = Sd;
}

// The reference of the overlap pass: p = 2^(x c + nr), nr = -(R + log2 L),
// in fp32 (the rounding is a common factor of the row's probabilities); 0
// for an all -inf row (every p is then 0).
__device__ __forceinline__ float neg_ref(float R, float L) {
  return (R == -INFINITY) ? 0.f : -(R + __builtin_amdgcn_logf(L));
}

// Row statistics from the slice statistics (wave 0; lane s holds slice s's
// {M_t, L_t, M_d, L_d}, lanes past the last slice {-inf, 0, -inf, 0}):
// M = the largest M_s; L = sum over lanes, in the wave's fixed reduction
// order and in fp64, of L_s 2^(fl32(M_s c) - fl32(M c)). Lane 0 writes
// {R_t, L_t, R_d, L_d} (R = fl32(M c), -inf for an all -inf row) and the
// references nr_t, nr_d to LDS.
__device__ __forceinline__ void combine_slices(const float (&v)[4], float c, StreamShared& sh) {
  const float Mt = wmax(v[0]), Md = wmax(v[2]);
  const double wt = (v[0] == -INFINITY) ? (double)v[1] * 0.0
                                        : (double)v[1] * (double)__builtin_amdgcn_exp2f(v[0] * c - Mt * c);
  const double wd = (v[2] == -INFINITY) ? (double)v[3] * 0.0
                                        : (double)v[3] * (double)__builtin_amdgcn_exp2f(v[2] * c - Md * c);
  const double Lt = wsum(wt), Ld = wsum(wd);
  if (threadIdx.x == 0) {
    const float Rt = (Mt == -INFINITY) ? -INFINITY : Mt * c;
    const float Rd = (Md == -INFINITY) ? -INFINITY : Md * c;
    sh.row[0] = Rt;
    sh.row[1] = (float)Lt;
    sh.row[2] = Rd;
    sh.row[3] = (float)Ld;
    sh.nr[0] = neg_ref(Rt, (float)Lt);
    sh.nr[1] = neg_ref(Rd, (float)Ld);
  }
}

// ------------------------------------------------------------------ polls

// The tagged words of one row a lane of wave 0 polls: words l and l + 64 of
// the row's 4 S (lanes past the end read word 0 again).
struct Poll {
  uint64_t w[kPollWords];
};

__device__ __forceinline__ void poll_issue(const Args& a, const Item& it, Poll& p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nw = 4 * a.S;
  uint64_t* row = a.words + size_t(is_sampling(it.kind) ? it.r : 0) * a.S * 4;
#pragma unroll
  for (int q = 0; q < kPollWords; ++q) {
    const int i = lane + q * kWave;
    p.w[q] = tag_load(row + (i < nw ? i : 0));
  }
}

__device__ __forceinline__ void touch_poll(const Poll& p) {
#pragma unroll
  for (int q = 0; q < kPollWords; ++q) asm volatile("" ::"v"(p.w[q]));
}

__device__ __forceinline__ bool poll_fresh(const Args& a, const Poll& p) {
  const int lane = threadIdx.x & (kWave - 1);
  bool f = true;
#pragma unroll
  for (int q = 0; q < kPollWords; ++q)
    f = f && (lane + q * kWave >= 4 * a.S || uint32_t(p.w[q] >> 32) == kStreamTag);
  return f;
}

// Combines the slice statistics of a row from its polled words (wave 0):
// lane s gathers slice s's words 4 s .. 4 s + 3 (word (4 s + q) mod 64 of
// poll register (4 s + q) / 64).
__device__ __forceinline__ void combine_words(const Args& a, const Poll& p, float c,
                                              StreamShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int src = (4 * lane + q) & (kWave - 1);
    const float x0 = __shfl(__uint_as_float(uint32_t(p.w[0])), src, kWave);
    const float x1 = __shfl(__uint_as_float(uint32_t(p.w[1])), src, kWave);
    const float y = lane < 16 ? x0 : x1;
    v[q] = lane < a.S ? y : ((q & 1) ? 0.f : -INFINITY);
  }
  combine_slices(v, c, sh);
}

// Row statistics of item it's row (wave 0) from the words polled one
// iteration earlier, or, if some slice's words are not there yet, from
// words polled again (into other registers) until they are, bounded by the
// spin limit (then row_ok = 0).
__device__ __forceinline__ void row_combine(const Args& a, const Item& it, const Poll& pin,
                                            StreamShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  bool ok = true;
  if (__all(poll_fresh(a, pin))) {
    combine_words(a, pin, exp_scale(it.T), sh);
  } else {
    Poll p;
    for (int spin = 0;; ++spin) {
      if (spin >= a.spin_limit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      poll_issue(a, it, p);
      if (__all(poll_fresh(a, p))) break;
    }
    if (ok) combine_words(a, p, exp_scale(it.T), sh);
  }
  if (lane == 0) sh.row_ok = ok ? 1 : 0;
}

// ------------------------------------------------------------------ overlap pass

// A thread's part of a slice's overlap pass: p = 2^(x c + nrt) and (pair
// rows) q = 2^(x c + nrd) of its group; returns its part of alpha (sum of
// min(p, q)) and sets r to the group's residual mass max(0, p - q) (p for a
// bonus row).
template <bool kPair>
__device__ __forceinline__ float grp_overlap(const Grp<1>& gt, const Grp<1>& gd, float c,
                                             float nrt, float nrd, float& r) {
  float mn[kVec], res[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(gelem(gt, j), c, nrt));
    if constexpr (kPair) {
      const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(gelem(gd, j), c, nrd));
      mn[j] = fminf(p, q);
      res[j] = p - mn[j];
    } else {
      mn[j] = 0.f;
      res[j] = p;
    }
  }
  r = ((res[0] + res[1]) + (res[2] + res[3])) + ((res[4] + res[5]) + (res[6] + res[7]));
  return ((mn[0] + mn[1]) + (mn[2] + mn[3])) + ((mn[4] + mn[5]) + (mn[6] + mn[7]));
}

// Chunk mass of one wave's 512 tokens of tile gt (lane 0 writes it).
__device__ __forceinline__ void put_chunk(float* chunk_row, int gt, int n_tiles, int t, float r) {
  const float cm = wsum(r);
  if ((t & (kWave - 1)) == 0 && gt < n_tiles) chunk_row[gt * kWaves + t / kWave] = cm;
}

// Alpha of a slice: the fp32 sum, in wave order, of the 16 wave sums.
__device__ __forceinline__ float slice_alpha(StreamShared& sh) {
  lds_barrier();
  float r = sh.al[0];
#pragma unroll
  for (int i = 1; i < kSWaves; ++i) r += sh.al[i];
  return r;
}

// ------------------------------------------------------------------ greedy slices

// A thread's argmax over one group (tokens past the row are -inf already and
// never win); NaN values are flagged and left out.
__device__ __forceinline__ void grp_argmax(const Grp<1>& g, int e, float& bv, int& bi, int& nan) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const float v = gelem(g, j);
    nan |= (v != v);
    if (v > bv) {
      bv = v;
      bi = e + j;
    }
  }
}

__device__ __forceinline__ void slice_argmax(const Args& a, const Item& it, int sub, int t,
                                             const Slot& sl, StreamShared& sh) {
  float vt = -INFINITY, vd = -INFINITY;
  int at = INT_MAX, ad = INT_MAX, nt = 0, nd = 0;
  const int gt = it.s * kSTiles + sub;
  const int e = grp_elem(gt, t);
  const bool pair = is_pair(it.kind);
  grp_argmax(sl.t, e, vt, at, nt);
  grp_argmax(sl.d, e, vd, ad, nd);
  // a thread whose tokens are all -inf reports its first in-range token
  if (gt < a.n_tiles && e < a.V) {
    if (at == INT_MAX) at = e;
    if (ad == INT_MAX) ad = e;
  }
  const ArgMax xt = wargmax(ArgMax{vt, at, nt});
  const ArgMax xd = wargmax(ArgMax{vd, ad, nd});
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.ga_v[wave][0] = xt.v;
    sh.ga_i[wave][0] = xt.i;
    sh.ga_n[wave][0] = xt.nan;
    sh.ga_v[wave][1] = xd.v;
    sh.ga_i[wave][1] = xd.i;
    sh.ga_n[wave][1] = xd.nan;
  }
  lds_barrier();
  if (threadIdx.x == 0) {
    ArgMax rt{sh.ga_v[0][0], sh.ga_i[0][0], sh.ga_n[0][0]};
    ArgMax rd{sh.ga_v[0][1], sh.ga_i[0][1], sh.ga_n[0][1]};
    for (int w = 1; w < kSWaves; ++w) {
      rt = argmax_combine(rt, ArgMax{sh.ga_v[w][0], sh.ga_i[w][0], sh.ga_n[w][0]});
      rd = argmax_combine(rd, ArgMax{sh.ga_v[w][1], sh.ga_i[w][1], sh.ga_n[w][1]});
    }
    GArg g;
    g.vt = rt.v;
    g.it = rt.i;
    g.vd = pair ? rd.v : -INFINITY;
    g.id = pair ? rd.i : INT_MAX;
    g.nan = (rt.nan ? 1 : 0) | (pair && rd.nan ? 2 : 0);
    a.garg[size_t(it.r) * a.S + it.s] = g;
  }
}

// ------------------------------------------------------------------ the pipeline step

// The LDS ring that holds a sampling item's groups from its statistics to
// its overlap pass: kSlots slots of 2 x 16 bytes per thread, laid out
// [slot][row][thread] so a wave's 16-byte accesses are contiguous. Every
// thread reads back only what it wrote itself.
struct Ring {
  u32x4 w[kSlots][2][kSThreads];
};

__device__ __forceinline__ void ring_put(Ring& r, int slot, const Slot& s) {
  r.w[slot][0][threadIdx.x] = s.t.q[0];
  r.w[slot][1][threadIdx.x] = s.d.q[0];
}

__device__ __forceinline__ void ring_get(const Ring& r, int slot, Slot& s) {
  s.t.q[0] = r.w[slot][0][threadIdx.x];
  s.d.q[0] = r.w[slot][1][threadIdx.x];
}

// One iteration j of the stream loop. On entry cur is item j (its loads
// issued three iterations ago into sc), nld is item j - 1 (whose slot sl
// takes item j + 3's loads), h1 is item j - 2; pin holds the words of item
// j - 2's row polled in iteration j - 1 (wave 0).
__device__ __forceinline__ void stream_step(const Args& a, StreamShared& sh, Ring& ring,
                                            int n_items, int& next, Item& nxt, const Item& cur,
                                            Slot& sc, int cslot, Item& nld, Slot& sl, Item& h1,
                                            Item& h2, Poll& pin, Poll& pout) {
  const int sub = threadIdx.x / kThreads, t = threadIdx.x % kThreads;
  const bool w0 = threadIdx.x < kWave;
  lds_barrier();  // every LDS value of the previous iteration has been read
  h2 = h1;
  h1 = nld;
  // 1. item j - 1's row (wave 0)
  if (w0) poll_issue(a, h1, pout);
  asm volatile("" ::: "memory");
  // 2. item j + 3
  nld = nxt;
  item_load(a, nld, sub, t, sl);
  asm volatile("" ::: "memory");
  nxt = item_at(a, next, n_items);
  next += gridDim.x;
  // 3. item j - 2's row statistics (wave 0); the words land here on every
  //    path (no register of a load in flight is reused before it lands)
  const bool h2_s = is_sampling(h2.kind);
  if (w0) {
    if (h2_s) row_combine(a, h2, pin, sh);
    touch_poll(pin);
  }
  // 4. item j's statistics (their barriers also publish step 3's LDS
  //    values); item j's loads land here on every path
  touch(sc);
  if (cur.kind == kNone) {
    lds_barrier();
  } else {
    item_mask(a, cur, sub, t, sc);
    if (is_sampling(cur.kind)) {
      const float c = exp_scale(cur.T);
      float mt, lt, md, ld;
      grp_ml(sc.t, c, mt, lt);
      grp_ml(sc.d, c, md, ld);
      float st[4];
      slice_stats(mt, lt, md, ld, c, sh, st);
      if (threadIdx.x == 0) {
        uint64_t* w = a.words + (size_t(cur.r) * a.S + cur.s) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) tag_store(w + q, kStreamTag, __float_as_uint(st[q]));
      }
      ring_put(ring, cslot, sc);
    } else {
      slice_argmax(a, cur, sub, t, sc, sh);
    }
  }
  // 5. item j - 2's overlap pass
  if (h2_s) {
    if (sh.row_ok) {
      const float c = exp_scale(h2.T);
      const float nrt = sh.nr[0], nrd = sh.nr[1];
      const RowStat rst{sh.row[0], sh.row[1], sh.row[2], sh.row[3]};
      Slot sp;
      ring_get(ring, (cslot + kSlots - 2) % kSlots, sp);
      const int gt = h2.s * kSTiles + sub;
      float* chunk_row = a.chunk + size_t(h2.r) * a.NC;
      float r;
      const float sa = (h2.kind == kPairS) ? grp_overlap<true>(sp.t, sp.d, c, nrt, nrd, r)
                                           : grp_overlap<false>(sp.t, sp.d, c, nrt, 0.f, r);
      put_chunk(chunk_row, gt, a.n_tiles, t, r);
      const float w = wsum(sa);
      if ((threadIdx.x & (kWave - 1)) == 0) sh.al[threadIdx.x / kWave] = w;
      const float al = slice_alpha(sh);
      if (threadIdx.x == 0) {
        a.apart[size_t(h2.r) * a.S + h2.s] = al;
        if (h2.s == 0) a.rstat[h2.r] = rst;
      }
    } else if (threadIdx.x == 0) {
      a.unfinished[h2.r] = 1u;
    }
  }
}

__global__ __launch_bounds__(kSThreads) void verify_stream(Args a) {
  __shared__ StreamShared sh;
  __shared__ Ring ring;
  const int n_items = sload(a.n_used) * a.S;
  if (int(blockIdx.x) >= n_items) return;
  const int sub = threadIdx.x / kThreads, t = threadIdx.x % kThreads;
  const Item none{0, 0, 0, kNone, 0.f};
  Slot s0, s1, s2, s3;
  Poll pa, pb;
  int next = blockIdx.x;
  Item i0 = item_at(a, next, n_items);
  next += gridDim.x;
  item_load(a, i0, sub, t, s0);
  Item i1 = item_at(a, next, n_items);
  next += gridDim.x;
  item_load(a, i1, sub, t, s1);
  Item i2 = item_at(a, next, n_items);
  next += gridDim.x;
  // the state the loop's back edge carries: the poll of the last iteration
  // (here of nothing) issued before the last item's loads
  if (threadIdx.x < kWave) poll_issue(a, none, pa);
  item_load(a, i2, sub, t, s2);
  Item nxt = item_at(a, next, n_items);
  next += gridDim.x;
  Item i3 = none, h1 = none, h2 = none;
  // four copies of the step, so that every slot is a fixed set of registers:
  // item j in slot j mod 4, whose previous item (j - 4) has gone to the ring
  // or finished. The loop ends once items j, j - 1 and j - 2 are past the end.
  for (;;) {
    if (i0.kind == kNone && i3.kind == kNone && h1.kind == kNone) break;
    stream_step(a, sh, ring, n_items, next, nxt, i0, s0, 0, i3, s3, h1, h2, pa, pb);
    if (i1.kind == kNone && i0.kind == kNone && h1.kind == kNone) break;
    stream_step(a, sh, ring, n_items, next, nxt, i1, s1, 1, i0, s0, h1, h2, pb, pa);
    if (i2.kind == kNone && i1.kind == kNone && h1.kind == kNone) break;
    stream_step(a, sh, ring, n_items, next, nxt, i2, s2, 2, i1, s1, h1, h2, pa, pb);
    if (i3.kind == kNone && i2.kind == kNone && h1.kind == kNone) break;
    stream_step(a, sh, ring, n_items, next, nxt, i3, s3, 3, i2, s2, h1, h2, pb, pa);
  }
}

// Preparation of the stream kernel: every workgroup zeroes part of the
// tagged words and row flags (a fill kernel, so a captured graph holds no
// memset node); workgroup 0 also lists the used rows (the rows 0 .. K_b of
// every request whose K_b and temperature are valid, request by request) as
// records, and their count.
__global__ __launch_bounds__(1024) void stream_prep(Args a, u32x4* w, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    w[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x != 0) return;
  __shared__ int part[1024 / kWave];
  __shared__ int base;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  const bool packed = a.toff != nullptr;
  const bool offs_ok = !packed || *a.packed_ok;
  for (int b0 = 0; b0 < a.B; b0 += 1024) {
    const int b = b0 + int(threadIdx.x);
    int n = 0, first = 0, kb = 0;
    float T = 0.f;
    if (b < a.B && offs_ok) {
      kb = packed ? a.toff[b + 1] - a.toff[b] - 1 : a.kreq[b];
      T = a.temp[b];
      if (kb >= 0 && kb <= a.Kmax && temperature_ok(T)) {
        n = kb + 1;
        first = packed ? a.toff[b] : b * (a.Kmax + 1);
      }
    }
    // block exclusive scan of n, in request order
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = n;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int pre = base;
    for (int q = 0; q < wave; ++q) pre += part[q];
    const int ex = pre + inc - n;
    for (int k = 0; k < n; ++k) {
      RowRec rec;
      rec.r = first + k;
      rec.dr = packed ? first + k - b : b * a.Kmax + k;
      rec.kind = (T == 0.f) ? (k < kb ? kPairG : kBonusG) : (k < kb ? kPairS : kBonusS);
      rec.T = T;
      a.recs[ex + k] = rec;
    }
    __syncthreads();
    if (threadIdx.x == 1023) base = ex + n;
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.n_used = base;
}

// ------------------------------------------------------------------ repair and gather (finalize)

// Recomputes one sampling row the stream kernel left unfinished, streaming
// it from memory with the finalize's 512 threads: thread t takes group t of
// both tiles of a slice and stands for the stream kernel's threads t and
// 512 + t, so the wave reductions, and the sums over the 16 waves in wave
// order, are the stream kernel's. Every slice's statistics, their
// combination in the same lane order, then every slice's overlap pass (chunk
// masses and parts of alpha) and the row record. Every thread of the block
// calls it.
__device__ __forceinline__ void repair_stream_row(const Args& a, int b, int k, int kb, float T,
                                                  StreamShared& sh) {
  const int r = int(target_row(a, b, k));
  Item it{r, 0, int(draft_row(a, b, k)), k < kb ? kPairS : kBonusS, T};
  const float c = exp_scale(T);
  const int t = threadIdx.x, wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  float mine[4] = {-INFINITY, 0.f, -INFINITY, 0.f};  // thread s < S keeps slice s's statistics
  for (int s = 0; s < a.S; ++s) {
    it.s = s;
    float mt[kSTiles], lt[kSTiles], md[kSTiles], ld[kSTiles];
#pragma unroll
    for (int h = 0; h < kSTiles; ++h) {
      Slot sl;
      item_load(a, it, h, t, sl);
      item_mask(a, it, h, t, sl);
      grp_ml(sl.t, c, mt[h], lt[h]);
      grp_ml(sl.d, c, md[h], ld[h]);
      const float Mtw = wmax(mt[h]), Mdw = wmax(md[h]);
      if (lane == 0) {
        sh.st[h * kWaves + wave][0] = Mtw;
        sh.st[h * kWaves + wave][1] = Mdw;
      }
    }
    lds_barrier();
    float Mt = sh.st[0][0], Md = sh.st[0][1];
    for (int w = 1; w < kSWaves; ++w) {
      Mt = fmaxf(Mt, sh.st[w][0]);
      Md = fmaxf(Md, sh.st[w][1]);
    }
#pragma unroll
    for (int h = 0; h < kSTiles; ++h) {
      const float Stw = wsum(grp_weight(mt[h], lt[h], Mt, c));
      const float Sdw = wsum(grp_weight(md[h], ld[h], Md, c));
      if (lane == 0) {
        sh.st2[h * kWaves + wave][0] = Stw;
        sh.st2[h * kWaves + wave][1] = Sdw;
      }
    }
    lds_barrier();
    float St = sh.st2[0][0], Sd = sh.st2[0][1];
    for (int w = 1; w < kSWaves; ++w) {
      St += sh.st2[w][0];
      Sd += sh.st2[w][1];
    }
    if (t == s) {
      mine[0] = Mt;
      mine[1] = St;
      mine[2] = Md;
      mine[3] = Sd;
    }
    lds_barrier();
  }
  if (t < kWave) combine_slices(mine, c, sh);
  lds_barrier();
  const float Rt = sh.row[0], Lt = sh.row[1], Rd = sh.row[2], Ld = sh.row[3];
  const bool pair = k < kb;
  const float nrt = sh.nr[0], nrd = pair ? sh.nr[1] : 0.f;
  float* chunk_row = a.chunk + size_t(r) * a.NC;
  for (int s = 0; s < a.S; ++s) {
    it.s = s;
#pragma unroll
    for (int h = 0; h < kSTiles; ++h) {
      Slot sl;
      item_load(a, it, h, t, sl);
      item_mask(a, it, h, t, sl);
      float rr;
      const float sa = pair ? grp_overlap<true>(sl.t, sl.d, c, nrt, nrd, rr)
                            : grp_overlap<false>(sl.t, sl.d, c, nrt, 0.f, rr);
      put_chunk(chunk_row, s * kSTiles + h, a.n_tiles, t, rr);
      const float w = wsum(sa);
      if (lane == 0) sh.al[h * kWaves + wave] = w;
    }
    const float al = slice_alpha(sh);
    if (t == 0) a.apart[size_t(r) * a.S + s] = al;
    lds_barrier();
  }
  if (t == 0) a.rstat[r] = RowStat{Rt, Lt, Rd, Ld};
  __syncthreads();
}

// The row record of target row k of request b from the stream kernel's
// records: greedy rows combine the slices' argmaxes in slice order; sampling
// rows take the row statistics, alpha as the fp64 sum of the slices' parts
// in slice order, and (draft rows) the accept ratio p(y_k)/q(y_k) in fp64.
__device__ __forceinline__ RowOut gather_stream_row(const Args& a, int b, int k, int kb,
                                                    bool greedy, float inv_t, bool unit) {
  const size_t r = size_t(target_row(a, b, k));
  RowOut o{0.f, 0.f, 0.f, 0.f, 0.f, 0, -1, -1};
  if (greedy) {
    const GArg* g = a.garg + r * a.S;
    ArgMax t{g[0].vt, g[0].it, g[0].nan & 1}, d{g[0].vd, g[0].id, g[0].nan & 2};
    for (int s = 1; s < a.S; ++s) {
      t = argmax_combine(t, ArgMax{g[s].vt, g[s].it, g[s].nan & 1});
      d = argmax_combine(d, ArgMax{g[s].vd, g[s].id, g[s].nan & 2});
    }
    o.Rt = t.v;
    o.arg_t = t.i;
    o.Rd = k < kb ? d.v : 0.f;
    o.arg_d = k < kb ? d.i : -1;
    o.nan = (t.nan ? 1 : 0) | (k < kb && d.nan ? 2 : 0);
    return o;
  }
  const RowStat st = a.rstat[r];
  o.Rt = st.Rt;
  o.Lt = st.Lt;
  if (k < kb) {
    o.Rd = st.Rd;
    o.Ld = st.Ld;
    double al = 0.0;
    for (int s = 0; s < a.S; ++s) al += (double)a.apart[r * a.S + s];
    o.alpha = (float)al;
    const int y = a.tokens[draft_row(a, b, k)];
    if (y >= 0 && y < a.V) {
      const KeepRow all = keep_all();
      const double p = prob64_of(load1<1>(row_ptr<1>(a, b, true, k), y), y, inv_t, unit, st.Rt,
                                 st.Lt, all);
      const double q = prob64_of(load1<1>(row_ptr<1>(a, b, false, k), y), y, inv_t, unit, st.Rd,
                                 st.Ld, all);
      set_ratio(o, accept_ratio(p, q));
    }
  } else {
    o.Rd = 0.f;
    o.Ld = 1.f;
  }
  return o;
}

}  // namespace
}  // namespace vr
}  // namespace lvtv
