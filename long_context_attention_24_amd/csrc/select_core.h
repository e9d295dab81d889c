// Exact top-k selection building blocks of the selection kernels (topk.hip).
// "DeepSeek V4 技术解读", §2.1: per query token the Lightning Indexer keeps the
// top-k compressed entries.
//
// Rule: the min(k, V) visible entries with the largest scores, ties to the
// lower index, -0.0 equal to +0.0, returned in ascending index order and
// padded with -1.
//
// Every block-wide routine is written for NW waves of one workgroup and uses
// a SelScratch object in LDS that the calling kernel owns; routines that
// produce output call an emitter: put(slot, entry, score) for slot
// 0 .. n_sel - 1 in ascending entry order, then pad(slot) for n_sel .. k - 1.
// Only integer LDS atomics (counts) are used, so results are deterministic.
#pragma once

#include <float.h>

#include "device_common.h"

namespace csa {
namespace sel {

constexpr int kBins = 2048;
constexpr int kMaxWaves = 16;
constexpr float kPosInf = __builtin_inff();
constexpr int kBrute = 256;                       // bin size finished by pairwise ranks
constexpr int kMaxBoundedN = 262144;              // longest row with chunk reports in registers

typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) int lds_int;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;

// Reduction slots, histogram and small tables of one workgroup.
struct SelScratch {
  int hist[kBins];
  float f0[2][kMaxWaves];
  float f1[2][kMaxWaves];
  uint32_t u[2][kMaxWaves];
  uint32_t tab[1024];                 // segment offsets, then threshold candidates
  int bstar, bstar_above, bstar_cnt;
  float lo, hi;                       // a row's bound and top, shared by its waves
  int last;                           // this workgroup arrived last at the row's counter
  uint32_t wcnt[kMaxWaves];           // survivors of each wave's own list
  uint32_t cand_n;                    // threshold candidates gathered so far
  float tval;
  int teq;
};

// ---- block-wide operations for NW waves ----------------------------------
// Consecutive operations alternate between two slot sets (parity p), so each
// needs one barrier: a slot set is rewritten two operations later, after all
// threads have passed the barrier in between.  The cross-wave step reads the
// NW slots in parallel lanes and reduces them with DPP, so its cost does not
// grow with the number of waves.
template <int NW>
__device__ __forceinline__ void block_minmax_count(SelScratch& sm, float& mn, float& mx,
                                                   uint32_t& cnt, int& p) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  cnt = wave_sum_u32(cnt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm.f0[p][wave] = mn;
    sm.f1[p][wave] = mx;
    sm.u[p][wave] = cnt;
  }
  __syncthreads();
  const bool in = lane < NW;
  mn = wave_min(in ? sm.f0[p][lane] : FLT_MAX);
  mx = wave_max(in ? sm.f1[p][lane] : -FLT_MAX);
  cnt = wave_sum_u32(in ? sm.u[p][lane] : 0u);
  p ^= 1;
}

// exclusive prefix over threads in thread order; also returns the total
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(SelScratch& sm, uint32_t v, uint32_t& total,
                                                    int& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) sm.u[p][wave] = incl;
  __syncthreads();
  const uint32_t x = lane < NW ? sm.u[p][lane] : 0u;
  const uint32_t y = wave_incl_scan_u32(x);
  const uint32_t off = __builtin_amdgcn_readlane(y, wave) - __builtin_amdgcn_readlane(x, wave);
  total = __builtin_amdgcn_readlane(y, NW - 1);
  p ^= 1;
  return incl - v + off;
}

template <int NW>
__device__ __forceinline__ void zero_hist(SelScratch& sm) {
  for (int b = threadIdx.x; b < kBins; b += NW * 64) sm.hist[b] = 0;
}

__device__ __forceinline__ int bin_of(float x, double dlo, double inv) {
  const double f = (static_cast<double>(x) - dlo) * inv;
  return f >= static_cast<double>(kBins - 1) ? kBins - 1 : static_cast<int>(f);
}

// ---- emitters --------------------------------------------------------------
// Global output rows idx [k] (and scores [k] or none).
struct GlobalOut {
  int32_t* __restrict__ oi;
  float* __restrict__ ov;
  __device__ __forceinline__ void put(int slot, int entry, float val) const {
    oi[slot] = entry;
    if (ov != nullptr) ov[slot] = val;
  }
  __device__ __forceinline__ void pad(int slot) const {
    oi[slot] = -1;
    if (ov != nullptr) ov[slot] = kNegInf;
  }
};

// ---- value runs ------------------------------------------------------------
// A run gives thread t the values at positions t*len() .. t*len()+len()-1
// (-inf for invalid ones, including positions past the end).  entry(pos)
// maps a position to its entry index.

// Threshold search over the valid values (> -inf) of the block's run: on
// return the top-k are every value > T plus the first take_eq values == T in
// position order (take_eq = 1 << 30: all of them).  On entry the histogram
// is zero and a barrier separates its zeroing (and any LDS writes of the run)
// from this call; on return it is zero again.  Run::kUnroll > 1 marks a run
// held in registers, whose loops must be unrolled completely.
template <int NW, typename Run>
__device__ __forceinline__ void threshold_search(SelScratch& sm, const Run& run, int k, int& p,
                                                 float& T, int& take_eq) {
  constexpr int THREADS = NW * 64;
  constexpr int BPT = kBins / THREADS;           // histogram bins per thread
  constexpr int UF = Run::kUnroll;
  const int tid = threadIdx.x;
  const int R = run.len();
  uint32_t n_valid = 0;
  float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll UF
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    if (x > kNegInf) {
      ++n_valid;
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
  }
  block_minmax_count<NW>(sm, mn, mx, n_valid, p);
  T = kNegInf;
  take_eq = 0;
  if (n_valid <= static_cast<uint32_t>(k)) return;
  float lo = mn, hi = mx;
  int need = k;
  for (int iter = 0;; ++iter) {
    if (lo == hi || iter >= 64) {     // all candidates equal (64 is never reached)
      T = lo;
      take_eq = need;
      return;
    }
    const double dlo = static_cast<double>(lo);
    const double inv = static_cast<double>(kBins) / (static_cast<double>(hi) - dlo);
#pragma unroll UF
    for (int i = 0; i < R; ++i) {
      const float x = run.get(i);
      if (x >= lo && x <= hi) atomicAdd(&sm.hist[bin_of(x, dlo, inv)], 1);
    }
    __syncthreads();
    // locate the bin b* holding the need-th largest candidate
    uint32_t h[BPT];
    uint32_t hs = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      h[j] = sm.hist[BPT * tid + j];
      hs += h[j];
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan<NW>(sm, hs, tot, p);
    uint32_t above = tot - pre - hs;                 // candidates in bins above this thread's
    const uint32_t un = static_cast<uint32_t>(need);
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (above < un && un <= above + h[j]) {
        sm.bstar = BPT * tid + j;
        sm.bstar_above = static_cast<int>(above);
        sm.bstar_cnt = static_cast<int>(h[j]);
      }
      above += h[j];
    }
    __syncthreads();
    const int bstar = sm.bstar;
    need -= sm.bstar_above;
    const int cnt = sm.bstar_cnt;
#pragma unroll
    for (int j = 0; j < BPT; ++j) sm.hist[BPT * tid + j] = 0;   // ready for the next pass
    float bmn = FLT_MAX, bmx = -FLT_MAX;
    uint32_t unused = 0;
#pragma unroll UF
    for (int i = 0; i < R; ++i) {
      const float x = run.get(i);
      if (x >= lo && x <= hi && bin_of(x, dlo, inv) == bstar) {
        bmn = fminf(bmn, x);
        bmx = fmaxf(bmx, x);
      }
    }
    block_minmax_count<NW>(sm, bmn, bmx, unused, p);
    if (cnt == need) {                // the whole bin is selected
      T = bmn;
      take_eq = 1 << 30;
      return;
    }
    lo = bmn;
    hi = bmx;
  }
}

// Selects the top-k of the block's run, whose positions are contiguous per
// thread (thread t holds positions t*len() ..), and emits each as
// out.put(slot, run.entry(position), value), slots 0.. in ascending position
// order.  Returns the number selected, min(k, #valid); does not pad.  Entry
// conditions as threshold_search.
template <int NW, typename Run, typename Out>
__device__ __forceinline__ int block_select(SelScratch& sm, const Run run, int k, int& p,
                                            const Out& out) {
  const int tid = threadIdx.x;
  const int R = run.len();
  float T;
  int take_eq;
  threshold_search<NW>(sm, run, k, p, T, take_eq);
  // ordered compaction: two scans, since a run can be a whole row (up to
  // 262144 values) and the counts do not fit 16-bit halves of one word
  uint32_t gt = 0, eq = 0;
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    gt += (x > T) ? 1u : 0u;
    eq += (x == T && x > kNegInf) ? 1u : 0u;
  }
  uint32_t gt_tot, eq_tot;
  const int gt_before = static_cast<int>(block_excl_scan<NW>(sm, gt, gt_tot, p));
  int eq_before = static_cast<int>(block_excl_scan<NW>(sm, eq, eq_tot, p));
  int slot = gt_before + min(eq_before, take_eq);
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    bool take = x > T;
    if (!take && x == T && x > kNegInf) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take) {
      if (slot < k) out.put(slot, run.entry(tid * R + i), x);   // always true; keeps writes in bounds
      ++slot;
    }
  }
  return min(k, static_cast<int>(gt_tot) + min(static_cast<int>(eq_tot), take_eq));
}

template <int NW, typename Out>
__device__ __forceinline__ void pad_output(const Out& out, int n, int k) {
  for (int s = n + threadIdx.x; s < k; s += NW * 64) out.pad(s);
}

// Global-memory run of a score row, linear, n values (-0.0 read as +0.0).
template <typename S>
struct GlobalRun {
  static constexpr int kUnroll = 1;
  const S* __restrict__ v;
  int n, r;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const {
    const int q = threadIdx.x * r + i;
    return q < n ? get_score(v + q) + 0.0f : kNegInf;
  }
  __device__ __forceinline__ int entry(int pos) const { return pos; }
};

// ---- top-k of an index-ordered survivor list in LDS --------------------------
__device__ __forceinline__ float lval(const lds_u32x2* lp, int j) { return __uint_as_float(lp[j].x); }

// Order-preserving keys of fp32 values (larger value, larger key; -0.0 must
// be normalised to +0.0 first).
__device__ __forceinline__ uint32_t f32_order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Histogram parameters of the first pass over [lo, hi] in select_sorted_list
// (a caller that holds the survivors in registers may build that pass's
// histogram itself): keys of lo and hi and the shift that takes their span
// down to kBins bins.
struct HistRange {
  uint32_t klo, khi;
  int shift;
};
__device__ __forceinline__ HistRange hist_range(float lo, float hi) {
  const uint32_t klo = f32_order_key(lo + 0.0f), khi = f32_order_key(hi + 0.0f);
  const uint32_t span = khi - klo;
  return {klo, khi, span < static_cast<uint32_t>(kBins) ? 0 : 21 - __builtin_clz(span)};
}
__device__ __forceinline__ void hist_add(SelScratch& sm, const HistRange& hr, float x) {
  const uint32_t key = f32_order_key(x);
  if (key >= hr.klo && key <= hr.khi) atomicAdd(&sm.hist[(key - hr.klo) >> hr.shift], 1);
}

// Survivor lists the selection reads, as (score bits, entry) pairs in LDS.
// each(f) calls f on the values of this thread's share, in any order;
// run(q0, q1) gives this thread's contiguous run of list positions, the runs
// in thread order being the list in ascending entry order; at(q) reads one.
template <int NT>
struct FlatList {                  // one list lp[0, n)
  const lds_u32x2* lp;
  int n;
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll 4
    for (int j = static_cast<int>(threadIdx.x); j < n; j += NT) f(lval(lp, j));
  }
  __device__ __forceinline__ void run(int& q0, int& q1) const {
    const int R = (n + NT - 1) / NT;
    q0 = static_cast<int>(threadIdx.x) * R;
    q1 = min(n, q0 + R);
  }
  __device__ __forceinline__ u32x2_t at(int q) const { return lp[q]; }
};
template <int CAP>
struct WaveLists {                 // wave w's list at lp[w CAP, w CAP + cnt_w), in wave order
  const lds_u32x2* lp;
  int cnt;                         // this wave's count (wave-uniform)
  int n;                           // all waves' (block-uniform)
  __device__ __forceinline__ int base() const { return static_cast<int>(threadIdx.x >> 6) * CAP; }
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
    const int b = base();
#pragma unroll 4
    for (int q = static_cast<int>(threadIdx.x & 63); q < cnt; q += 64) f(lval(lp, b + q));
  }
  __device__ __forceinline__ void run(int& q0, int& q1) const {
    const int R = (cnt + 63) / 64;
    q0 = base() + static_cast<int>(threadIdx.x & 63) * R;
    q1 = min(base() + cnt, q0 + R);
  }
  __device__ __forceinline__ u32x2_t at(int q) const { return lp[q]; }
};

// Top-k of the survivor list ls (n (score bits, entry) pairs in ascending
// entry order, values > -inf and -0.0 stored as +0.0, all within [lo, hi]
// when have_range, else the range is computed here).  Emits min(k, n)
// entries in ascending order and pads to k.
//   Threshold: radix selection on order-preserving keys, offset by the key
//   of lo: each pass histograms (key - klo) >> shift into 2048 LDS bins, the
//   shift taking the span of the keys still in play down to 11 bits, so at
//   most three passes resolve a 32-bit key.  One block scan locates the bin
//   of the need-th largest; a bin taken whole ends the search (its lower
//   edge is the threshold), a bin of at most kBrute entries is finished by
//   pairwise ranks (each candidate counts the larger and the equal ones), a
//   larger one becomes the next pass's range.
//   Output: the list is in index order, so one block scan of the pair
//   (count > T, count == T) over contiguous per-thread runs (two 16-bit
//   halves of one word: n < 65536) gives every output slot; entries equal to
//   T are taken lowest index first.
// Entry: the histogram is zero (or, with hist_ready, holds the first pass
// over [lo, hi] as hist_add builds it), sm.cand_n is zero and a barrier
// separates the list (and histogram) writes from this call.
template <int NW, typename List, typename Out>
__device__ __forceinline__ void select_sorted_list(SelScratch& sm, const List& ls, float lo,
                                                   float hi, bool have_range, int k, int& p,
                                                   const Out& out, bool hist_ready = false) {
  constexpr int NT = NW * 64;
  constexpr int BPT = kBins / NT;                 // histogram bins per thread
  const int tid = threadIdx.x;
  const int n = ls.n;
  float T = kNegInf;
  int take_eq = 1 << 30;                          // n <= k: everything is taken
  if (n > k) {
    if (!have_range) {
      float mn = FLT_MAX, mx = -FLT_MAX;
      uint32_t unused = 0;
      ls.each([&](float x) {
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      });
      block_minmax_count<NW>(sm, mn, mx, unused, p);
      lo = mn;
      hi = mx;
    }
    uint32_t klo = f32_order_key(lo + 0.0f), khi = f32_order_key(hi + 0.0f);
    int need = k;
    for (int pass = 0;; ++pass) {
      const uint32_t span = khi - klo;
      if (span == 0 || pass >= 4) {               // all candidates equal (4 is never reached)
        T = f32_from_order_key(klo);
        take_eq = need;
        break;
      }
      const int shift = span < static_cast<uint32_t>(kBins) ? 0 : 21 - __builtin_clz(span);
      if (!(hist_ready && have_range && pass == 0)) {
        ls.each([&](float x) {
          const uint32_t key = f32_order_key(x);
          if (key >= klo && key <= khi) atomicAdd(&sm.hist[(key - klo) >> shift], 1);
        });
      }
      __syncthreads();
      uint32_t h[BPT];
      uint32_t hs = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        h[j] = sm.hist[BPT * tid + j];
        hs += h[j];
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan<NW>(sm, hs, tot, p);
      uint32_t above = tot - pre - hs;            // candidates in higher bins
      const uint32_t un = static_cast<uint32_t>(need);
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (above < un && un <= above + h[j]) {
          sm.bstar = BPT * tid + j;
          sm.bstar_above = static_cast<int>(above);
          sm.bstar_cnt = static_cast<int>(h[j]);
        }
        above += h[j];
      }
#pragma unroll
      for (int j = 0; j < BPT; ++j) sm.hist[BPT * tid + j] = 0;
      __syncthreads();
      const uint32_t bstar = static_cast<uint32_t>(sm.bstar);
      need -= sm.bstar_above;
      const int cnt = sm.bstar_cnt;
      const uint32_t blo = klo + (bstar << shift);
      const uint32_t bhi = min(khi, blo + ((1u << shift) - 1u));
      if (cnt == need) {                          // the whole bin is taken
        T = f32_from_order_key(blo);
        take_eq = 1 << 30;
        break;
      }
      if (cnt <= kBrute) {
        // the need-th largest of the bin: the candidate with fewer than need
        // larger ones and at least need larger-or-equal ones
        ls.each([&](float x) {
          const uint32_t key = f32_order_key(x);
          if (key >= blo && key <= bhi) {
            const uint32_t slot = atomicAdd(&sm.cand_n, 1u);
            sm.tab[slot] = __float_as_uint(x);
          }
        });
        __syncthreads();
        for (int c = tid; c < cnt; c += NT) {
          const float v = __uint_as_float(sm.tab[c]);
          int g = 0, e = 0;
          for (int u = 0; u < cnt; ++u) {
            const float y = __uint_as_float(sm.tab[u]);
            g += y > v ? 1 : 0;
            e += y == v ? 1 : 0;
          }
          if (g < need && need <= g + e) {        // every such candidate writes the same
            sm.tval = v;
            sm.teq = need - g;
          }
        }
        __syncthreads();
        T = sm.tval;
        take_eq = sm.teq;
        break;
      }
      klo = blo;
      khi = bhi;
    }
  }
  // ordered compaction over contiguous runs of list positions per thread
  int j0, j1;
  ls.run(j0, j1);
  uint32_t gt = 0, eq = 0;
#pragma unroll 4
  for (int j = j0; j < j1; ++j) {
    const float x = __uint_as_float(ls.at(j).x);
    gt += x > T ? 1u : 0u;
    eq += x == T ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_excl_scan<NW>(sm, gt | (eq << 16), tot, p);
  int eq_before = static_cast<int>(pre >> 16);
  int slot = static_cast<int>(pre & 0xffffu) + min(eq_before, take_eq);
  for (int j = j0; j < j1; ++j) {
    const u32x2_t e = ls.at(j);
    const float x = __uint_as_float(e.x);
    bool take = x > T;
    if (!take && x == T) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take) {
      if (slot < k) out.put(slot, static_cast<int>(e.y), x);   // always true
      ++slot;
    }
  }
  const int n_sel =
      min(k, static_cast<int>(tot & 0xffffu) + min(static_cast<int>(tot >> 16), take_eq));
  pad_output<NW>(out, n_sel, k);
}

// ---- row bound from the chunk reports --------------------------------------
// A report other than +inf certifies c entries of its chunk at or above it
// (+inf: the chunk had fewer than c scored entries, or none).  With
// r = ceil(k / c), any value that at least r reports reach is therefore
// reached by at least k entries: a valid bound.  bound: the r-th largest
// report, approached from below by bisection over order-preserving keys,
// kBoundSteps steps (the
// minimum when there are exactly r reports; -inf when fewer).  Taking the
// r-th largest rather than the minimum keeps a few low chunks (for example
// freshly pooled entries with smaller norms) from loosening the whole row's
// bound.  top: the largest report top (at least every score of the row).
// c = 0: no reports were written; both are -inf.  The reports are loaded
// before c is looked at (they are in bounds either way).  n_chunks >= 1.
// Every wave computes the bound on its own (no barrier).
constexpr int kRepPerLane = kMaxBoundedN / kBoundChunk / 64;   // reports per lane
constexpr int kBoundSteps = 10;                                 // bisection steps

// The row's reports into registers, lane l holding reports l, l + 64, ...
// (index clamped to the last report, n_chunks >= 1; row_bound masks the
// slots past n_chunks): slots 0-3 always, 4-7 for rows of more than 256
// reports, 8-15 for more than 512, each group under one branch with no use
// inside, so that callers can issue them next to their other early loads.
constexpr int kRepA = 4, kRepB = 8;
__device__ __forceinline__ int report_slots(int n_chunks) {
  return n_chunks > 64 * kRepB ? kRepPerLane : n_chunks > 64 * kRepA ? kRepB : kRepA;
}
template <int U0, int U1>
__device__ __forceinline__ void load_report_slots(const float2* __restrict__ rep, int n_chunks,
                                                  float2 (&t)[kRepPerLane], bool in_use) {
  const int lane = threadIdx.x & 63;
  if (in_use) {
#pragma unroll
    for (int u = U0; u < U1; ++u) t[u] = rep[min(64 * u + lane, n_chunks - 1)];
  } else {
#pragma unroll
    for (int u = U0; u < U1; ++u) t[u] = make_float2(kPosInf, kNegInf);
  }
}
__device__ __forceinline__ void load_reports(const float2* __restrict__ rep, int n_chunks,
                                             float2 (&t)[kRepPerLane]) {
  const int ns = report_slots(n_chunks);
  load_report_slots<0, kRepA>(rep, n_chunks, t, true);
  load_report_slots<kRepA, kRepB>(rep, n_chunks, t, ns > kRepA);
  load_report_slots<kRepB, kRepPerLane>(rep, n_chunks, t, ns > kRepB);
}

// Order keys and extrema of the report slots [U0, U1) (key 0: none).
template <int U0, int U1>
__device__ __forceinline__ void report_keys(const float2 (&t)[kRepPerLane], int n_chunks,
                                            uint32_t (&key)[kRepPerLane], uint32_t& kmin,
                                            uint32_t& kmax, float& mx) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    const bool in = 64 * u + lane < n_chunks;
    key[u] = in && t[u].x != kPosInf ? f32_order_key(t[u].x) : 0u;
    if (key[u] != 0u) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
    }
    if (in) mx = fmaxf(mx, t[u].y);
  }
}

// Wave-wide reductions for the bound: DPP quad swaps, half-row and row
// mirrors leave every lane with its 16-lane row's result, and four readlanes
// combine the rows on the scalar unit (a short dependent chain, which the
// bisection below repeats every step).
template <int C>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), C, 0xF, 0xF, false));
}
template <typename F>
__device__ __forceinline__ uint32_t dpp_reduce_u32(uint32_t v, F f) {
  v = f(v, dpp_u32<0xB1>(v));                     // quad lanes [1, 0, 3, 2]
  v = f(v, dpp_u32<0x4E>(v));                     // quad lanes [2, 3, 0, 1]
  v = f(v, dpp_u32<0x141>(v));                    // row half mirror
  v = f(v, dpp_u32<0x140>(v));                    // row mirror
  return f(f(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
           f(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ uint32_t dpp_sum_u32(uint32_t v) {
  return dpp_reduce_u32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t dpp_min_u32(uint32_t v) {
  return dpp_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  return dpp_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ float dpp_max_f32(float v) {
  return __uint_as_float(dpp_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

// Keys of the wave's slots [0, U1) that are >= mid (0: none): this lane's
// count, summed in four independent chains.
template <int U1>
__device__ __forceinline__ uint32_t keys_at_least(const uint32_t (&key)[kRepPerLane], uint32_t mid) {
  uint32_t n[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U1; ++u) n[u & 3] += key[u] >= mid ? 1u : 0u;
  return (n[0] + n[1]) + (n[2] + n[3]);
}

// Bisection over [lo, hi) for the r-th largest of the keys in slots [0, U1)
// (invariant: at least r keys >= lo, fewer than r keys >= hi; keys of finite
// scores are below 0xff800000, so hi fits 32 bits).
template <int U1>
__device__ __forceinline__ uint32_t bisect_keys(const uint32_t (&key)[kRepPerLane], uint32_t lo,
                                                uint32_t hi, uint32_t r) {
#pragma unroll 1
  for (int it = 0; it < kBoundSteps && hi - lo > 1; ++it) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (dpp_sum_u32(keys_at_least<U1>(key, mid)) >= r) lo = mid;
    else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ float2 row_bound(const float2 (&t)[kRepPerLane], int n_chunks, int c,
                                            int k) {
  float mx = -FLT_MAX;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  uint32_t key[kRepPerLane];
  const int ns = report_slots(n_chunks);         // uniform: slots in use
  report_keys<0, kRepA>(t, n_chunks, key, kmin, kmax, mx);
  if (ns > kRepA) report_keys<kRepA, kRepB>(t, n_chunks, key, kmin, kmax, mx);
  if (ns > kRepB) report_keys<kRepB, kRepPerLane>(t, n_chunks, key, kmin, kmax, mx);
  if (c <= 0) return make_float2(kNegInf, kNegInf);
  mx = dpp_max_f32(mx);
  const uint32_t cnt = dpp_sum_u32(ns > kRepB   ? keys_at_least<kRepPerLane>(key, 1u)
                                   : ns > kRepA ? keys_at_least<kRepB>(key, 1u)
                                                : keys_at_least<kRepA>(key, 1u));
  const uint32_t r = static_cast<uint32_t>((k + c - 1) / c);
  if (cnt < r) return make_float2(kNegInf, mx);
  uint32_t lo = dpp_min_u32(kmin);
  if (cnt > r) {                                  // uniform; the slot count picked once
    const uint32_t hi = dpp_max_u32(kmax) + 1;
    lo = ns > kRepB   ? bisect_keys<kRepPerLane>(key, lo, hi, r)
         : ns > kRepA ? bisect_keys<kRepB>(key, lo, hi, r)
                      : bisect_keys<kRepA>(key, lo, hi, r);
  }
  return make_float2(f32_from_order_key(lo), mx);
}

__device__ __forceinline__ float2 wave_row_bound(const float2* __restrict__ rep, int n_chunks,
                                                 int c, int k) {
  float2 t[kRepPerLane];
  load_reports(rep, n_chunks, t);
  return row_bound(t, n_chunks, c, k);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t msk, uint32_t add) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(msk >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(msk), add));
}

// ---- survivor lists ------------------------------------------------------------
// four consecutive scores (16-byte aligned fp32 or 8-byte aligned bf16)
__device__ __forceinline__ float4 load4_scores(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load4_scores(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// One round of a wave's contiguous segment: lane l holds entries
// base + 64 s + l, s < SL (-inf at or past N_max); every load instruction
// reads 64 consecutive scores.
template <int SL, typename S>
__device__ __forceinline__ void load_round(const S* __restrict__ srow, int base, int N_max,
                                           float (&x)[SL]) {
  const int lane = threadIdx.x & 63;
  if (base + 64 * SL <= N_max) {
#pragma unroll
    for (int s = 0; s < SL; ++s) x[s] = get_score(srow + base + 64 * s + lane);
  } else {
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int q = base + 64 * s + lane;
      x[s] = q < N_max ? get_score(srow + q) : kNegInf;
    }
  }
}

// Streams the visible entries [0, V) of a score row into the LDS list lp in
// ascending index order, keeping those >= bnd: rounds of NW * 64 * SL
// entries, wave w owning the round's w-th contiguous segment with lane l
// taking every 64th entry from l.  x holds the first round (loaded by the
// caller with load_round at w * 64 * SL); the next round's loads are issued
// before the current round is compacted.  Per round: per-wave survivor
// counts (ballots) -> block scan -> every wave writes its survivors at its
// offset plus their rank among the wave's survivors (ballot + mbcnt).
// Returns the number of survivors (block-uniform); a value above cap means
// the list overflowed and is incomplete.  -0.0 is stored as +0.0.
template <int NW, int SL, typename S>
__device__ __forceinline__ int stream_survivors(SelScratch& sm, const S* __restrict__ srow, int V,
                                                int N_max, float bnd, lds_u32x2* lp, int cap,
                                                float (&x)[SL], int& p) {
  constexpr int kWaveSeg = 64 * SL;
  constexpr int kRoundLen = NW * kWaveSeg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n = 0;                                      // block-uniform
  for (int r0 = 0; r0 < V; r0 += kRoundLen) {
    float y[SL];
    const bool more = r0 + kRoundLen < V;
    if (more) load_round(srow, r0 + kRoundLen + wave * kWaveSeg, N_max, y);
    const int sb = r0 + wave * kWaveSeg;
    if (sb + kWaveSeg > V) {                     // entries at or past V are not visible
#pragma unroll
      for (int s = 0; s < SL; ++s)
        if (sb + 64 * s + lane >= V) x[s] = kNegInf;
    }
    uint32_t wt = 0;
#pragma unroll
    for (int s = 0; s < SL; ++s)
      wt += static_cast<uint32_t>(__builtin_popcountll(__builtin_amdgcn_ballot_w64(x[s] >= bnd)));
    if (lane == 0) sm.u[p][wave] = wt;
    __syncthreads();
    const uint32_t xs = lane < NW ? sm.u[p][lane] : 0u;
    const uint32_t ys = wave_incl_scan_u32(xs);
    uint32_t o = static_cast<uint32_t>(n) + __builtin_amdgcn_readlane(ys, wave) -
                 __builtin_amdgcn_readlane(xs, wave);
    n += static_cast<int>(__builtin_amdgcn_readlane(ys, NW - 1));
    p ^= 1;
    if (n > cap) break;                           // uniform: the caller falls back
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const bool take = x[s] >= bnd;
      const uint64_t msk = __builtin_amdgcn_ballot_w64(take);
      if (take)
        lp[lanes_below(msk, o)] =
            u32x2_t{__float_as_uint(x[s] + 0.0f), static_cast<uint32_t>(sb + 64 * s + lane)};
      o += static_cast<uint32_t>(__builtin_popcountll(msk));
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < SL; ++s) x[s] = y[s];
    }
  }
  return n;
}

// One round of a wave's segment (entries sb + 64 s + lane, as load_round
// lays them out) into the wave's own list lp[w CAP, ...), in ascending entry
// order, keeping those >= bnd: the wave's ballots give each survivor its rank
// among the wave's survivors, with no barrier and no exchange with the other
// waves, so each wave compacts as soon as its own scores have arrived.
// Every lane stores for every slot, a lane without a survivor (or with one
// past CAP, counted but not kept: the caller checks the counts) into its own
// spare entry lp[spare + tid], so the stores need no branch.  Returns the
// wave's count (wave-uniform).  -0.0 is stored as +0.0.
template <int CAP, int SL>
__device__ __forceinline__ int stream_wave_list(int sb, int V, float bnd, lds_u32x2* lp,
                                                int spare, float (&x)[SL]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (sb + 64 * SL > V) {                        // entries at or past V are not visible
#pragma unroll
    for (int s = 0; s < SL; ++s)
      if (sb + 64 * s + lane >= V) x[s] = kNegInf;
  }
  lds_u32x2* wl = lp + wave * CAP;
  // all ballots first, then their running counts on the scalar unit, so that
  // no slot's position waits for the previous slot's ballot
  uint64_t msk[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) msk[s] = __builtin_amdgcn_ballot_w64(x[s] >= bnd);
  uint32_t off[SL];
  uint32_t o = 0;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    off[s] = o;
    o += static_cast<uint32_t>(__builtin_popcountll(msk[s]));
  }
  lds_u32x2* own = lp + spare + threadIdx.x;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const uint32_t pos = lanes_below(msk[s], off[s]);
    lds_u32x2* dst = x[s] >= bnd && pos < static_cast<uint32_t>(CAP) ? wl + pos : own;
    *dst = u32x2_t{__float_as_uint(x[s] + 0.0f), static_cast<uint32_t>(sb + 64 * s + lane)};
  }
  return static_cast<int>(o);
}

}  // namespace sel
}  // namespace csa
