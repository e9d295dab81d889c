// Top-k selection of compressed entries per query token ("DeepSeek V4 技术解读",
// §2.1: the Lightning Indexer keeps the top-k compressed blocks).
//
// Exact rule: the min(k, V) visible entries with the largest fp32 scores,
// ties to the lower index, -0.0 equal to +0.0, returned in ascending index
// order and padded with -1.
//
// Selection core (block_select): the values are split into contiguous runs,
// one per thread, so thread order is index order.
//   * Threshold search: an LDS histogram of 2048 equal-width bins over
//     [lo, hi] (the bin is a monotone function of the score) finds the bin
//     of the k-th largest; [lo, hi] shrinks to that bin's min / max until the
//     bin is taken whole or all candidates are equal.  Each pass shrinks the
//     range 2048-fold, so fp32 needs at most ~26 passes.
//   * Ordered compaction: block-wide scans of (count > T) and (count == T)
//     give every thread its output slots; entries equal to the threshold are
//     taken lowest index first.
// Only integer LDS atomics (counts) are used, so results are deterministic.
//
// Drivers.
//   * Bounded (topk_bounded_kernel), used with the chunk reports the tuned
//     score kernels leave: per 256-key chunk of a row its c-th largest and
//     its largest score.  The ceil(k / c)-th largest of these reports is at
//     most the row's k-th largest (see row_bound), so entries below it can
//     never be selected: one workgroup per row keeps the few survivors in LDS, in
//     index order, and selects there (select_sorted_list: the same histogram
//     search over [bound, largest report], finished by pairwise ranks inside
//     a small bin).
//   * Unbounded (topk_seg_kernel): one workgroup per row segment of up to
//     32768 scores.  Rows longer than one segment take two passes: each
//     segment keeps its own top-k (a superset of its share of the row's
//     top-k) and one workgroup selects from the concatenation, which is in
//     index order.
#include <float.h>
#include <limits.h>

#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr int kBins = 2048;
constexpr int kMaxWaves = 16;
constexpr float kPosInf = __builtin_inff();

// row-segment kernel
constexpr int kSegThreads = 256;
constexpr int kSegCap = 32768;                    // values per workgroup (128 per thread)
constexpr int kMaxK = 2048;

typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) int lds_int;

// Reduction slots and histogram: one file-scope LDS object per workgroup,
// accessed directly (never through a generic pointer).
struct Scratch {
  int hist[kBins];
  float f0[2][kMaxWaves];
  float f1[2][kMaxWaves];
  uint32_t u[2][kMaxWaves];
  uint32_t tab[1024];                 // region offsets, then threshold candidates
  int bstar, bstar_above, bstar_cnt;
  uint32_t cand_n;                    // threshold candidates gathered so far
  float tval;
  int teq;
};
__shared__ Scratch g_sm;

// ---- block-wide operations for NW waves ----------------------------------
// Consecutive operations alternate between two slot sets (parity p), so each
// needs one barrier: a slot set is rewritten two operations later, after all
// threads have passed the barrier in between.  The cross-wave step reads the
// NW slots in parallel lanes and reduces them with DPP, so its cost does not
// grow with the number of waves.
template <int NW>
__device__ __forceinline__ void block_minmax_count(float& mn, float& mx, uint32_t& cnt, int& p) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  cnt = wave_sum_u32(cnt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    g_sm.f0[p][wave] = mn;
    g_sm.f1[p][wave] = mx;
    g_sm.u[p][wave] = cnt;
  }
  __syncthreads();
  const bool in = lane < NW;
  mn = wave_min(in ? g_sm.f0[p][lane] : FLT_MAX);
  mx = wave_max(in ? g_sm.f1[p][lane] : -FLT_MAX);
  cnt = wave_sum_u32(in ? g_sm.u[p][lane] : 0u);
  p ^= 1;
}

// exclusive prefix over threads in thread order; also returns the total
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, int& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) g_sm.u[p][wave] = incl;
  __syncthreads();
  const uint32_t x = lane < NW ? g_sm.u[p][lane] : 0u;
  const uint32_t y = wave_incl_scan_u32(x);
  const uint32_t off = __builtin_amdgcn_readlane(y, wave) - __builtin_amdgcn_readlane(x, wave);
  total = __builtin_amdgcn_readlane(y, NW - 1);
  p ^= 1;
  return incl - v + off;
}

template <int THREADS>
__device__ __forceinline__ void zero_hist() {
  for (int b = threadIdx.x; b < kBins; b += THREADS) g_sm.hist[b] = 0;
}

// ---- value runs ------------------------------------------------------------
// A run gives thread t the values at positions t*len() .. t*len()+len()-1
// (-inf for invalid ones, including positions past the end); see SplitRun
// and GlobalRun below.
// Writes one selected entry: index = gmap[pos] if given, else
// base + lmap[pos] if use_lmap, else base + pos.  Passed by value.  (An LDS pointer can
// legitimately be address 0, so its presence is a flag, not a null test.)
struct Emitter {
  int32_t* __restrict__ oi;
  float* __restrict__ ov;
  int base;
  bool use_lmap;
  const lds_int* lmap;
  const int32_t* __restrict__ gmap;
  __device__ __forceinline__ void operator()(int pos, float val, int slot) const {
    int e;
    if (gmap != nullptr) e = gmap[pos];
    else if (use_lmap) e = base + lmap[pos];
    else e = base + pos;
    oi[slot] = e;
    if (ov != nullptr) ov[slot] = val;
  }
};

__device__ __forceinline__ int bin_of(float x, double dlo, double inv) {
  const double f = (static_cast<double>(x) - dlo) * inv;
  return f >= static_cast<double>(kBins - 1) ? kBins - 1 : static_cast<int>(f);
}

// Threshold search over the valid values (> -inf) of the block's run: on
// return the top-k are every value > T plus the first take_eq values == T in
// position order (take_eq = 1 << 30: all of them).  On entry the histogram
// is zero and a barrier separates its zeroing (and any LDS writes of the run)
// from this call; on return it is zero again.  Run::kUnroll > 1 marks a run
// held in registers, whose loops must be unrolled completely.
template <int NW, typename Run>
__device__ __forceinline__ void threshold_search(const Run& run, int k, int& p, float& T,
                                                 int& take_eq) {
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
  block_minmax_count<NW>(mn, mx, n_valid, p);
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
      if (x >= lo && x <= hi) atomicAdd(&g_sm.hist[bin_of(x, dlo, inv)], 1);
    }
    __syncthreads();
    // locate the bin b* holding the need-th largest candidate
    uint32_t h[BPT];
    uint32_t hs = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      h[j] = g_sm.hist[BPT * tid + j];
      hs += h[j];
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan<NW>(hs, tot, p);
    uint32_t above = tot - pre - hs;                 // candidates in bins above this thread's
    const uint32_t un = static_cast<uint32_t>(need);
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (above < un && un <= above + h[j]) {
        g_sm.bstar = BPT * tid + j;
        g_sm.bstar_above = static_cast<int>(above);
        g_sm.bstar_cnt = static_cast<int>(h[j]);
      }
      above += h[j];
    }
    __syncthreads();
    const int bstar = g_sm.bstar;
    need -= g_sm.bstar_above;
    const int cnt = g_sm.bstar_cnt;
#pragma unroll
    for (int j = 0; j < BPT; ++j) g_sm.hist[BPT * tid + j] = 0;   // ready for the next pass
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
    block_minmax_count<NW>(bmn, bmx, unused, p);
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
// thread (thread t holds positions t*len() ..), and calls emit(position,
// value, slot) for each, slots 0.. in ascending position order.  Returns the
// number selected, min(k, #valid).  Entry conditions as threshold_search.
template <int NW, typename Run>
__device__ __forceinline__ int block_select(const Run run, int k, int& p, const Emitter emit) {
  const int tid = threadIdx.x;
  const int R = run.len();
  float T;
  int take_eq;
  threshold_search<NW>(run, k, p, T, take_eq);
  // ordered compaction
  uint32_t gt = 0, eq = 0;
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    gt += (x > T) ? 1u : 0u;
    eq += (x == T && x > kNegInf) ? 1u : 0u;
  }
  // two scans: a run can be a whole row (up to 262144 values), so the counts
  // do not fit 16-bit halves of one word
  uint32_t gt_tot, eq_tot;
  const int gt_before = static_cast<int>(block_excl_scan<NW>(gt, gt_tot, p));
  int eq_before = static_cast<int>(block_excl_scan<NW>(eq, eq_tot, p));
  const int gt_total = static_cast<int>(gt_tot);
  const int eq_total = static_cast<int>(eq_tot);
  int slot = gt_before + min(eq_before, take_eq);
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    bool take = x > T;
    if (!take && x == T && x > kNegInf) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take) {
      if (slot < k) emit(tid * R + i, x, slot);   // always true; keeps writes in bounds
      ++slot;
    }
  }
  return min(k, gt_total + min(eq_total, take_eq));
}

template <int THREADS>
__device__ __forceinline__ void pad_output(const Emitter& em, int n, int k) {
  for (int s = n + threadIdx.x; s < k; s += THREADS) {
    em.oi[s] = -1;
    if (em.ov != nullptr) em.ov[s] = kNegInf;
  }
}

// LDS run of R values per thread in the transposed layout v[i*THREADS + t].
template <int THREADS>
struct SplitRun {
  static constexpr int kUnroll = 1;
  const lds_float* v;
  int r;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const { return v[i * THREADS + threadIdx.x]; }
};

// Global-memory run, linear, n values (-0.0 read as +0.0).
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
};

// One 256-thread workgroup per (segment, row); a segment holds up to 32768
// values, 128 per thread.  Every load of the segment is issued at once
// (coalesced 16-byte chunks, chunk g to thread g % 256) and staged in LDS with
// the chunk slot XOR-swizzled, so both the writes and the per-thread run reads
// are bank-conflict free; thread t then holds positions 128t .. 128t+127 and
// stores them transposed (conflict-free) for block_select.
// MERGE: the input is the per-segment candidates of a previous pass (values
// and entry indices, -inf padded) instead of a score row.
template <bool MERGE>
__global__ __launch_bounds__(kSegThreads) void topk_seg_kernel(
    const float* __restrict__ src, int64_t src_rs, const int32_t* __restrict__ src_idx,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq, int N_max,
    int m, int k, int nseg, int32_t* __restrict__ out_idx, float* __restrict__ out_val,
    float* __restrict__ cand_val, int32_t* __restrict__ cand_idx) {
  constexpr int NW = kSegThreads / 64;
  constexpr int R = kSegCap / kSegThreads;        // 128 values per thread
  constexpr int CH = R / 4;                       // 32 chunks of 16 bytes per thread
  __shared__ float buf[kSegCap];
  const int tid = threadIdx.x;
  const int seg = MERGE ? 0 : blockIdx.x, row = MERGE ? blockIdx.x : blockIdx.y;
  int L;                                          // valid values in this segment
  const float* sp;
  if (MERGE) {
    L = nseg * k;
    sp = src + static_cast<int64_t>(row) * L;
  } else {
    const int b = row / Tq;
    const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
    L = max(0, min(V - seg * kSegCap, kSegCap));
    sp = src + row * src_rs + static_cast<int64_t>(seg) * kSegCap;
  }
  lds_float* lb = (lds_float*)buf;
  {
    float4 x[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = 4 * (i * kSegThreads + tid);
      if (q + 3 < L) {
        x[i] = *reinterpret_cast<const float4*>(sp + q);
      } else {
        x[i].x = q < L ? sp[q] : kNegInf;
        x[i].y = q + 1 < L ? sp[q + 1] : kNegInf;
        x[i].z = q + 2 < L ? sp[q + 2] : kNegInf;
        x[i].w = q + 3 < L ? sp[q + 3] : kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = i * kSegThreads + tid;
      const int t = g / CH, c = g % CH;           // owner thread and chunk within its run
      lds_float* d = lb + 4 * (t * CH + (c ^ (t & (CH - 1))));
      d[0] = x[i].x + 0.0f;                       // -0.0 -> +0.0
      d[1] = x[i].y + 0.0f;
      d[2] = x[i].z + 0.0f;
      d[3] = x[i].w + 0.0f;
    }
  }
  int p = 0;
  zero_hist<kSegThreads>();
  __syncthreads();
  float v[R];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const lds_float* s4 = lb + 4 * (tid * CH + (c ^ (tid & (CH - 1))));
    v[4 * c] = s4[0];
    v[4 * c + 1] = s4[1];
    v[4 * c + 2] = s4[2];
    v[4 * c + 3] = s4[3];
  }
  __syncthreads();                                // every run has left LDS
#pragma unroll
  for (int i = 0; i < R; ++i) lb[i * kSegThreads + tid] = v[i];
  __syncthreads();
  Emitter em;
  if (MERGE || nseg == 1) {
    em.oi = out_idx + static_cast<int64_t>(row) * k;
    em.ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  } else {
    const int64_t base = (static_cast<int64_t>(row) * nseg + seg) * k;
    em.oi = cand_idx + base;
    em.ov = cand_val + base;
  }
  em.base = MERGE ? 0 : seg * kSegCap;            // MERGE: positions first, mapped below
  em.use_lmap = false;
  em.lmap = nullptr;
  em.gmap = nullptr;
  const int n_sel = block_select<NW>(SplitRun<kSegThreads>{lb, R}, k, p, em);
  if (MERGE) {
    // positions in the candidate list -> entry indices, all loads in flight
    __syncthreads();
    const int32_t* gi = src_idx + static_cast<int64_t>(row) * L;
    constexpr int kMaxPer = kMaxK / kSegThreads;
    int pos[kMaxPer];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int sl = tid + j * kSegThreads;
      pos[j] = sl < n_sel ? em.oi[sl] : 0;
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) pos[j] = gi[pos[j]];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int sl = tid + j * kSegThreads;
      if (sl < n_sel) em.oi[sl] = pos[j];
    }
  }
  pad_output<kSegThreads>(em, n_sel, k);
}

// ============================================================ bounded path
// topk_bounded_kernel: one 1024-thread workgroup per row.
//   1. The row bound and the top of the survivors' range come from the chunk
//      reports, every wave computing them on its own (row_bound), the
//      reports loaded next to the first score loads.
//   2. Survivor list in LDS, in ascending index order, as (score bits, entry
//      index) pairs.  Streamed rows: rounds of 16384 scores, each lane
//      loading 16 scalar scores (entries 64 s + lane of its wave's segment),
//      the next round's loads in flight while the current one is compacted;
//      per round the waves count their survivors with ballots, one block scan
//      gives every wave its offset, and each survivor's slot is that offset
//      plus its rank among the wave's survivors (ballot + mbcnt).  Filtered
//      rows (topk_filter_kernel first): the per-region survivor counts are
//      scanned and the regions copied at their offsets.
//   3. select_sorted_list: a 2048-bin equal-width histogram over [bound, top]
//      locates the bin of the k-th largest; a bin of at most 256 entries is
//      finished by pairwise ranks, a larger one narrows the range to the bin
//      and repeats.  Because the list is in index order, one block scan of
//      the pair (count > T, count == T) over contiguous per-thread runs (two
//      16-bit halves of one word: the list holds fewer than 65536 entries)
//      gives every selected entry its output slot: ascending indices, and
//      among entries equal to the threshold the lowest indices.
// A row whose survivors overflow the list selects from the score row
// directly (block_select, slow but exact).
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
static_assert(kBins % kSelThreads == 0, "whole bins per thread");
constexpr int kMaxBoundedN = 262144;
constexpr int kListCap = 16 * kSelThreads;        // survivors held in LDS
static_assert(kListCap < 65536, "select_sorted_list packs two list counts into one word");
constexpr int kBrute = 256;                       // bin size finished by pairwise ranks
constexpr int kStreamSlots = 16;                  // 4-byte loads per lane per round
constexpr int kWaveSeg = 64 * kStreamSlots;       // entries per wave per round
constexpr int kRoundLen = kSelWaves * kWaveSeg;   // entries per round

// survivor list: (score bits, entry index) pairs in ascending index order
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;

__device__ __forceinline__ float lval(const lds_u32x2* lp, int j) { return __uint_as_float(lp[j].x); }

// Top-k of the survivor list lp[0..n) (values > -inf, -0.0 and +0.0 equal,
// all within [lo, hi] when have_range, else the range is computed here).
// Writes min(k, n) entry indices in ascending order to oi (their scores to
// ov), pads with -1 / -inf.
//   Threshold: one 2048-bin histogram over [lo, hi] (the bin is a monotone
//   function of the score) locates the bin of the k-th largest; a bin of at
//   most kBrute entries is finished by pairwise ranks (each candidate counts
//   the larger and the equal ones), a larger one narrows [lo, hi] to the bin
//   and repeats.
//   Output: the list is in index order, so one block scan of (count > T,
//   count == T) over contiguous per-thread runs gives every output slot;
//   entries equal to T are taken lowest index first.
// Entry: the histogram is zero, g_sm.cand_n is zero and a barrier separates
// the list writes from this call.
template <int NT>
__device__ __forceinline__ void select_sorted_list(const lds_u32x2* lp, int n, float lo, float hi,
                                                   bool have_range, int k, int& p,
                                                   int32_t* __restrict__ oi,
                                                   float* __restrict__ ov) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kBins / NT;                 // histogram bins per thread
  const int tid = threadIdx.x;
  float T = kNegInf;
  int take_eq = 1 << 30;                          // n <= k: everything is taken
  if (n > k) {
    if (!have_range) {
      float mn = FLT_MAX, mx = -FLT_MAX;
      uint32_t unused = 0;
      for (int j = tid; j < n; j += NT) {
        const float x = lval(lp, j);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      block_minmax_count<NW>(mn, mx, unused, p);
      lo = mn;
      hi = mx;
    }
    lo += 0.0f;                                   // -0.0 -> +0.0
    hi += 0.0f;
    int need = k;
    for (int iter = 0;; ++iter) {
      if (lo == hi || iter >= 64) {               // all candidates equal (64 is never reached)
        T = lo;
        take_eq = need;
        break;
      }
      const double dlo = static_cast<double>(lo);
      const double inv = static_cast<double>(kBins) / (static_cast<double>(hi) - dlo);
      for (int j = tid; j < n; j += NT) {
        const float x = lval(lp, j);
        if (x >= lo && x <= hi) atomicAdd(&g_sm.hist[bin_of(x, dlo, inv)], 1);
      }
      __syncthreads();
      uint32_t h[BPT];
      uint32_t hs = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        h[j] = g_sm.hist[BPT * tid + j];
        hs += h[j];
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan<NW>(hs, tot, p);
      uint32_t above = tot - pre - hs;            // candidates in higher bins
      const uint32_t un = static_cast<uint32_t>(need);
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (above < un && un <= above + h[j]) {
          g_sm.bstar = BPT * tid + j;
          g_sm.bstar_above = static_cast<int>(above);
          g_sm.bstar_cnt = static_cast<int>(h[j]);
        }
        above += h[j];
      }
#pragma unroll
      for (int j = 0; j < BPT; ++j) g_sm.hist[BPT * tid + j] = 0;
      __syncthreads();
      const int bstar = g_sm.bstar;
      need -= g_sm.bstar_above;
      const int cnt = g_sm.bstar_cnt;
      if (cnt <= kBrute) {
        // the need-th largest of the bin: the candidate with fewer than need
        // larger ones and at least need larger-or-equal ones
        for (int j = tid; j < n; j += NT) {
          const float x = lval(lp, j);
          if (x >= lo && x <= hi && bin_of(x, dlo, inv) == bstar) {
            const uint32_t slot = atomicAdd(&g_sm.cand_n, 1u);
            g_sm.tab[slot] = __float_as_uint(x);
          }
        }
        __syncthreads();
        if (tid < cnt) {
          const float v = __uint_as_float(g_sm.tab[tid]);
          int g = 0, e = 0;
          for (int u = 0; u < cnt; ++u) {
            const float y = __uint_as_float(g_sm.tab[u]);
            g += y > v ? 1 : 0;
            e += y == v ? 1 : 0;
          }
          if (g < need && need <= g + e) {        // every such candidate writes the same
            g_sm.tval = v + 0.0f;
            g_sm.teq = need - g;
          }
        }
        __syncthreads();
        T = g_sm.tval;
        take_eq = g_sm.teq;
        break;
      }
      float bmn = FLT_MAX, bmx = -FLT_MAX;
      uint32_t unused = 0;
      for (int j = tid; j < n; j += NT) {
        const float x = lval(lp, j);
        if (x >= lo && x <= hi && bin_of(x, dlo, inv) == bstar) {
          bmn = fminf(bmn, x);
          bmx = fmaxf(bmx, x);
        }
      }
      block_minmax_count<NW>(bmn, bmx, unused, p);
      lo = bmn + 0.0f;
      hi = bmx + 0.0f;
    }
  }
  // ordered compaction over contiguous runs of R list positions per thread
  const int R = (n + NT - 1) / NT;
  const int j0 = tid * R, j1 = min(n, j0 + R);
  uint32_t gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const float x = lval(lp, j);
    gt += x > T ? 1u : 0u;
    eq += x == T ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_excl_scan<NW>(gt | (eq << 16), tot, p);
  int eq_before = static_cast<int>(pre >> 16);
  int slot = static_cast<int>(pre & 0xffffu) + min(eq_before, take_eq);
  for (int j = j0; j < j1; ++j) {
    const u32x2_t e = lp[j];
    const float x = __uint_as_float(e.x);
    bool take = x > T;
    if (!take && x == T) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take) {
      if (slot < k) {                             // always true; keeps writes in bounds
        oi[slot] = static_cast<int32_t>(e.y);
        if (ov != nullptr) ov[slot] = x + 0.0f;
      }
      ++slot;
    }
  }
  const int n_sel =
      min(k, static_cast<int>(tot & 0xffffu) + min(static_cast<int>(tot >> 16), take_eq));
  for (int sl = n_sel + tid; sl < k; sl += NT) {
    oi[sl] = -1;
    if (ov != nullptr) ov[sl] = kNegInf;
  }
}

// One round of a wave's contiguous segment: lane l holds entries
// base + 64 s + l, s < kStreamSlots (-inf at or past N_max).
template <typename S>
__device__ __forceinline__ void load_round(const S* __restrict__ srow, int base, int N_max,
                                           float (&x)[kStreamSlots]) {
  const int lane = threadIdx.x & 63;
  if (base + kWaveSeg <= N_max) {
#pragma unroll
    for (int s = 0; s < kStreamSlots; ++s) x[s] = get_score(srow + base + 64 * s + lane);
  } else {
#pragma unroll
    for (int s = 0; s < kStreamSlots; ++s) {
      const int q = base + 64 * s + lane;
      x[s] = q < N_max ? get_score(srow + q) : kNegInf;
    }
  }
}

// Row bound and range top from the chunk reports, computed by every wave on
// its own.  A report other than +inf certifies c entries of its chunk at or
// above it (+inf: the chunk had fewer than c scored entries, or none).  With
// r = ceil(k / c), any value that at least r reports reach is therefore
// reached by at least k entries: a valid bound.  bound: the r-th largest
// report, found from below by bisection over order-preserving keys (the
// minimum when there are exactly r reports; -inf when fewer).  Taking the
// r-th largest rather than the minimum keeps a few low chunks (for example
// freshly pooled entries with smaller norms) from loosening the whole row's
// bound.  top: the largest report top (at least every score of the row).
// c = 0: no reports were written; both are -inf.  The reports are loaded
// before c is looked at (they are in bounds either way).  n_chunks >= 1.
constexpr int kRepPerLane = kMaxBoundedN / kBoundChunk / 64;   // reports per lane
constexpr int kBoundSteps = 10;                                 // bisection steps

__device__ __forceinline__ uint32_t f32_order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

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

// Order keys, count and extrema of the report slots [U0, U1) (key 0: none).
template <int U0, int U1>
__device__ __forceinline__ void report_keys(const float2 (&t)[kRepPerLane], int n_chunks,
                                            uint32_t (&key)[kRepPerLane], uint32_t& kmin,
                                            uint32_t& kmax, uint32_t& cnt, float& mx) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    const bool in = 64 * u + lane < n_chunks;
    key[u] = in && t[u].x != kPosInf ? f32_order_key(t[u].x) : 0u;
    if (key[u] != 0u) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
      ++cnt;
    }
    if (in) mx = fmaxf(mx, t[u].y);
  }
}

template <int U1>
__device__ __forceinline__ uint32_t keys_at_least(const uint32_t (&key)[kRepPerLane], uint32_t mid) {
  uint32_t n = 0;
#pragma unroll
  for (int u = 0; u < U1; ++u) n += key[u] >= mid ? 1u : 0u;
  return n;
}

__device__ __forceinline__ float2 row_bound(const float2 (&t)[kRepPerLane], int n_chunks, int c,
                                            int k) {
  float mx = -FLT_MAX;
  uint32_t kmin = 0xffffffffu, kmax = 0u, cnt = 0;
  uint32_t key[kRepPerLane];
  const int ns = report_slots(n_chunks);         // uniform: slots in use
  report_keys<0, kRepA>(t, n_chunks, key, kmin, kmax, cnt, mx);
  if (ns > kRepA) report_keys<kRepA, kRepB>(t, n_chunks, key, kmin, kmax, cnt, mx);
  if (ns > kRepB) report_keys<kRepB, kRepPerLane>(t, n_chunks, key, kmin, kmax, cnt, mx);
  if (c <= 0) return make_float2(kNegInf, kNegInf);
  mx = wave_max(mx);
  cnt = wave_sum_u32(cnt);
  const uint32_t r = static_cast<uint32_t>((k + c - 1) / c);
  if (cnt < r) return make_float2(kNegInf, mx);
  // invariant: at least r keys >= lo, fewer than r keys >= hi
  uint32_t lo = wave_min_u32(kmin);
  if (cnt > r) {
    uint64_t hi = static_cast<uint64_t>(wave_max_u32(kmax)) + 1;
    for (int it = 0; it < kBoundSteps && hi - lo > 1; ++it) {
      const uint32_t mid = static_cast<uint32_t>(lo + ((hi - lo) >> 1));
      const uint32_t n = ns > kRepB   ? keys_at_least<kRepPerLane>(key, mid)
                         : ns > kRepA ? keys_at_least<kRepB>(key, mid)
                                      : keys_at_least<kRepA>(key, mid);
      if (wave_sum_u32(n) >= r) lo = mid;
      else hi = mid;
    }
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

// Few long rows (more than kStreamMaxN entries, at most kRegionMaxRows rows:
// too little parallelism for one workgroup per row) are filtered first by
// topk_filter_kernel: one 256-thread workgroup per 4096 entries, each wave
// owning 1024 of them (a region) and working alone (no barrier, no atomic):
// it derives the row bound from the chunk reports, compacts its entries at or
// above the bound, in index order, to the front of its region of the
// survivor buffers and stores their number.  The bounded kernel then gathers
// the regions instead of streaming the row.
constexpr int kStreamMaxN = 65536;
constexpr int kRegionMaxRows = 64;
constexpr int kFiltSeg = 4096;
constexpr int kRegion = 1024;
static_assert(kMaxBoundedN / kRegion <= kSelThreads, "one region per thread in the offset scan");

// four consecutive scores (16-byte aligned fp32 or 8-byte aligned bf16)
__device__ __forceinline__ float4 load4_scores(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load4_scores(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

template <typename S>
__global__ __launch_bounds__(kSegThreads) void topk_filter_kernel(
    const S* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float2* __restrict__ chunk_rep, int n_chunks, int nreg, float* __restrict__ reg_val,
    int32_t* __restrict__ reg_idx, int32_t* __restrict__ reg_cnt) {
  const int seg = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = seg * kFiltSeg + wave * kRegion;
  const int r = seg * (kFiltSeg / kRegion) + wave;
  if (r >= nreg) return;
  // loads bounded by N_max, issued before the visible count is known
  const int Ln = max(0, min(N_max - e0, kRegion));
  const S* src = scores + row * s_rs + e0;
  float v[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 256 * i + 4 * lane;
    if (q + 3 < Ln) {
      const float4 x = load4_scores(src + q);
      v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = (q + e < Ln) ? get_score(src + q + e) : kNegInf;
    }
  }
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int L = max(0, min(V - e0, kRegion));
  if (L < kRegion) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (256 * i + 4 * lane + e >= L) v[i][e] = kNegInf;
  }
  const float bound = wave_row_bound(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks,
                                     bound_c_row(V, k), k).x;
  const float bnd = bound > kNegInf ? bound : -FLT_MAX;   // x >= bnd: a finite survivor
  const int64_t base = (static_cast<int64_t>(row) * nreg + r) * kRegion;
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t cl = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) cl += v[i][e] >= bnd ? 1u : 0u;
    const uint32_t incl = wave_incl_scan_u32(cl);
    uint32_t q = o + incl - cl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[i][e] >= bnd) {
        reg_val[base + q] = v[i][e];
        reg_idx[base + q] = e0 + 256 * i + 4 * lane + e;
        ++q;
      }
    }
    o += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) reg_cnt[static_cast<int64_t>(row) * nreg + r] = static_cast<int32_t>(o);
}

int filter_regions(int N_max) { return (N_max + kFiltSeg - 1) / kFiltSeg * (kFiltSeg / kRegion); }

// One 1024-thread workgroup per row builds the row's survivor list in LDS in
// ascending index order and selects from it (select_sorted_list).
// Streaming (REGIONS false): rounds of kRoundLen entries, wave w owning the
// round's w-th contiguous segment with lane l taking every 64th entry from l;
// the score loads are issued before the row's visible count and bound are
// known (bounded by N_max, masked after), and the next round's loads before
// the current round is compacted.  Each round: per-wave survivor counts
// (ballots) -> block scan -> every wave writes its survivors at its offset
// plus their rank among the wave's survivors, i.e. in index order.
// REGIONS: the per-region counts of topk_filter_kernel are scanned in region
// order and wave w copies regions w, w + 16, ... (the counts and first 128
// survivors of eight regions are loaded together).
// The bound (when the row has one) and the largest chunk report delimit the
// survivors' range.  More than kListCap survivors (inputs far from the
// expected distribution): the row is selected from global memory by
// block_select instead.
template <bool REGIONS, typename S>
__global__ __launch_bounds__(kSelThreads) void topk_bounded_kernel(
    const S* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float2* __restrict__ chunk_rep, int n_chunks, int nreg,
    const float* __restrict__ reg_val, const int32_t* __restrict__ reg_idx,
    const int32_t* __restrict__ reg_cnt, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  constexpr int NW = kSelWaves;
  __shared__ u32x2_t lp_s[kListCap];
  lds_u32x2* lp = (lds_u32x2*)lp_s;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const S* srow = scores + row * s_rs;
  float x[kStreamSlots];
  float2 rt[kRepPerLane];
  if (!REGIONS) {
    load_round(srow, wave * kWaveSeg, N_max, x);
    load_reports(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks, rt);
  }
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  float2 rb = make_float2(kNegInf, kNegInf);
  if (!REGIONS) rb = row_bound(rt, n_chunks, bound_c_row(V, k), k);
  g_sm.hist[2 * tid] = 0;
  g_sm.hist[2 * tid + 1] = 0;
  if (tid == 0) g_sm.cand_n = 0;
  int p = 0;
  int n = 0;                                      // block-uniform
  if (REGIONS) {
    const int32_t* cnt_row = reg_cnt + static_cast<int64_t>(row) * nreg;
    uint32_t total;
    const uint32_t off = block_excl_scan<NW>(tid < nreg ? static_cast<uint32_t>(cnt_row[tid]) : 0u,
                                             total, p);
    if (tid < nreg) g_sm.tab[tid] = off;
    n = static_cast<int>(total);
    __syncthreads();                              // offsets visible
    if (n <= kListCap) {
      constexpr int kBatch = 8;
      for (int r0 = wave; r0 < nreg; r0 += kSelWaves * kBatch) {
        int cnt[kBatch];
        float v0[kBatch], v1[kBatch];
        int i0[kBatch], i1[kBatch];
#pragma unroll
        for (int rr = 0; rr < kBatch; ++rr) {
          const int r = r0 + kSelWaves * rr;
          if (r < nreg) {
            const int64_t base = (static_cast<int64_t>(row) * nreg + r) * kRegion;
            cnt[rr] = cnt_row[r];
            v0[rr] = reg_val[base + lane];
            v1[rr] = reg_val[base + 64 + lane];
            i0[rr] = reg_idx[base + lane];
            i1[rr] = reg_idx[base + 64 + lane];
          }
        }
#pragma unroll
        for (int rr = 0; rr < kBatch; ++rr) {
          const int r = r0 + kSelWaves * rr;
          if (r < nreg && cnt[rr] > 0) {
            const int c = cnt[rr];
            const int o = static_cast<int>(g_sm.tab[r]);
            if (lane < c) lp[o + lane] = u32x2_t{__float_as_uint(v0[rr]), static_cast<uint32_t>(i0[rr])};
            if (64 + lane < c)
              lp[o + 64 + lane] = u32x2_t{__float_as_uint(v1[rr]), static_cast<uint32_t>(i1[rr])};
            const int64_t rg = (static_cast<int64_t>(row) * nreg + r) * kRegion;
            for (int j = 128 + lane; j < c; j += 64)   // rare: more than 128 survivors
              lp[o + j] = u32x2_t{__float_as_uint(reg_val[rg + j]), static_cast<uint32_t>(reg_idx[rg + j])};
          }
        }
      }
    }
    rb = wave_row_bound(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks, bound_c_row(V, k), k);
  } else {
    const float bnd = rb.x > kNegInf ? rb.x : -FLT_MAX;     // x >= bnd: a finite survivor
    for (int r0 = 0; r0 < V; r0 += kRoundLen) {
      float y[kStreamSlots];
      const bool more = r0 + kRoundLen < V;
      if (more) load_round(srow, r0 + kRoundLen + wave * kWaveSeg, N_max, y);
      const int sb = r0 + wave * kWaveSeg;
      if (sb + kWaveSeg > V) {                     // entries at or past V are not visible
#pragma unroll
        for (int s = 0; s < kStreamSlots; ++s)
          if (sb + 64 * s + lane >= V) x[s] = kNegInf;
      }
      uint32_t wt = 0;
#pragma unroll
      for (int s = 0; s < kStreamSlots; ++s)
        wt += static_cast<uint32_t>(__builtin_popcountll(__builtin_amdgcn_ballot_w64(x[s] >= bnd)));
      if (lane == 0) g_sm.u[p][wave] = wt;
      __syncthreads();
      const uint32_t xs = lane < NW ? g_sm.u[p][lane] : 0u;
      const uint32_t ys = wave_incl_scan_u32(xs);
      uint32_t o = static_cast<uint32_t>(n) + __builtin_amdgcn_readlane(ys, wave) -
                   __builtin_amdgcn_readlane(xs, wave);
      n += static_cast<int>(__builtin_amdgcn_readlane(ys, NW - 1));
      p ^= 1;
      if (n > kListCap) break;                    // uniform: fall back below
#pragma unroll
      for (int s = 0; s < kStreamSlots; ++s) {
        const bool take = x[s] >= bnd;
        const uint64_t msk = __builtin_amdgcn_ballot_w64(take);
        if (take)
          lp[lanes_below(msk, o)] = u32x2_t{__float_as_uint(x[s]), static_cast<uint32_t>(sb + 64 * s + lane)};
        o += static_cast<uint32_t>(__builtin_popcountll(msk));
      }
      if (more) {
#pragma unroll
        for (int s = 0; s < kStreamSlots; ++s) x[s] = y[s];
      }
    }
  }
  __syncthreads();                                // the list is complete
  int32_t* oi = out_idx + static_cast<int64_t>(row) * k;
  float* ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  if (n <= kListCap) {
    const bool have_range = rb.x > kNegInf;       // survivors lie in [bound, largest report]
    select_sorted_list<kSelThreads>(lp, n, rb.x, rb.y, have_range, k, p, oi, ov);
  } else {
    Emitter em;
    em.oi = oi;
    em.ov = ov;
    em.base = 0;
    em.use_lmap = false;
    em.lmap = nullptr;
    em.gmap = nullptr;
    const int n_sel =
        block_select<NW>(GlobalRun<S>{srow, V, (V + kSelThreads - 1) / kSelThreads}, k, p, em);
    pad_output<kSelThreads>(em, n_sel, k);
  }
}

int num_segments(int N_max) { return (N_max + kSegCap - 1) / kSegCap; }

}  // namespace

bool topk_supported(int N_max, int k) {
  if (k < 1 || k > kMaxK || N_max < 1) return false;
  const int nseg = num_segments(N_max);
  return nseg == 1 || static_cast<long long>(nseg) * k <= kSegCap;
}

size_t topk_workspace_bytes(int rows, int N_max, int k) {
  const int nseg = num_segments(N_max);
  if (nseg == 1) return 0;
  return static_cast<size_t>(rows) * nseg * k * (sizeof(float) + sizeof(int32_t));
}

bool topk_bounded_ok(int N_max) { return N_max <= kMaxBoundedN; }

bool use_regions(int rows, int N_max) { return N_max > kStreamMaxN && rows <= kRegionMaxRows; }

size_t topk_bounded_workspace_bytes(int rows, int N_max) {
  if (!topk_bounded_ok(N_max) || !use_regions(rows, N_max)) return 0;
  const size_t regs = static_cast<size_t>(rows) * filter_regions(N_max);
  return regs * kRegion * (sizeof(float) + sizeof(int32_t)) + regs * sizeof(int32_t);
}

template <typename S>
hipError_t launch_topk_bounded(const S* scores, int64_t s_rs, const int32_t* q_pos,
                               const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                               const float2* chunk_rep, int n_chunks, int32_t* idx,
                               float* out_scores, void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (!use_regions(rows, N_max)) {
    hipLaunchKernelGGL((topk_bounded_kernel<false, S>), dim3(rows), dim3(kSelThreads), 0, s, scores,
                       s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_rep, n_chunks, 0, nullptr,
                       nullptr, nullptr, idx, out_scores);
    return hipGetLastError();
  }
  const int nreg = filter_regions(N_max);
  const size_t slots = static_cast<size_t>(rows) * nreg * kRegion;
  float* rv = static_cast<float*>(ws);
  int32_t* ri = reinterpret_cast<int32_t*>(rv + slots);
  int32_t* rc = ri + slots;
  hipLaunchKernelGGL(topk_filter_kernel<S>, dim3((N_max + kFiltSeg - 1) / kFiltSeg, rows),
                     dim3(kSegThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                     chunk_rep, n_chunks, nreg, rv, ri, rc);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_bounded_kernel<true, S>), dim3(rows), dim3(kSelThreads), 0, s, scores,
                     s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_rep, n_chunks, nreg, rv, ri,
                     rc, idx, out_scores);
  return hipGetLastError();
}

hipError_t launch_topk(const void* scores_v, bool score16, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       const float2* chunk_rep, int n_chunks, int32_t* idx, float* out_scores,
                       void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (score16)   // bf16 rows: the bounded path only (the caller checks chunk_rep and N_max)
    return launch_topk_bounded(static_cast<const uint16_t*>(scores_v), s_rs, q_pos, n_entries, B,
                               Tq, N_max, m, k, chunk_rep, n_chunks, idx, out_scores, ws, s);
  const float* scores = static_cast<const float*>(scores_v);
  if (chunk_rep != nullptr && topk_bounded_ok(N_max))
    return launch_topk_bounded(scores, s_rs, q_pos, n_entries, B, Tq, N_max, m, k, chunk_rep,
                               n_chunks, idx, out_scores, ws, s);
  const int nseg = num_segments(N_max);
  float* cv = static_cast<float*>(ws);
  int32_t* ci = reinterpret_cast<int32_t*>(cv + static_cast<size_t>(rows) * nseg * k);
  hipLaunchKernelGGL(topk_seg_kernel<false>, dim3(nseg, rows), dim3(kSegThreads), 0, s, scores,
                     s_rs, nullptr, q_pos, n_entries, Tq, N_max, m, k, nseg, idx, out_scores, cv,
                     ci);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nseg == 1) return e;
  hipLaunchKernelGGL(topk_seg_kernel<true>, dim3(rows), dim3(kSegThreads), 0, s, cv, 0, ci, q_pos,
                     n_entries, Tq, N_max, m, k, nseg, idx, out_scores, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace csa
