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
//   * Ordered compaction: one block-wide scan of (count > T, count == T)
//     gives every thread its output slots; entries equal to the threshold are
//     taken lowest index first.
// Only integer LDS atomics (counts) are used, so results are deterministic.
//
// Drivers.
//   * Bounded (topk_bounded_kernel), used with the chunk bounds the tuned
//     score kernels leave: per 256-key chunk of a row its c-th largest
//     score, whose minimum over the row is at most the row's k-th largest
//     (see bound_c_row).  Entries below it can never be selected, so one
//     workgroup per row keeps the few survivors in LDS and selects there.
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
  uint32_t tab[1024];                 // per-thread prefix of the index bitmap
  int bstar, bstar_above, bstar_cnt;
  uint32_t list_n;                    // survivors appended so far
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
// (-inf for invalid ones, including positions past the end).
struct LdsRun {                   // LDS, linear, n values
  static constexpr int kUnroll = 1;
  const lds_float* v;
  int n, r;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const {
    const int q = threadIdx.x * r + i;
    return q < n ? v[q] : kNegInf;
  }
};
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
  uint32_t tot;
  const uint32_t pre = block_excl_scan<NW>(gt | (eq << 16), tot, p);
  const int gt_before = static_cast<int>(pre & 0xffffu);
  int eq_before = static_cast<int>(pre >> 16);
  const int gt_total = static_cast<int>(tot & 0xffffu);
  const int eq_total = static_cast<int>(tot >> 16);
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

// ================================================================ bounds
// Per-row bound from the chunk values; -inf if unusable.
template <int NW>
__device__ __forceinline__ float row_bound(const float* __restrict__ thr, int n_chunks, int c, int k,
                                           int& p) {
  float mn = FLT_MAX, unused = -FLT_MAX;
  uint32_t cnt = 0;
  const int nc = c > 0 ? n_chunks : 0;           // no bound: the reports are not written
  for (int i = threadIdx.x; i < nc; i += NW * 64) {
    const float x = thr[i];
    if (x != kPosInf) {
      mn = fminf(mn, x);
      ++cnt;
    }
  }
  block_minmax_count<NW>(mn, unused, cnt, p);
  return static_cast<long long>(cnt) * c >= k ? mn : kNegInf;
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
struct GlobalRun {
  static constexpr int kUnroll = 1;
  const float* __restrict__ v;
  int n, r;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const {
    const int q = threadIdx.x * r + i;
    return q < n ? v[q] + 0.0f : kNegInf;
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
//   1. The row bound comes from the chunk reports (one block reduction).
//   2. The row is streamed in chunks of 32768 scores (eight coalesced 16-byte
//      loads per thread, the next chunk's loads in flight while the current
//      one is filtered); entries at or above the bound are appended to an LDS
//      list, one LDS atomic per wave reserving the wave's range.  The list is
//      unordered.
//   3. Radix selection on order-preserving 32-bit keys, offset by the
//      smallest survivor key: each pass histograms the next (up to) 11 bits
//      of the keys still in play (2048 LDS bins, two per thread), one block
//      scan locates the bin of the k-th largest, and the pass ends the search
//      when that bin is wholly taken or holds a single key.
//   4. The taken entries set their bit in an LDS bitmap over entry indices; a
//      block scan of its popcounts gives every taken entry its output slot,
//      which puts the result in ascending index order.  Among entries equal
//      to the threshold value only the lowest indices are taken.
// A row whose survivors overflow the list selects from the score row
// directly (block_select, slow but exact).
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRadixBits = 11;
static_assert((1 << kRadixBits) == kBins && kBins == 2 * kSelThreads, "two bins per thread");
constexpr int kMaxBoundedN = 262144;              // index bitmap: 8192 words of LDS
constexpr int kBitmapWords = kMaxBoundedN / 32;
constexpr int kStageVec = 8;                      // 16-byte loads per thread per chunk
constexpr int kStageChunk = kSelThreads * 4 * kStageVec;
constexpr int kListCap = 12 * kSelThreads;        // survivors held in LDS

typedef __attribute__((address_space(3))) uint32_t lds_uint;

// order-preserving key of a float that is not NaN and not -0.0
__device__ __forceinline__ uint32_t ord_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Survivors of one row: element (i, thread t) is survivor i * 1024 + t.
template <int NV>
struct RegSrc {                         // held in registers
  static constexpr int kUnroll = NV;
  float v[NV];
  int e[NV];
  __device__ __forceinline__ int len() const { return NV; }
  __device__ __forceinline__ float val(int i) const { return v[i]; }
  __device__ __forceinline__ int idx(int i) const { return e[i]; }
};
__device__ __forceinline__ void set_bit(lds_uint* bm, int e) {
  __hip_atomic_fetch_or(&bm[e >> 5], 1u << (e & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bitmap ranks: after the bits are set and a barrier, bitmap_prefix gives each
// thread the number of set bits before its words (WPT words per thread) in
// g_sm.tab; after one more barrier bitmap_rank(e) is the number of set bits
// below bit e.
__device__ __forceinline__ uint32_t bitmap_prefix(const lds_uint* bm, int W, int WPT, int& p) {
  uint32_t ps = 0;
  for (int j = 0; j < WPT; ++j) {
    const int w = threadIdx.x * WPT + j;
    if (w < W) ps += __popc(bm[w]);
  }
  uint32_t tot;
  g_sm.tab[threadIdx.x] = block_excl_scan<kSelWaves>(ps, tot, p);
  return tot;
}
__device__ __forceinline__ int bitmap_rank(const lds_uint* bm, int WPT, int e) {
  const int w = e >> 5, t = w / WPT;
  uint32_t r = g_sm.tab[t];
  for (int x = t * WPT; x < w; ++x) r += __popc(bm[x]);
  return static_cast<int>(r + __popc(bm[w] & ((1u << (e & 31)) - 1u)));
}

template <typename Src>
__device__ __forceinline__ void radix_select(const Src& src, int n, uint32_t kmin, uint32_t kmax,
                                             int k, int W, int WPT, lds_uint* bm, int& p,
                                             int32_t* __restrict__ oi, float* __restrict__ ov) {
  constexpr int NW = kSelWaves;
  constexpr int UF = Src::kUnroll;
  const int tid = threadIdx.x;
  const int R = src.len();
  // selection: key u = ord_key(x) - kmin; taken if u > Tu, or u == Tu and
  // index <= Emax
  int64_t Tu = -1;
  int take_eq = 0;
  if (n > k) {
    const uint32_t range = kmax - kmin;
    int hs = range == 0 ? 0 : 32 - __clz(range);  // keys still in play: (u >> hs) == prefix
    uint64_t prefix = 0;
    int need = k;
    if (hs == 0) {
      Tu = 0;
      take_eq = k;
    }
    while (hs > 0) {
      const int shift = max(hs - kRadixBits, 0);
      const uint32_t dmask = (1u << (hs - shift)) - 1u;
#pragma unroll UF
      for (int i = 0; i < R; ++i) {
        const float x = src.val(i);
        if (x > kNegInf) {
          const uint64_t u = ord_key(x) - kmin;
          if ((u >> hs) == prefix) atomicAdd(&g_sm.hist[(u >> shift) & dmask], 1);
        }
      }
      __syncthreads();
      const uint32_t h0 = g_sm.hist[2 * tid], h1 = g_sm.hist[2 * tid + 1];
      uint32_t tot;
      const uint32_t pre = block_excl_scan<NW>(h0 + h1, tot, p);
      uint32_t above = tot - pre - h0 - h1;
      const uint32_t un = static_cast<uint32_t>(need);
      if (above < un && un <= above + h1) {
        g_sm.bstar = 2 * tid + 1;
        g_sm.bstar_above = static_cast<int>(above);
        g_sm.bstar_cnt = static_cast<int>(h1);
      }
      above += h1;
      if (above < un && un <= above + h0) {
        g_sm.bstar = 2 * tid;
        g_sm.bstar_above = static_cast<int>(above);
        g_sm.bstar_cnt = static_cast<int>(h0);
      }
      g_sm.hist[2 * tid] = 0;
      g_sm.hist[2 * tid + 1] = 0;
      __syncthreads();
      need -= g_sm.bstar_above;
      const int cnt = g_sm.bstar_cnt;
      prefix = (prefix << (hs - shift)) | static_cast<uint64_t>(g_sm.bstar);
      hs = shift;
      if (cnt == need) {                          // the whole bin is taken
        Tu = static_cast<int64_t>(prefix << hs) - 1;
        take_eq = 0;
        break;
      }
      if (hs == 0) {                              // the bin is the single key Tu
        Tu = static_cast<int64_t>(prefix);
        take_eq = need;
      }
    }
  }
  int emax = INT_MAX;
  if (take_eq > 0) {
    // more entries equal the threshold than are taken: keep the take_eq
    // lowest indices, found from the ranks of the equal entries' bits
#pragma unroll UF
    for (int i = 0; i < R; ++i) {
      const float x = src.val(i);
      if (x > kNegInf && static_cast<int64_t>(ord_key(x) - kmin) == Tu) {
        const int e = src.idx(i);
        set_bit(bm, e);
      }
    }
    __syncthreads();
    bitmap_prefix(bm, W, WPT, p);
    __syncthreads();
#pragma unroll UF
    for (int i = 0; i < R; ++i) {
      const float x = src.val(i);
      if (x > kNegInf && static_cast<int64_t>(ord_key(x) - kmin) == Tu) {
        const int e = src.idx(i);
        if (bitmap_rank(bm, WPT, e) == take_eq - 1) g_sm.bstar = e;
      }
    }
    __syncthreads();
    emax = g_sm.bstar;
    for (int j = 0; j < WPT; ++j) {
      const int w = tid * WPT + j;
      if (w < W) bm[w] = 0;
    }
    __syncthreads();
  }
  // bitmap of the taken indices -> output slots
#pragma unroll UF
  for (int i = 0; i < R; ++i) {
    const float x = src.val(i);
    if (x > kNegInf) {
      const int64_t u = static_cast<int64_t>(ord_key(x) - kmin);
      const int e = src.idx(i);
      if (u > Tu || (u == Tu && e <= emax)) set_bit(bm, e);
    }
  }
  __syncthreads();
  const int n_sel = static_cast<int>(bitmap_prefix(bm, W, WPT, p));
  __syncthreads();
#pragma unroll UF
  for (int i = 0; i < R; ++i) {
    const float x = src.val(i);
    if (x > kNegInf) {
      const int64_t u = static_cast<int64_t>(ord_key(x) - kmin);
      const int e = src.idx(i);
      if (u > Tu || (u == Tu && e <= emax)) {
        const int slot = bitmap_rank(bm, WPT, e);
        if (slot < k) {                           // always true; keeps writes in bounds
          oi[slot] = e;
          if (ov != nullptr) ov[slot] = x;
        }
      }
    }
  }
  for (int sl = n_sel + tid; sl < k; sl += kSelThreads) {
    oi[sl] = -1;
    if (ov != nullptr) ov[sl] = kNegInf;
  }
}

template <int NV>
__device__ __forceinline__ void select_list(const lds_float* lv, const lds_int* li, int n,
                                            uint32_t kmin, uint32_t kmax, int k, int W, int WPT,
                                            lds_uint* bm, int& p, int32_t* __restrict__ oi,
                                            float* __restrict__ ov) {
  RegSrc<NV> src;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int q = i * kSelThreads + threadIdx.x;
    src.v[i] = q < n ? lv[q] : kNegInf;
    src.e[i] = q < n ? li[q] : 0;
  }
  radix_select(src, n, kmin, kmax, k, W, WPT, bm, p, oi, ov);
}

__device__ __forceinline__ void load_stage(const float* __restrict__ srow, int c0, int V,
                                           float4 (&x)[kStageVec]) {
#pragma unroll
  for (int i = 0; i < kStageVec; ++i) {
    const int q = c0 + 4 * (i * kSelThreads + static_cast<int>(threadIdx.x));
    if (q + 3 < V) {
      x[i] = *reinterpret_cast<const float4*>(srow + q);
    } else {
      x[i].x = q < V ? srow[q] : kNegInf;
      x[i].y = q + 1 < V ? srow[q + 1] : kNegInf;
      x[i].z = q + 2 < V ? srow[q + 2] : kNegInf;
      x[i].w = q + 3 < V ? srow[q + 3] : kNegInf;
    }
  }
}

// Few long rows (more than kStreamMaxN entries, at most kRegionMaxRows rows:
// too little parallelism for one workgroup per row) are filtered first by
// topk_filter_kernel: one 256-thread workgroup per 4096 entries, each wave
// owning 1024 of them (a region) and working alone (no barrier, no atomic):
// it derives the row bound from the chunk reports, compacts its entries at or
// above the bound to the front of its region of the survivor buffers and
// stores their number.  The bounded kernel then gathers the regions instead
// of streaming the row.
constexpr int kStreamMaxN = 65536;
constexpr int kRegionMaxRows = 64;
constexpr int kFiltSeg = 4096;
constexpr int kRegion = 1024;

__global__ __launch_bounds__(kSegThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float* __restrict__ chunk_thr, int n_chunks, int nreg, float* __restrict__ reg_val,
    int32_t* __restrict__ reg_idx, int32_t* __restrict__ reg_cnt) {
  const int seg = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int e0 = seg * kFiltSeg + wave * kRegion;
  const int L = max(0, min(V - e0, kRegion));
  const int r = seg * (kFiltSeg / kRegion) + wave;
  if (r >= nreg) return;
  const float* src = scores + row * s_rs + e0;
  float v[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 256 * i + 4 * lane;
    if (q + 3 < L) {
      const float4 x = *reinterpret_cast<const float4*>(src + q);
      v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = (q + e < L) ? src[q + e] : kNegInf;
    }
  }
  const int c = bound_c_row(V, k);
  float bound = kNegInf;
  if (c > 0) {
    const float* thr = chunk_thr + static_cast<int64_t>(row) * n_chunks;
    float mn = FLT_MAX;
    uint32_t cnt = 0;
    for (int i = lane; i < n_chunks; i += 64) {
      const float t = thr[i];
      if (t != kPosInf) {
        mn = fminf(mn, t);
        ++cnt;
      }
    }
    mn = wave_min(mn);
    cnt = wave_sum_u32(cnt);
    if (static_cast<long long>(cnt) * c >= k) bound = mn;
  }
  uint32_t cl = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) cl += (v[i][e] > kNegInf && v[i][e] >= bound) ? 1u : 0u;
  const uint32_t incl = wave_incl_scan_u32(cl);
  const int64_t base = (static_cast<int64_t>(row) * nreg + r) * kRegion;
  uint32_t o = incl - cl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[i][e] > kNegInf && v[i][e] >= bound) {
        reg_val[base + o] = v[i][e] + 0.0f;       // -0.0 -> +0.0
        reg_idx[base + o] = e0 + 256 * i + 4 * lane + e;
        ++o;
      }
    }
  }
  if (lane == 63) reg_cnt[static_cast<int64_t>(row) * nreg + r] = static_cast<int32_t>(incl);
}

int filter_regions(int N_max) { return (N_max + kFiltSeg - 1) / kFiltSeg * (kFiltSeg / kRegion); }

// REGIONS: the survivors come from topk_filter_kernel's regions (wave w
// takes regions w, w + 16, ...; the counts and the first 128 survivors of
// eight regions are loaded together); otherwise the row is streamed.
template <bool REGIONS>
__global__ __launch_bounds__(kSelThreads) void topk_bounded_kernel(
    const float* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float* __restrict__ chunk_thr, int n_chunks, int nreg,
    const float* __restrict__ reg_val, const int32_t* __restrict__ reg_idx,
    const int32_t* __restrict__ reg_cnt, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  constexpr int NW = kSelWaves;
  __shared__ uint32_t bm_s[kBitmapWords];
  __shared__ float lv_s[kListCap];
  __shared__ int li_s[kListCap];
  lds_uint* bm = (lds_uint*)bm_s;
  lds_float* lv = (lds_float*)lv_s;
  lds_int* li = (lds_int*)li_s;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const float* srow = scores + row * s_rs;
  float4 x[kStageVec];
  if (!REGIONS) load_stage(srow, 0, V, x);
  const int W = (N_max + 31) >> 5;
  const int WPT = (W + kSelThreads - 1) / kSelThreads;
  g_sm.hist[2 * tid] = 0;
  g_sm.hist[2 * tid + 1] = 0;
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    if (w < W) bm[w] = 0;
  }
  if (tid == 0) g_sm.list_n = 0;
  float smin = FLT_MAX, smax = -FLT_MAX;
  int p = 0;
  if (REGIONS) {
    __syncthreads();                                // LDS state zeroed
    const int wave = tid >> 6;
    const int32_t* cnt_row = reg_cnt + static_cast<int64_t>(row) * nreg;
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
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(&g_sm.list_n, static_cast<uint32_t>(c));
          base = __builtin_amdgcn_readfirstlane(base);
          if (lane < c) {
            smin = fminf(smin, v0[rr]);
            smax = fmaxf(smax, v0[rr]);
            if (base + lane < kListCap) {
              lv[base + lane] = v0[rr];
              li[base + lane] = i0[rr];
            }
          }
          if (64 + lane < c) {
            smin = fminf(smin, v1[rr]);
            smax = fmaxf(smax, v1[rr]);
            if (base + 64 + lane < kListCap) {
              lv[base + 64 + lane] = v1[rr];
              li[base + 64 + lane] = i1[rr];
            }
          }
          const int64_t rb = (static_cast<int64_t>(row) * nreg + r) * kRegion;
          for (int j = 128 + lane; j < c; j += 64) {   // rare: more than 128 survivors
            const float x1 = reg_val[rb + j];
            smin = fminf(smin, x1);
            smax = fmaxf(smax, x1);
            if (base + j < kListCap) {
              lv[base + j] = x1;
              li[base + j] = reg_idx[rb + j];
            }
          }
        }
      }
    }
  } else {
  // 1. row bound
  const int c = bound_c_row(V, k);
  float bmn = FLT_MAX, unused_f = -FLT_MAX;
  uint32_t bcnt = 0;
  if (c > 0) {
    const float* thr = chunk_thr + static_cast<int64_t>(row) * n_chunks;
    for (int i = tid; i < n_chunks; i += kSelThreads) {
      const float t = thr[i];
      if (t != kPosInf) {
        bmn = fminf(bmn, t);
        ++bcnt;
      }
    }
  }
  block_minmax_count<NW>(bmn, unused_f, bcnt, p);   // barrier: LDS state zeroed
  const float bound = (c > 0 && static_cast<long long>(bcnt) * c >= k) ? bmn : kNegInf;
  // 2. stream the row, appending survivors
  for (int c0 = 0; c0 < V; c0 += kStageChunk) {
    float4 y[kStageVec];
    const bool more = c0 + kStageChunk < V;
    if (more) load_stage(srow, c0 + kStageChunk, V, y);
    uint32_t cl = 0;
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const float e4[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) cl += (e4[e] > kNegInf && e4[e] >= bound) ? 1u : 0u;
    }
    const uint32_t incl = wave_incl_scan_u32(cl);
    const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
    if (tot > 0) {                                  // uniform in the wave
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&g_sm.list_n, tot);
      base = __builtin_amdgcn_readfirstlane(base);
      uint32_t o = base + incl - cl;
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) {
        const float e4[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = e4[e];
          if (v > kNegInf && v >= bound) {
            smin = fminf(smin, v);
            smax = fmaxf(smax, v);
            if (o < static_cast<uint32_t>(kListCap)) {
              lv[o] = v + 0.0f;                     // -0.0 -> +0.0
              li[o] = c0 + 4 * (i * kSelThreads + tid) + e;
            }
            ++o;
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) x[i] = y[i];
    }
  }
  }
  uint32_t unused_u = 0;
  block_minmax_count<NW>(smin, smax, unused_u, p);  // barrier: the list is complete
  const int n = static_cast<int>(g_sm.list_n);
  int32_t* oi = out_idx + static_cast<int64_t>(row) * k;
  float* ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  const uint32_t kmin = ord_key(smin + 0.0f), kmax = ord_key(smax + 0.0f);
  if (n <= 4 * kSelThreads) {
    select_list<4>(lv, li, n, kmin, kmax, k, W, WPT, bm, p, oi, ov);
  } else if (n <= 8 * kSelThreads) {
    select_list<8>(lv, li, n, kmin, kmax, k, W, WPT, bm, p, oi, ov);
  } else if (n <= kListCap) {
    select_list<12>(lv, li, n, kmin, kmax, k, W, WPT, bm, p, oi, ov);
  } else {
    Emitter em;
    em.oi = oi;
    em.ov = ov;
    em.base = 0;
    em.use_lmap = false;
    em.lmap = nullptr;
    em.gmap = nullptr;
    const int n_sel =
        block_select<NW>(GlobalRun{srow, V, (V + kSelThreads - 1) / kSelThreads}, k, p, em);
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

hipError_t launch_topk(const float* scores, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       const float* chunk_thr, int n_chunks, int32_t* idx, float* out_scores,
                       void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (chunk_thr != nullptr && topk_bounded_ok(N_max)) {
    if (!use_regions(rows, N_max)) {
      hipLaunchKernelGGL(topk_bounded_kernel<false>, dim3(rows), dim3(kSelThreads), 0, s, scores,
                         s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_thr, n_chunks, 0, nullptr,
                         nullptr, nullptr, idx, out_scores);
      return hipGetLastError();
    }
    const int nreg = filter_regions(N_max);
    const size_t slots = static_cast<size_t>(rows) * nreg * kRegion;
    float* rv = static_cast<float*>(ws);
    int32_t* ri = reinterpret_cast<int32_t*>(rv + slots);
    int32_t* rc = ri + slots;
    hipLaunchKernelGGL(topk_filter_kernel, dim3((N_max + kFiltSeg - 1) / kFiltSeg, rows),
                       dim3(kSegThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                       chunk_thr, n_chunks, nreg, rv, ri, rc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_bounded_kernel<true>, dim3(rows), dim3(kSelThreads), 0, s, scores,
                       s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_thr, n_chunks, nreg, rv, ri,
                       rc, idx, out_scores);
    return hipGetLastError();
  }
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
