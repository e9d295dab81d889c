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
//   * Bounded (topk_filter_kernel + topk_select_kernel), used with the chunk
//     bounds the tuned score kernels leave: per 256-key chunk of a row its
//     c-th largest score, whose minimum over the row is at most the row's
//     k-th largest (see bound_c_row).  Entries below it can never be selected.
//     The filter spreads the row over many workgroups (4096 entries each) and
//     compacts the survivors of each slice in index order; the select kernel
//     gathers a row's survivors into LDS and selects from them.
//   * Unbounded (topk_seg_kernel): one workgroup per row segment of up to
//     32768 scores.  Rows longer than one segment take two passes: each
//     segment keeps its own top-k (a superset of its share of the row's
//     top-k) and one workgroup selects from the concatenation, which is in
//     index order.
#include <float.h>

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
  int bstar, bstar_above, bstar_cnt;
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

// Selects the top-k of the valid values (> -inf) of the block's run and calls
// emit(position, value, slot) for each, slots 0.. in ascending position
// order.  Returns the number selected, min(k, #valid).  On entry the
// histogram is zero and a barrier separates its zeroing (and any LDS writes
// of the run) from this call.
template <int NW, typename Run>
__device__ __forceinline__ int block_select(const Run run, int k, int& p, const Emitter emit) {
  constexpr int THREADS = NW * 64;
  constexpr int BPT = kBins / THREADS;           // histogram bins per thread
  const int tid = threadIdx.x;
  const int R = run.len();
  uint32_t n_valid = 0;
  float mn = FLT_MAX, mx = -FLT_MAX;
  for (int i = 0; i < R; ++i) {
    const float x = run.get(i);
    if (x > kNegInf) {
      ++n_valid;
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
  }
  block_minmax_count<NW>(mn, mx, n_valid, p);

  float T = kNegInf;          // selection: all v > T, plus the first take_eq with v == T
  int take_eq = 0;
  if (n_valid > static_cast<uint32_t>(k)) {
    float lo = mn, hi = mx;
    int need = k;
    for (int iter = 0;; ++iter) {
      if (lo == hi || iter >= 64) {     // all candidates equal (64 is never reached)
        T = lo;
        take_eq = need;
        break;
      }
      const double dlo = static_cast<double>(lo);
      const double inv = static_cast<double>(kBins) / (static_cast<double>(hi) - dlo);
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
        break;
      }
      lo = bmn;
      hi = bmx;
    }
  }

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
  const lds_float* v;
  int r;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const { return v[i * THREADS + threadIdx.x]; }
};

// Global-memory run, linear, n values (-0.0 read as +0.0).
struct GlobalRun {
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
constexpr int kFiltSeg = 4096;                    // entries per filter workgroup (16 per thread)
constexpr int kMaxSlices = kSegThreads;           // slices per row: N_max <= 1M
constexpr int kSelCap = 16384;                    // survivors a select workgroup holds in LDS

// One workgroup per (slice of 4096 entries, row).  The slice's scores (four
// coalesced 16-byte loads per thread) and the row's chunk bounds are all in
// flight together; the entries at or above the row bound (all valid entries
// when the row has no bound) are written, in index order, to the front of the
// slice's region of the survivor buffers, and their number to slice_cnt.
__global__ __launch_bounds__(kSegThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float* __restrict__ chunk_thr, int n_chunks, int nslice,
    float* __restrict__ slice_val, int32_t* __restrict__ slice_idx,
    int32_t* __restrict__ slice_cnt) {
  constexpr int NW = kSegThreads / 64;
  const int seg = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int seg0 = seg * kFiltSeg;
  const int L = max(0, min(V - seg0, kFiltSeg));
  const float* srow = scores + row * s_rs + seg0;
  float v[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = kSegThreads * 4 * i + 4 * tid;
    if (q + 3 < L) {
      const float4 x = *reinterpret_cast<const float4*>(srow + q);
      v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = (q + e < L) ? srow[q + e] : kNegInf;
    }
  }
  int p = 0;
  const float bound = row_bound<NW>(chunk_thr + static_cast<int64_t>(row) * n_chunks, n_chunks,
                                    bound_c_row(V, k), k, p);
  // positions: 1024 i + 4 tid + e, so (i, wave, lane, e) order is index order
  uint32_t c[4], incl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c[i] += (v[i][e] > kNegInf && v[i][e] >= bound) ? 1u : 0u;
    incl[i] = wave_incl_scan_u32(c[i]);
    if (lane == 63) g_sm.u[p][NW * i + wave] = incl[i];
  }
  __syncthreads();
  const uint32_t x = lane < 4 * NW ? g_sm.u[p][lane] : 0u;
  const uint32_t y = wave_incl_scan_u32(x);
  const int64_t slice = (static_cast<int64_t>(row) * nslice + seg) * kFiltSeg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t o = __builtin_amdgcn_readlane(y, NW * i + wave) -
                 __builtin_amdgcn_readlane(x, NW * i + wave) + incl[i] - c[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[i][e] > kNegInf && v[i][e] >= bound) {
        slice_val[slice + o] = v[i][e] + 0.0f;   // -0.0 -> +0.0
        slice_idx[slice + o] = seg0 + kSegThreads * 4 * i + 4 * tid + e;
        ++o;
      }
    }
  }
  if (tid == 0) {
    slice_cnt[static_cast<int64_t>(row) * nslice + seg] =
        static_cast<int32_t>(__builtin_amdgcn_readlane(y, 4 * NW - 1));
  }
}

// One workgroup per row: slice counts -> block scan -> every survivor loaded
// (consecutive survivors to consecutive threads, slice found by binary search
// over the LDS prefix) and stored at its rank in LDS -> block_select.  Rows
// with more survivors than LDS holds select from the score row directly.
__global__ __launch_bounds__(kSegThreads) void topk_select_kernel(
    const float* __restrict__ slice_val, const int32_t* __restrict__ slice_idx,
    const int32_t* __restrict__ slice_cnt, int nslice, const float* __restrict__ scores,
    int64_t s_rs, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries,
    int Tq, int N_max, int m, int k, int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  constexpr int NW = kSegThreads / 64;
  constexpr int U = 8;                            // survivor loads in flight per thread
  __shared__ float cv[kSelCap];
  __shared__ int cp[kSelCap];
  __shared__ int offs[kMaxSlices];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint32_t my_cnt =
      tid < nslice ? static_cast<uint32_t>(slice_cnt[static_cast<int64_t>(row) * nslice + tid]) : 0u;
  zero_hist<kSegThreads>();
  int p = 0;
  uint32_t n_u;
  const uint32_t pre = block_excl_scan<NW>(my_cnt, n_u, p);
  if (tid < nslice) offs[tid] = static_cast<int>(pre);
  __syncthreads();
  const int n = static_cast<int>(n_u);
  Emitter em;
  em.oi = out_idx + static_cast<int64_t>(row) * k;
  em.ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  em.base = 0;
  em.use_lmap = false;
  em.lmap = nullptr;
  em.gmap = nullptr;
  int n_sel;
  if (n <= kSelCap) {
    const float* sv = slice_val + static_cast<int64_t>(row) * nslice * kFiltSeg;
    const int32_t* si = slice_idx + static_cast<int64_t>(row) * nslice * kFiltSeg;
    for (int q0 = 0; q0 < n; q0 += U * kSegThreads) {
      float xv[U];
      int xi[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kSegThreads + tid;
        int lo = 0, hi = nslice;                  // largest s with offs[s] <= q
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (offs[mid] <= q) lo = mid;
          else hi = mid;
        }
        const int64_t at = static_cast<int64_t>(lo) * kFiltSeg + (q - offs[lo]);
        xv[u] = q < n ? sv[at] : 0.f;
        xi[u] = q < n ? si[at] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kSegThreads + tid;
        if (q < n) {
          cv[q] = xv[u];
          cp[q] = xi[u];
        }
      }
    }
    __syncthreads();
    em.use_lmap = true;
    em.lmap = (const lds_int*)cp;
    // an odd run length keeps the strided run reads free of bank conflicts
    const int r = ((n + kSegThreads - 1) / kSegThreads) | 1;
    n_sel = block_select<NW>(LdsRun{(const lds_float*)cv, n, r}, k, p, em);
  } else {
    const int b = row / Tq;
    const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
    n_sel = block_select<NW>(GlobalRun{scores + row * s_rs, V, (V + kSegThreads - 1) / kSegThreads},
                             k, p, em);
  }
  pad_output<kSegThreads>(em, n_sel, k);
}

int bounded_slices(int N_max) { return (N_max + kFiltSeg - 1) / kFiltSeg; }

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

bool topk_bounded_ok(int N_max) { return bounded_slices(N_max) <= kMaxSlices; }

size_t topk_bounded_workspace_bytes(int rows, int N_max) {
  if (!topk_bounded_ok(N_max)) return 0;
  const size_t ns = static_cast<size_t>(rows) * bounded_slices(N_max);
  return ns * kFiltSeg * (sizeof(float) + sizeof(int32_t)) + ns * sizeof(int32_t);
}

hipError_t launch_topk(const float* scores, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       const float* chunk_thr, int n_chunks, int32_t* idx, float* out_scores,
                       void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (chunk_thr != nullptr && topk_bounded_ok(N_max)) {
    const int ns = bounded_slices(N_max);
    const size_t slots = static_cast<size_t>(rows) * ns * kFiltSeg;
    float* sv = static_cast<float*>(ws);
    int32_t* si = reinterpret_cast<int32_t*>(sv + slots);
    int32_t* sc = si + slots;
    hipLaunchKernelGGL(topk_filter_kernel, dim3(ns, rows), dim3(kSegThreads), 0, s, scores, s_rs,
                       q_pos, n_entries, Tq, N_max, m, k, chunk_thr, n_chunks, ns, sv, si, sc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSegThreads), 0, s, sv, si, sc, ns,
                       scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, idx, out_scores);
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
