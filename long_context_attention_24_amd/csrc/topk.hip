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
#include <limits.h>

#include "device_common.h"
#include "internal.h"
#include "select_core.h"

namespace csa {
namespace {

using sel::kBins;
using sel::kMaxBoundedN;
using sel::lds_float;
using sel::lds_u32x2;
using sel::u32x2_t;

// row-segment kernel
constexpr int kSegThreads = 256;
constexpr int kSegCap = 32768;                    // values per workgroup (128 per thread)
constexpr int kMaxK = 2048;

// the selection kernels' scratch: one file-scope LDS object per workgroup
__shared__ sel::SelScratch g_sm;

// LDS run of R values per thread in the transposed layout v[i*THREADS + t];
// position pos is entry base + pos.
template <int THREADS>
struct SplitRun {
  static constexpr int kUnroll = 1;
  const lds_float* v;
  int r;
  int base;
  __device__ __forceinline__ int len() const { return r; }
  __device__ __forceinline__ float get(int i) const { return v[i * THREADS + threadIdx.x]; }
  __device__ __forceinline__ int entry(int pos) const { return base + pos; }
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
  sel::zero_hist<NW>(g_sm);
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
  sel::GlobalOut em;
  if (MERGE || nseg == 1) {
    em.oi = out_idx + static_cast<int64_t>(row) * k;
    em.ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  } else {
    const int64_t base = (static_cast<int64_t>(row) * nseg + seg) * k;
    em.oi = cand_idx + base;
    em.ov = cand_val + base;
  }
  // MERGE: list positions first, mapped to entry indices below
  const int n_sel = sel::block_select<NW>(
      g_sm, SplitRun<kSegThreads>{lb, R, MERGE ? 0 : seg * kSegCap}, k, p, em);
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
  sel::pad_output<NW>(em, n_sel, k);
}

// ============================================================ bounded path
// topk_bounded_kernel: one 1024-thread workgroup per row (topk_fused_kernel
// below for few long rows).
//   1. The row bound and the top of the survivors' range come from the chunk
//      reports, every wave computing them on its own (sel::row_bound), the
//      reports loaded next to the first score loads.
//   2. Survivor lists in LDS, in ascending index order, as (score bits, entry
//      index) pairs, each lane loading scalar scores (entries 64 s + lane of
//      its wave's segment).  Rows of at most 32768 entries are read in one
//      round of 32 scores per lane, and every wave compacts its segment into
//      its own list as soon as its scores arrive (sel::stream_wave_list:
//      ballots, mbcnt, branch-free stores), the wave lists in wave order
//      being the row's survivors in index order (sel::WaveLists).  Longer
//      rows stream in rounds of 16384 scores into one list
//      (sel::stream_survivors), the next round's loads in flight while the
//      current one is compacted; per round the waves count their survivors
//      with ballots, one block scan gives every wave its offset, and each
//      survivor's slot is that offset plus its rank among the wave's
//      survivors (ballot + mbcnt).
//   3. sel::select_sorted_list: a 2048-bin equal-width histogram over
//      [bound, top] locates the bin of the k-th largest; a bin of at most 256
//      entries is finished by pairwise ranks, a larger one narrows the range
//      to the bin and repeats.  Because the list is in index order, one block
//      scan of the pair (count > T, count == T) over contiguous per-thread
//      runs gives every selected entry its output slot: ascending indices,
//      and among entries equal to the threshold the lowest indices.
// A row whose survivors overflow the list selects from the score row
// directly (sel::block_select, slow but exact).
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
static_assert(kBins % kSelThreads == 0, "whole bins per thread");
constexpr int kListCap = 16 * kSelThreads;        // survivors held in LDS
constexpr int kWaveCap = kListCap / kSelWaves;    // per wave, for rows streamed in one round
static_assert(kListCap < 65536, "select_sorted_list packs two list counts into one word");
constexpr int kStreamSlots = 16;                  // scores per lane per round (64 apart)
constexpr int kShortRow = 32768;                  // rows streamed in one round of 32 per thread

// Few long rows (at most kFusedMaxRows rows of more than kFusedMinN entries:
// one workgroup per row would leave most of the chip idle while it reads the
// row) are filtered and selected by one kernel, topk_fused_kernel: one
// 1024-thread workgroup per 4096 entries of a row, each wave owning 256 of
// them (four per lane, one 16- or 8-byte load).  Wave 0 derives the row
// bound and the top of the survivors' range from the chunk reports while the
// other waves' loads are in flight; every workgroup then compacts its entries
// at or above the bound, in index order, to its segment of the survivor
// buffer (one block scan of the wave counts; a segment keeps at most
// kFusedSegCap, and a row with a fuller segment takes the fallback), stores
// their number, and arrives at the row's counter.  The workgroup that
// arrives last (no wait: the others simply end) gathers the row's segments
// into an LDS list in index order, one load per list position (the
// position's segment found by binary search over the segment offsets), and
// selects from it with sel::select_sorted_list.  Survivor stores, counts and the gather's loads
// are device-coherent (they bypass the per-XCD L2), each workgroup's stores
// complete before it arrives, and the last workgroup resets the counter, so
// the counters (one 64-byte line per row, at the front of the workspace)
// are zero before and after every call.
constexpr int kFusedSeg = kSelThreads / 64 * 256; // entries per workgroup
constexpr int kFusedSegCap = 1024;                // survivors a segment keeps (more: fallback)
constexpr int kFusedMaxRows = 64;
constexpr int kFusedMinN = 65536;
constexpr int kSyncStride = 16;                   // uint32 words per row's counter
static_assert(kMaxBoundedN / kFusedSeg <= 64, "segment offsets scanned by one wave");

__device__ __forceinline__ void st_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int fused_segments(int N_max) { return (N_max + kFusedSeg - 1) / kFusedSeg; }

template <typename S>
__global__ __launch_bounds__(kSelThreads) void topk_fused_kernel(
    const S* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float2* __restrict__ chunk_rep, int n_chunks, int nseg, uint64_t* __restrict__ seg_buf,
    uint32_t* __restrict__ seg_cnt, uint32_t* __restrict__ sync, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  constexpr int NW = kSelWaves;
  constexpr int NT = kSelThreads;
  __shared__ u32x2_t lp_s[kListCap];
  lds_u32x2* lp = (lds_u32x2*)lp_s;
  const int seg = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const S* srow = scores + row * s_rs;
  // four scores per lane: entries e0 .. e0 + 3, loads bounded by N_max
  const int e0 = seg * kFusedSeg + wave * 256 + 4 * lane;
  float v[4];
  if (e0 + 3 < N_max) {
    const float4 x = sel::load4_scores(srow + e0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e0 + e < N_max ? get_score(srow + e0 + e) : kNegInf;
  }
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  if (wave == 0) {
    const float2 rb = sel::wave_row_bound(chunk_rep + static_cast<int64_t>(row) * n_chunks,
                                          n_chunks, bound_c_row(V, k), k);
    if (lane == 0) {
      g_sm.lo = rb.x;
      g_sm.hi = rb.y;
    }
  }
  g_sm.hist[2 * tid] = 0;
  g_sm.hist[2 * tid + 1] = 0;
  if (tid == 0) g_sm.cand_n = 0;
  __syncthreads();
  const float lo = g_sm.lo, hi = g_sm.hi;
  const float bnd = lo > kNegInf ? lo : -FLT_MAX;            // x >= bnd: a finite survivor
  bool keep[4];
  uint32_t cl = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    keep[e] = e0 + e < V && v[e] >= bnd;
    cl += keep[e] ? 1u : 0u;
  }
  int p = 0;
  uint32_t seg_n;
  uint32_t q = sel::block_excl_scan<NW>(g_sm, cl, seg_n, p);
  uint64_t* dst = seg_buf + (static_cast<int64_t>(row) * nseg + seg) * kFusedSegCap;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (keep[e]) {
      if (q < static_cast<uint32_t>(kFusedSegCap))   // the count keeps growing: see below
        st_coherent(dst + q, static_cast<uint64_t>(__float_as_uint(v[e] + 0.0f)) |
                                 (static_cast<uint64_t>(e0 + e) << 32));
      ++q;
    }
  }
  if (tid == 0) st_coherent(seg_cnt + static_cast<int64_t>(row) * nseg + seg, seg_n);
  __builtin_amdgcn_s_waitcnt(0);                  // this thread's stores are complete
  __syncthreads();
  if (tid == 0) {
    uint32_t* ctr = sync + kSyncStride * row;
    const bool last =
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        static_cast<uint32_t>(nseg - 1);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_sm.last = last ? 1 : 0;
  }
  __syncthreads();
  if (g_sm.last == 0) return;                     // block-uniform
  // the last workgroup of the row: segment offsets (nseg <= 64: wave 0 scans),
  // padded to 64 entries with an offset no list position reaches; a segment
  // with more survivors than it kept sends the row to the fallback
  if (wave == 0) {
    const uint32_t c =
        lane < nseg ? ld_coherent(seg_cnt + static_cast<int64_t>(row) * nseg + lane) : 0u;
    const uint32_t incl = wave_incl_scan_u32(c);
    g_sm.tab[lane] = lane < nseg ? incl - c : 0x7fffffffu;
    const bool over = __builtin_amdgcn_ballot_w64(c > static_cast<uint32_t>(kFusedSegCap)) != 0;
    if (lane == 63) g_sm.cand_n = over ? 0xffffffffu : incl;   // the list length, read below
  }
  __syncthreads();
  const uint32_t nl = g_sm.cand_n;
  __syncthreads();
  if (tid == 0) g_sm.cand_n = 0;
  sel::GlobalOut out{out_idx + static_cast<int64_t>(row) * k,
                     out_val ? out_val + static_cast<int64_t>(row) * k : nullptr};
  if (nl > static_cast<uint32_t>(kListCap)) {     // far from the expected distribution
    const int n_sel = sel::block_select<NW>(
        g_sm, sel::GlobalRun<S>{srow, V, (V + NT - 1) / NT}, k, p, out);
    sel::pad_output<NW>(out, n_sel, k);
    return;
  }
  // gather: list position j from segment s = the last with offset <= j; all
  // of a thread's loads in flight together; the first histogram pass of the
  // selection is built from the gathered values
  const int n = static_cast<int>(nl);
  const uint64_t* rowbuf = seg_buf + static_cast<int64_t>(row) * nseg * kFusedSegCap;
  constexpr int kG = kListCap / NT;
  constexpr int kQ = 4;                           // positions searched together
  uint64_t e[kG];
#pragma unroll
  for (int g0 = 0; g0 < kG; g0 += kQ) {
    if (g0 * NT >= n) break;                      // uniform
    int sg[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) sg[q] = 0;
#pragma unroll
    for (int st = 32; st > 0; st >>= 1) {         // six halvings over the 64 offsets, every
#pragma unroll                                    // position's read issued unconditionally
      for (int q = 0; q < kQ; ++q)
        sg[q] += static_cast<int>(g_sm.tab[sg[q] + st]) <= tid + (g0 + q) * NT ? st : 0;
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int j = tid + (g0 + q) * NT;
      if (j < n)
        e[g0 + q] = ld_coherent(rowbuf + static_cast<int64_t>(sg[q]) * kFusedSegCap +
                                (j - static_cast<int>(g_sm.tab[sg[q]])));
    }
  }
  const bool have_range = lo > kNegInf;           // survivors lie in [bound, largest report]
  const sel::HistRange hr = sel::hist_range(lo, hi);
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int j = tid + g * NT;
    if (j < n) {
      lp[j] = u32x2_t{static_cast<uint32_t>(e[g]), static_cast<uint32_t>(e[g] >> 32)};
      if (have_range) sel::hist_add(g_sm, hr, __uint_as_float(static_cast<uint32_t>(e[g])));
    }
  }
  __syncthreads();                                // the list and first histogram are complete
  sel::select_sorted_list<NW>(g_sm, sel::FlatList<NT>{lp, n}, lo, hi, have_range, k, p, out,
                              true);
}

// One 1024-thread workgroup per row streams the row into a survivor list in
// LDS, in ascending index order, and selects from it.  The first round's
// score loads are issued before the row's visible count and bound are known
// (bounded by N_max, masked after).  The bound (when the row has one) and the
// largest chunk report delimit the survivors' range.  More than kListCap
// survivors (inputs far from the expected distribution): the row is selected
// from global memory by block_select instead.
template <int SL, typename S>
__global__ __launch_bounds__(kSelThreads) void topk_bounded_kernel(
    const S* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float2* __restrict__ chunk_rep, int n_chunks, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  constexpr int NW = kSelWaves;
  constexpr bool kOneRound = SL * kSelThreads >= kShortRow;
  __shared__ u32x2_t lp_s[kListCap + (kOneRound ? kSelThreads : 0)];   // + a spare entry per thread
  lds_u32x2* lp = (lds_u32x2*)lp_s;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, wave = tid >> 6;
  const S* srow = scores + row * s_rs;
  float x[SL];
  float2 rt[sel::kRepPerLane];
  sel::load_round(srow, wave * 64 * SL, N_max, x);
  sel::load_reports(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks, rt);
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const float2 rb = sel::row_bound(rt, n_chunks, bound_c_row(V, k), k);
  g_sm.hist[2 * tid] = 0;
  g_sm.hist[2 * tid + 1] = 0;
  if (tid == 0) g_sm.cand_n = 0;
  int p = 0;
  const float bnd = rb.x > kNegInf ? rb.x : -FLT_MAX;       // x >= bnd: a finite survivor
  const bool have_range = rb.x > kNegInf;         // survivors lie in [bound, largest report]
  sel::GlobalOut out{out_idx + static_cast<int64_t>(row) * k,
                     out_val ? out_val + static_cast<int64_t>(row) * k : nullptr};
  bool fits;
  if constexpr (kOneRound) {
    // every wave compacts into its own list as its scores arrive
    const int cnt = sel::stream_wave_list<kWaveCap, SL>(wave * 64 * SL, V, bnd, lp, kListCap, x);
    if ((tid & 63) == 0) g_sm.wcnt[wave] = static_cast<uint32_t>(cnt);
    __syncthreads();                              // the lists are complete
    const uint32_t c = (tid & 63) < NW ? g_sm.wcnt[tid & 63] : 0u;
    const int n = static_cast<int>(sel::dpp_sum_u32(c));
    fits = sel::dpp_max_u32(c) <= static_cast<uint32_t>(kWaveCap);
    if (fits)
      sel::select_sorted_list<NW>(g_sm, sel::WaveLists<kWaveCap>{lp, cnt, n}, rb.x, rb.y,
                                  have_range, k, p, out);
  } else {
    const int n =                                 // block-uniform
        sel::stream_survivors<NW, SL>(g_sm, srow, V, N_max, bnd, lp, kListCap, x, p);
    __syncthreads();                              // the list is complete
    fits = n <= kListCap;
    if (fits)
      sel::select_sorted_list<NW>(g_sm, sel::FlatList<kSelThreads>{lp, n}, rb.x, rb.y,
                                  have_range, k, p, out);
  }
  if (!fits) {
    const int n_sel = sel::block_select<NW>(
        g_sm, sel::GlobalRun<S>{srow, V, (V + kSelThreads - 1) / kSelThreads}, k, p, out);
    sel::pad_output<NW>(out, n_sel, k);
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

bool use_fused(int rows, int N_max) { return N_max > kFusedMinN && rows <= kFusedMaxRows; }

size_t topk_bounded_workspace_bytes(int rows, int N_max) {
  if (!topk_bounded_ok(N_max) || !use_fused(rows, N_max)) return 0;
  const size_t segs = static_cast<size_t>(rows) * fused_segments(N_max);
  return segs * kFusedSegCap * sizeof(uint64_t) + segs * sizeof(uint32_t);
}

size_t topk_sync_bytes() {
  return static_cast<size_t>(kFusedMaxRows) * kSyncStride * sizeof(uint32_t);
}

template <typename S>
hipError_t launch_topk_bounded(const S* scores, int64_t s_rs, const int32_t* q_pos,
                               const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                               const float2* chunk_rep, int n_chunks, int32_t* idx,
                               float* out_scores, void* ws, uint32_t* sync, hipStream_t s) {
  const int rows = B * Tq;
  if (!use_fused(rows, N_max)) {
    if (N_max <= kShortRow)
      hipLaunchKernelGGL((topk_bounded_kernel<kShortRow / kSelThreads, S>), dim3(rows),
                         dim3(kSelThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                         chunk_rep, n_chunks, idx, out_scores);
    else
      hipLaunchKernelGGL((topk_bounded_kernel<kStreamSlots, S>), dim3(rows), dim3(kSelThreads),
                         0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_rep,
                         n_chunks, idx, out_scores);
    return hipGetLastError();
  }
  // survivor segments at the front of ws, then their counts
  const int nseg = fused_segments(N_max);
  uint64_t* seg_buf = static_cast<uint64_t*>(ws);
  uint32_t* seg_cnt =
      reinterpret_cast<uint32_t*>(seg_buf + static_cast<size_t>(rows) * nseg * kFusedSegCap);
  hipLaunchKernelGGL(topk_fused_kernel<S>, dim3(nseg, rows), dim3(kSelThreads), 0, s, scores,
                     s_rs, q_pos, n_entries, Tq, N_max, m, k, chunk_rep, n_chunks, nseg, seg_buf,
                     seg_cnt, sync, idx, out_scores);
  return hipGetLastError();
}

hipError_t launch_topk(const void* scores_v, bool score16, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       const float2* chunk_rep, int n_chunks, int32_t* idx, float* out_scores,
                       void* ws, uint32_t* sync, hipStream_t s) {
  const int rows = B * Tq;
  if (score16)   // bf16 rows: the bounded path only (the caller checks chunk_rep and N_max)
    return launch_topk_bounded(static_cast<const uint16_t*>(scores_v), s_rs, q_pos, n_entries, B,
                               Tq, N_max, m, k, chunk_rep, n_chunks, idx, out_scores, ws, sync, s);
  const float* scores = static_cast<const float*>(scores_v);
  if (chunk_rep != nullptr && topk_bounded_ok(N_max))
    return launch_topk_bounded(scores, s_rs, q_pos, n_entries, B, Tq, N_max, m, k, chunk_rep,
                               n_chunks, idx, out_scores, ws, sync, s);
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
