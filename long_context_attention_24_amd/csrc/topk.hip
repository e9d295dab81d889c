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
using sel::kRegion;
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
// topk_bounded_kernel: one 1024-thread workgroup per row.
//   1. The row bound and the top of the survivors' range come from the chunk
//      reports, every wave computing them on its own (sel::row_bound), the
//      reports loaded next to the first score loads.
//   2. Survivor list in LDS, in ascending index order, as (score bits, entry
//      index) pairs.  Streamed rows (sel::stream_survivors): rounds of 16384
//      scores, each lane loading 16 scalar scores (entries 64 s + lane of its
//      wave's segment), the next round's loads in flight while the current
//      one is compacted; per round the waves count their survivors with
//      ballots, one block scan gives every wave its offset, and each
//      survivor's slot is that offset plus its rank among the wave's
//      survivors (ballot + mbcnt).  Filtered rows (topk_filter_kernel first,
//      sel::gather_regions): the per-region survivor counts are scanned and
//      the regions copied at their offsets.
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
static_assert(kListCap < 65536, "select_sorted_list packs two list counts into one word");
constexpr int kStreamSlots = 16;                  // scores per lane per round (64 apart)
constexpr int kShortRow = 32768;                  // rows streamed in one round of 32 per thread
static_assert(kMaxBoundedN / kRegion <= kSelThreads, "one region per thread in the offset scan");

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
      const float4 x = sel::load4_scores(src + q);
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
  const float bound = sel::wave_row_bound(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks,
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
// ascending index order and selects from it.  Streaming (REGIONS false): the
// first round's score loads are issued before the row's visible count and
// bound are known (bounded by N_max, masked after).  REGIONS: the per-region
// counts of topk_filter_kernel are gathered.  The bound (when the row has
// one) and the largest chunk report delimit the survivors' range.  More than
// kListCap survivors (inputs far from the expected distribution): the row is
// selected from global memory by block_select instead.
template <bool REGIONS, int SL, typename S>
__global__ __launch_bounds__(kSelThreads) void topk_bounded_kernel(
    const S* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k,
    const float2* __restrict__ chunk_rep, int n_chunks, int nreg,
    const float* __restrict__ reg_val, const int32_t* __restrict__ reg_idx,
    const int32_t* __restrict__ reg_cnt, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  constexpr int NW = kSelWaves;
  constexpr bool kOneRound = SL * kSelThreads >= kShortRow;
  __shared__ u32x2_t lp_s[kListCap];
  lds_u32x2* lp = (lds_u32x2*)lp_s;
  const int row = blockIdx.x, b = row / Tq;
  const int tid = threadIdx.x, wave = tid >> 6;
  const S* srow = scores + row * s_rs;
  float x[SL];
  float2 rt[sel::kRepPerLane];
  if (!REGIONS) {
    sel::load_round(srow, wave * 64 * SL, N_max, x);
    sel::load_reports(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks, rt);
  }
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  float2 rb = make_float2(kNegInf, kNegInf);
  if (!REGIONS) rb = sel::row_bound(rt, n_chunks, bound_c_row(V, k), k);
  g_sm.hist[2 * tid] = 0;
  g_sm.hist[2 * tid + 1] = 0;
  if (tid == 0) g_sm.cand_n = 0;
  int p = 0;
  int n;                                          // block-uniform
  if (REGIONS) {
    const int64_t rbase = static_cast<int64_t>(row) * nreg;
    n = sel::gather_regions<NW>(g_sm, reg_cnt + rbase, reg_val + rbase * kRegion,
                                reg_idx + rbase * kRegion, nreg, lp, kListCap, p);
    rb = sel::wave_row_bound(chunk_rep + static_cast<int64_t>(row) * n_chunks, n_chunks,
                             bound_c_row(V, k), k);
  } else {
    const float bnd = rb.x > kNegInf ? rb.x : -FLT_MAX;     // x >= bnd: a finite survivor
    n = sel::stream_survivors<NW, SL, kOneRound>(g_sm, srow, V, N_max, bnd, lp, kListCap, x, p);
  }
  __syncthreads();                                // the list is complete
  sel::GlobalOut out{out_idx + static_cast<int64_t>(row) * k,
                     out_val ? out_val + static_cast<int64_t>(row) * k : nullptr};
  if (n <= kListCap) {
    const bool have_range = rb.x > kNegInf;       // survivors lie in [bound, largest report]
    sel::select_sorted_list<NW>(g_sm, lp, n, rb.x, rb.y, have_range, k, p, out);
  } else {
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

bool use_regions(int rows, int N_max) { return N_max > kStreamMaxN && rows <= kRegionMaxRows; }

size_t topk_bounded_workspace_bytes(int rows, int N_max) {
  if (!topk_bounded_ok(N_max) || !use_regions(rows, N_max)) return 0;
  const size_t regs = static_cast<size_t>(rows) * filter_regions(N_max);
  return regs * kRegion * (sizeof(float) + sizeof(int32_t)) + regs * sizeof(int32_t);
}

// survivor region buffers at the front of ws: values, entries, counts
void region_buffers(void* ws, int rows, int N_max, float** rv, int32_t** ri, int32_t** rc) {
  const size_t slots = static_cast<size_t>(rows) * filter_regions(N_max) * kRegion;
  *rv = static_cast<float*>(ws);
  *ri = reinterpret_cast<int32_t*>(*rv + slots);
  *rc = *ri + slots;
}

template <typename S>
hipError_t launch_filter(const S* scores, int64_t s_rs, const int32_t* q_pos,
                         const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                         const float2* chunk_rep, int n_chunks, float* rv, int32_t* ri,
                         int32_t* rc, hipStream_t s) {
  const int rows = B * Tq;
  hipLaunchKernelGGL(topk_filter_kernel<S>, dim3((N_max + kFiltSeg - 1) / kFiltSeg, rows),
                     dim3(kSegThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                     chunk_rep, n_chunks, filter_regions(N_max), rv, ri, rc);
  return hipGetLastError();
}

template <typename S>
hipError_t launch_topk_bounded(const S* scores, int64_t s_rs, const int32_t* q_pos,
                               const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                               const float2* chunk_rep, int n_chunks, int32_t* idx,
                               float* out_scores, void* ws, hipStream_t s) {
  const int rows = B * Tq;
  if (!use_regions(rows, N_max)) {
    if (N_max <= kShortRow)
      hipLaunchKernelGGL((topk_bounded_kernel<false, kShortRow / kSelThreads, S>), dim3(rows),
                         dim3(kSelThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                         chunk_rep, n_chunks, 0, nullptr, nullptr, nullptr, idx, out_scores);
    else
      hipLaunchKernelGGL((topk_bounded_kernel<false, kStreamSlots, S>), dim3(rows),
                         dim3(kSelThreads), 0, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k,
                         chunk_rep, n_chunks, 0, nullptr, nullptr, nullptr, idx, out_scores);
    return hipGetLastError();
  }
  const int nreg = filter_regions(N_max);
  float* rv;
  int32_t *ri, *rc;
  region_buffers(ws, rows, N_max, &rv, &ri, &rc);
  const hipError_t e = launch_filter(scores, s_rs, q_pos, n_entries, B, Tq, N_max, m, k, chunk_rep,
                                     n_chunks, rv, ri, rc, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_bounded_kernel<true, kStreamSlots, S>), dim3(rows), dim3(kSelThreads), 0, s, scores,
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
