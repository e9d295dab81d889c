// Top-k selection of compressed entries per query token ("DeepSeek V4 技术解读",
// §2.1: the Lightning Indexer keeps the top-k compressed blocks).
//
// Exact rule: the min(k, V) visible entries with the largest fp32 scores,
// ties to the lower index, -0.0 equal to +0.0, returned in ascending index
// order and padded with -1.
//
// Design (one 1024-thread workgroup per row segment of up to 1024*VPT
// scores, held in LDS; thread t owns a contiguous run of VPT entries so
// thread order is index order):
//   1. block min / max of the valid scores;
//   2. threshold search: an LDS histogram of 2048 equal-width bins over
//      [lo, hi] (bin index is a monotone function of the score), locate the
//      bin holding the k-th largest, narrow [lo, hi] to that bin's min / max
//      and repeat until the bin is taken whole or all candidates are equal;
//   3. ordered compaction: one block-wide exclusive scan of (count > T,
//      count == T) gives every thread its output slot; entries equal to the
//      threshold are taken lowest index first.
// Integer LDS atomics only (counts), so the result is deterministic.  Rows
// longer than one segment are reduced in two passes: each segment keeps its
// own top-k (a superset of its share of the row's top-k), then one workgroup
// selects from the concatenated candidates, which are in index order.
#include <float.h>

#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kSegVpt = 32;
constexpr int kSegLen = kThreads * kSegVpt;   // 32768 scores per workgroup

struct Smem {
  int hist[kBins];
  float rf[kWaves];
  float rf2[kWaves];
  uint32_t ru[kWaves];
  int bstar;
  int bstar_above;
};

__device__ __forceinline__ void block_minmax(float& mn, float& mx, Smem& sm) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm.rf[wave] = mn;
    sm.rf2[wave] = mx;
  }
  __syncthreads();
  float a = sm.rf[0], b = sm.rf2[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    a = fminf(a, sm.rf[w]);
    b = fmaxf(b, sm.rf2[w]);
  }
  __syncthreads();
  mn = a;
  mx = b;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, Smem& sm) {
  v = wave_sum_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sm.ru[wave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += sm.ru[w];
  __syncthreads();
  return r;
}

// exclusive prefix over threads in thread order; also returns the total
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t& total, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane == 63) sm.ru[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t x = sm.ru[w];
    off += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return incl - v + off;
}

// Selects the top-k of the valid values (v > -inf) held by the block in LDS
// (value i of thread t at vals[i * kThreads + t], i.e. row position
// t * VPT + i) and calls emit(position, value, slot) for each, slots 0.. in
// ascending position order.  Returns the number selected (min(k, #valid)).
template <int VPT, typename Emit>
__device__ int block_select(const float* vals, int k, Smem& sm, Emit emit) {
  const int tid = threadIdx.x;
  uint32_t my_valid = 0;
  float mn = FLT_MAX, mx = -FLT_MAX;
  for (int i = 0; i < VPT; ++i) {
    const float x = vals[i * kThreads + tid];
    if (x > kNegInf) {
      ++my_valid;
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
  }
  const uint32_t n_valid = block_sum_u32(my_valid, sm);

  float T = kNegInf;          // selection: all v > T, plus the first take_eq with v == T
  int take_eq = 0;
  if (n_valid > static_cast<uint32_t>(k)) {
    block_minmax(mn, mx, sm);
    float lo = mn, hi = mx;
    int need = k;
    // Each pass shrinks [lo, hi] to one of 2048 equal bins, so at most
    // ceil(log2(range / min spacing) / 11) ~ 26 passes for fp32; 64 is a cap
    // that is never reached.
    for (int iter = 0;; ++iter) {
      if (lo == hi || iter >= 64) {     // all candidates equal
        T = lo;
        take_eq = need;
        break;
      }
      for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0;
      __syncthreads();
      const double dlo = static_cast<double>(lo);
      const double inv = static_cast<double>(kBins) / (static_cast<double>(hi) - dlo);
      for (int i = 0; i < VPT; ++i) {
        const float x = vals[i * kThreads + tid];
        if (x >= lo && x <= hi) {
          const double f = (static_cast<double>(x) - dlo) * inv;
          const int bin = f >= static_cast<double>(kBins - 1) ? kBins - 1 : static_cast<int>(f);
          atomicAdd(&sm.hist[bin], 1);
        }
      }
      __syncthreads();
      // locate the bin b* holding the need-th largest candidate
      const int b0 = 2 * tid, b1 = 2 * tid + 1;
      const uint32_t h0 = sm.hist[b0], h1 = sm.hist[b1];
      uint32_t tot;
      const uint32_t pre = block_excl_scan_u32(h0 + h1, tot, sm);
      const uint32_t above1 = tot - pre - h0 - h1;   // candidates in bins > b1
      const uint32_t above0 = above1 + h1;
      const uint32_t un = static_cast<uint32_t>(need);
      if (above1 < un && un <= above1 + h1) {
        sm.bstar = b1;
        sm.bstar_above = static_cast<int>(above1);
      }
      if (above0 < un && un <= above0 + h0) {
        sm.bstar = b0;
        sm.bstar_above = static_cast<int>(above0);
      }
      __syncthreads();
      const int bstar = sm.bstar;
      need -= sm.bstar_above;
      const int cnt = sm.hist[bstar];
      // min / max of the candidates in bin b*
      float bmn = FLT_MAX, bmx = -FLT_MAX;
      for (int i = 0; i < VPT; ++i) {
        const float x = vals[i * kThreads + tid];
        if (x >= lo && x <= hi) {
          const double f = (static_cast<double>(x) - dlo) * inv;
          const int bin = f >= static_cast<double>(kBins - 1) ? kBins - 1 : static_cast<int>(f);
          if (bin == bstar) {
            bmn = fminf(bmn, x);
            bmx = fmaxf(bmx, x);
          }
        }
      }
      block_minmax(bmn, bmx, sm);
      if (cnt == need) {                // the whole bin is selected
        T = bmn;
        take_eq = kThreads * VPT;
        break;
      }
      lo = bmn;
      hi = bmx;
    }
  }

  // ordered compaction
  uint32_t gt = 0, eq = 0;
  for (int i = 0; i < VPT; ++i) {
    const float x = vals[i * kThreads + tid];
    gt += (x > T) ? 1u : 0u;
    eq += (x == T && x > kNegInf) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_excl_scan_u32(gt | (eq << 16), tot, sm);
  const int gt_before = static_cast<int>(pre & 0xffffu);
  int eq_before = static_cast<int>(pre >> 16);
  const int gt_total = static_cast<int>(tot & 0xffffu);
  const int eq_total = static_cast<int>(tot >> 16);
  int slot = gt_before + min(eq_before, take_eq);
  for (int i = 0; i < VPT; ++i) {
    const float x = vals[i * kThreads + tid];
    bool take = x > T;
    if (!take && x == T && x > kNegInf) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take) {
      if (slot < k) emit(tid * VPT + i, x, slot);   // always true; keeps writes in bounds
      ++slot;
    }
  }
  return min(k, gt_total + min(eq_total, take_eq));
}

// Loads this thread's VPT consecutive values (positions >= valid read as
// -inf, -0.0 stored as +0.0) into the block's LDS row buffer.
template <int VPT>
__device__ __forceinline__ void load_run(const float* __restrict__ p, int valid, float* vals) {
  const int tid = threadIdx.x;
  if (VPT % 4 == 0 && valid >= VPT) {
#pragma unroll
    for (int i = 0; i < VPT; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + i);
      vals[(i + 0) * kThreads + tid] = x.x + 0.0f;
      vals[(i + 1) * kThreads + tid] = x.y + 0.0f;
      vals[(i + 2) * kThreads + tid] = x.z + 0.0f;
      vals[(i + 3) * kThreads + tid] = x.w + 0.0f;
    }
  } else {
    for (int i = 0; i < VPT; ++i) vals[i * kThreads + tid] = (i < valid) ? p[i] + 0.0f : kNegInf;
  }
  __syncthreads();
}

// Pass 1: one workgroup per (segment, row) of the score matrix.  With a single
// segment per row it writes the final answer; otherwise the segment's top-k
// candidates (value, entry index) go to the workspace.
template <int VPT>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t s_rs, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, int k, int nseg,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, float* __restrict__ cand_val,
    int32_t* __restrict__ cand_idx) {
  __shared__ Smem sm;
  __shared__ float vals[kThreads * VPT];
  constexpr int seg_len = kThreads * VPT;
  const int seg = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int seg0 = seg * seg_len;
  const int L = max(0, min(V - seg0, seg_len));
  const int my0 = threadIdx.x * VPT;
  load_run<VPT>(scores + row * s_rs + seg0 + my0, L - my0, vals);

  int32_t* oi;
  float* ov;
  if (nseg == 1) {
    oi = out_idx + static_cast<int64_t>(row) * k;
    ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  } else {
    const int64_t base = (static_cast<int64_t>(row) * nseg + seg) * k;
    oi = cand_idx + base;
    ov = cand_val + base;
  }
  const int n = block_select<VPT>(vals, k, sm, [&](int pos, float val, int slot) {
    oi[slot] = seg0 + pos;
    if (ov) ov[slot] = val;
  });
  for (int s = n + threadIdx.x; s < k; s += kThreads) {
    oi[s] = -1;
    if (ov) ov[s] = kNegInf;
  }
}

// Pass 2: one workgroup per row over the nseg*k candidates of pass 1.
template <int VPT>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(
    const float* __restrict__ cand_val, const int32_t* __restrict__ cand_idx, int nseg, int k,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  __shared__ Smem sm;
  __shared__ float vals[kThreads * VPT];
  const int row = blockIdx.x;
  const int len = nseg * k;
  const int my0 = threadIdx.x * VPT;
  const float* cv = cand_val + static_cast<int64_t>(row) * len;
  const int32_t* ci = cand_idx + static_cast<int64_t>(row) * len;
  load_run<VPT>(cv + my0, len - my0, vals);
  int32_t* oi = out_idx + static_cast<int64_t>(row) * k;
  float* ov = out_val ? out_val + static_cast<int64_t>(row) * k : nullptr;
  const int n = block_select<VPT>(vals, k, sm, [&](int pos, float val, int slot) {
    oi[slot] = ci[pos];
    if (ov) ov[slot] = val;
  });
  for (int s = n + threadIdx.x; s < k; s += kThreads) {
    oi[s] = -1;
    if (ov) ov[s] = kNegInf;
  }
}

int rows_vpt(int N_max) {
  if (N_max <= kThreads) return 1;
  if (N_max <= 4 * kThreads) return 4;
  if (N_max <= 16 * kThreads) return 16;
  return kSegVpt;
}

int num_segments(int N_max) {
  const int vpt = rows_vpt(N_max);
  const int seg_len = kThreads * vpt;
  return (N_max + seg_len - 1) / seg_len;
}

template <int VPT>
void launch_rows(dim3 grid, hipStream_t s, const float* scores, int64_t s_rs, const int32_t* q_pos,
                 const int32_t* n_entries, int Tq, int N_max, int m, int k, int nseg, int32_t* idx,
                 float* val, float* cv, int32_t* ci) {
  hipLaunchKernelGGL(topk_rows_kernel<VPT>, grid, dim3(kThreads), 0, s, scores, s_rs, q_pos,
                     n_entries, Tq, N_max, m, k, nseg, idx, val, cv, ci);
}

template <int VPT>
void launch_merge(int rows, hipStream_t s, const float* cv, const int32_t* ci, int nseg, int k,
                  int32_t* idx, float* val) {
  hipLaunchKernelGGL(topk_merge_kernel<VPT>, dim3(rows), dim3(kThreads), 0, s, cv, ci, nseg, k,
                     idx, val);
}

}  // namespace

bool topk_supported(int N_max, int k) {
  if (k < 1 || k > 2048 || N_max < 1) return false;
  const long long cand = static_cast<long long>(num_segments(N_max)) * k;
  return num_segments(N_max) == 1 || cand <= kSegLen;
}

size_t topk_workspace_bytes(int rows, int N_max, int k) {
  const int nseg = num_segments(N_max);
  if (nseg == 1) return 0;
  return static_cast<size_t>(rows) * nseg * k * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_topk(const float* scores, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       int32_t* idx, float* out_scores, void* ws, hipStream_t s) {
  const int rows = B * Tq;
  const int vpt = rows_vpt(N_max);
  const int nseg = num_segments(N_max);
  float* cv = nullptr;
  int32_t* ci = nullptr;
  if (nseg > 1) {
    cv = static_cast<float*>(ws);
    ci = reinterpret_cast<int32_t*>(cv + static_cast<size_t>(rows) * nseg * k);
  }
  const dim3 grid(nseg, rows);
  switch (vpt) {
    case 1: launch_rows<1>(grid, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, nseg, idx, out_scores, cv, ci); break;
    case 4: launch_rows<4>(grid, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, nseg, idx, out_scores, cv, ci); break;
    case 16: launch_rows<16>(grid, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, nseg, idx, out_scores, cv, ci); break;
    default: launch_rows<kSegVpt>(grid, s, scores, s_rs, q_pos, n_entries, Tq, N_max, m, k, nseg, idx, out_scores, cv, ci); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nseg == 1) return e;
  const int len = nseg * k;
  if (len <= kThreads) launch_merge<1>(rows, s, cv, ci, nseg, k, idx, out_scores);
  else if (len <= 4 * kThreads) launch_merge<4>(rows, s, cv, ci, nseg, k, idx, out_scores);
  else if (len <= 16 * kThreads) launch_merge<16>(rows, s, cv, ci, nseg, k, idx, out_scores);
  else launch_merge<kSegVpt>(rows, s, cv, ci, nseg, k, idx, out_scores);
  return hipGetLastError();
}

}  // namespace csa
