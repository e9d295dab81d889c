// Core attention over compressed entries: CSA attends only the top-k
// entries chosen by the indexer ("DeepSeek V4 技术解读", §2.1 core attention);
// HCA attends every visible entry (§2.2).  One shared KV head for all query
// heads.
//
// Tuned path (bf16, 64 heads x 128): split the entry list into fixed-length
// splits (a constant, so a sequence's result never depends on its batch),
// one workgroup per (query, split), then a combine kernel merges the split
// partials with their running maxima.  Inside a split, tiles of 32 entries
// go through MFMA with the entries as M and the heads as N:
//     S^T[j, h] = K[j] . q[h]           (A = K rows, B = q^T, in registers)
//     O^T[d, h] += V^T[d, j] P^T[j, h]  (A = V^T from LDS, B = P^T)
// With that orientation each lane owns one head column, so the online
// softmax is lane-local (plus one exchange with lane l^32) and the softmax
// probabilities leave the S accumulator already in the B-operand layout of
// the PV product.  V rows are transposed into LDS (double buffered).
// Softmax runs in base 2 with the scale folded into log2(e).
#include <float.h>

#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

// ---------------------------------------------------------------- generic (VALU)
template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename T>
__device__ __forceinline__ void stf(T* p, float v);
template <>
__device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void stf<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

constexpr int kGenThreads = 128;

template <typename T, int D, bool HCA>
__global__ __launch_bounds__(kGenThreads) void attend_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ Vc, int64_t kv_sb,
    int64_t kv_sn, const int32_t* __restrict__ idx, int kk, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int H, int N_max, int m, float scale_log2,
    T* __restrict__ out, float* __restrict__ lse) {
  __shared__ float qs[D];
  __shared__ float p_s[kGenThreads];
  __shared__ int j_s[kGenThreads];
  __shared__ float red[kGenThreads / 64];
  const int h = blockIdx.x, row = blockIdx.y, b = row / Tq, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const T* qh = q + (static_cast<int64_t>(row) * H + h) * D;
  for (int d = tid; d < D; d += kGenThreads) qs[d] = ldf<T>(qh + d) * scale_log2;
  const int n_ent = min(n_entries[b], N_max);
  const int n = HCA ? visible_count(q_pos[row], m, n_entries[b], N_max) : kk;
  const T* Kb = K + b * kv_sb;
  const T* Vb = Vc + b * kv_sb;
  __syncthreads();
  float m_run = kNegInf, l_run = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < n; c0 += kGenThreads) {
    const int i = c0 + tid;
    int j = -1;
    if (i < n) {
      j = HCA ? i : idx[static_cast<int64_t>(row) * kk + i];
      if (j < 0 || j >= n_ent) j = -1;
    }
    float logit = kNegInf;
    if (j >= 0) {
      const T* kr = Kb + static_cast<int64_t>(j) * kv_sn;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], ldf<T>(kr + d), dot);
      logit = dot;
    }
    float cmax = wave_max(logit);
    if (lane == 0) red[wave] = cmax;
    __syncthreads();
    cmax = red[0];
    for (int w = 1; w < kGenThreads / 64; ++w) cmax = fmaxf(cmax, red[w]);
    __syncthreads();
    const float m_new = fmaxf(m_run, cmax);
    float p = 0.f, alpha = 1.f;
    if (m_new != kNegInf) {
      alpha = exp2_fast(m_run - m_new);
      p = (j >= 0) ? exp2_fast(logit - m_new) : 0.f;
    }
    p_s[tid] = p;
    j_s[tid] = j;
    float psum = wave_sum(p);
    if (lane == 0) red[wave] = psum;
    __syncthreads();
    psum = 0.f;
    for (int w = 0; w < kGenThreads / 64; ++w) psum += red[w];
    l_run = l_run * alpha + psum;
    for (int d = tid; d < D; d += kGenThreads) {
      float a = acc * alpha;
      const int cnt = min(kGenThreads, n - c0);
      for (int t = 0; t < cnt; ++t) {
        const int jj = j_s[t];
        if (jj >= 0) a = fmaf(p_s[t], ldf<T>(Vb + static_cast<int64_t>(jj) * kv_sn + d), a);
      }
      acc = a;
    }
    m_run = m_new;
    __syncthreads();
  }
  T* oh = out + (static_cast<int64_t>(row) * H + h) * D;
  for (int d = tid; d < D; d += kGenThreads) stf<T>(oh + d, l_run > 0.f ? acc / l_run : 0.f);
  if (lse != nullptr && tid == 0)
    lse[static_cast<int64_t>(row) * H + h] =
        l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------- bf16 64 x 128, split
constexpr int kCsaSplit = 64;      // entries of the top-k list per workgroup (one tile per wave)
constexpr int kHcaSplit = 512;     // visible entries per workgroup
constexpr int kPartStride = 132;   // floats per (split, head): O[128], m, l, pad
constexpr int kVtRow = 36;         // bf16 per V^T row in LDS (32 entries + pad)

struct AttnSmem {
  uint16_t vt[2][2][128 * kVtRow];   // [buffer][key group][d][entry]
};

template <bool HCA>
__global__ __launch_bounds__(256) void attend_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vc, int64_t kv_sb, int64_t kv_sn, const int32_t* __restrict__ idx,
    int kk, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq,
    int N_max, int m, float scale_log2, int split_len, int nsplit, float* __restrict__ part) {
  __shared__ AttnSmem sm;
  const int split = blockIdx.x, row = blockIdx.y, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = wave & 1, kg = wave >> 1;
  const int jl = lane & 31, g = lane >> 5;
  const int h = 32 * hh + jl;        // this lane's head (S^T / O^T column)
  const int n_ent = min(n_entries[b], N_max);
  const int n = HCA ? visible_count(q_pos[row], m, n_entries[b], N_max) : kk;
  const int s0 = split * split_len;
  const int s_end = min(n, s0 + split_len);
  const int ntiles = s_end > s0 ? (s_end - s0 + 31) / 32 : 0;
  const int nrounds = (ntiles + 1) / 2;

  // B operand: q^T for this wave's 32 heads, 8 k-steps; dims 16s + 8g + e
  const uint16_t* qrow = q + static_cast<int64_t>(row) * 64 * 128;
  bf16x8_t bq[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) bq[s] = ld_bf16x8(qrow + h * 128 + 16 * s + 8 * g);

  const uint16_t* Kb = K + b * kv_sb;
  const uint16_t* Vb = Vc + b * kv_sb;
  f32x16_t o[4] = {};
  float m_run = kNegInf, l_run = 0.f;

  for (int r = 0; r < nrounds; ++r) {
    const int t = 2 * r + kg;
    const bool active = t < ntiles;
    const int p0 = s0 + 32 * t;
    // entry of tile row jl (the A-operand row this lane loads)
    int ej = -1;
    if (active && p0 + jl < s_end) {
      ej = HCA ? p0 + jl : idx[static_cast<int64_t>(row) * kk + p0 + jl];
      if (ej < 0 || ej >= n_ent) ej = -1;
    }
    const uint32_t vmask = static_cast<uint32_t>(__ballot(ej >= 0));   // bits 0..31: rows
    // A operand: K rows (zero for invalid rows)
    bf16x8_t ak[8];
    if (ej >= 0) {
      const uint16_t* kr = Kb + static_cast<int64_t>(ej) * kv_sn + 8 * g;
#pragma unroll
      for (int s = 0; s < 8; ++s) ak[s] = ld_bf16x8(kr + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) ak[s] = bf16x8_t{};
    }
    // V rows -> V^T in LDS: the key group's 128 threads cover 32 rows x 16 chunks
    uint16_t* vt = sm.vt[r & 1][kg];
    {
      const int t128 = hh * 64 + lane;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int pair = t128 + 128 * it;      // 0..511
        const int vr = pair >> 4, ch = pair & 15;
        int ev = -1;
        if (active && p0 + vr < s_end) {
          ev = HCA ? p0 + vr : idx[static_cast<int64_t>(row) * kk + p0 + vr];
          if (ev < 0 || ev >= n_ent) ev = -1;
        }
        uint4 x = make_uint4(0, 0, 0, 0);
        if (ev >= 0) x = ld16(Vb + static_cast<int64_t>(ev) * kv_sn + 8 * ch);
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[(8 * ch + 2 * e) * kVtRow + vr] = static_cast<uint16_t>(w4[e] & 0xffffu);
          vt[(8 * ch + 2 * e + 1) * kVtRow + vr] = static_cast<uint16_t>(w4[e] >> 16);
        }
      }
    }
    __syncthreads();
    if (!active) continue;

    // S^T = K q^T : lane holds column h, rows j = 8*(i/4) + 4*g + i%4
    f32x16_t sacc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[s], bq[s], sacc, 0, 0, 0);
    float x[16];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 8 * (i >> 2) + 4 * g + (i & 3);
      x[i] = ((vmask >> j) & 1u) ? sacc[i] * scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.f;
    uint32_t pb[8];
    float psum = 0.f;
    if (m_new != kNegInf) {
      alpha = exp2_fast(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint16_t lo = f32_to_bf16(exp2_fast(x[i] - m_new));
        const uint16_t hi = f32_to_bf16(exp2_fast(x[i + 1] - m_new));
        psum += bf16_to_f32(lo) + bf16_to_f32(hi);
        pb[i >> 1] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = 0;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    // O^T += V^T P^T over the tile's two 16-entry k-steps
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8_t bp;
      __builtin_memcpy(&bp, &pb[4 * s2], 16);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vrow = vt + (32 * dt + jl) * kVtRow + 16 * s2 + 4 * g;
        uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        const uint32_t av[4] = {lo.x, lo.y, hi.x, hi.y};
        bf16x8_t a;
        __builtin_memcpy(&a, av, 16);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[dt], 0, 0, 0);
      }
    }
  }

  // merge the two key groups of each head half through LDS (reuses V^T space)
  l_run = l_run + __shfl_xor(l_run, 32, 64);
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&sm.vt[0][0][0]);   // [hh][lane][64 + 2]
  constexpr int kX = 66;
  if (kg == 1) {
    float* dst = xo + (hh * 64 + lane) * kX;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[16 * dt + i] = o[dt][i];
    dst[64] = m_run;
    dst[65] = l_run;
  }
  __syncthreads();
  if (kg == 0) {
    const float* src = xo + (hh * 64 + lane) * kX;
    const float m1 = src[64], l1 = src[65];
    const float M = fmaxf(m_run, m1);
    float a0 = 0.f, a1 = 0.f;
    if (M != kNegInf) {
      a0 = exp2_fast(m_run - M);
      a1 = exp2_fast(m1 - M);
    }
    float* pr = part + ((static_cast<int64_t>(row) * nsplit + split) * 64 + h) * kPartStride;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3);
        pr[d] = a0 * o[dt][i] + a1 * src[16 * dt + i];
      }
    if (g == 0) {
      pr[128] = M;
      pr[129] = a0 * l_run + a1 * l1;
    }
  }
}

// Merge of the split partials.  Grid (rows, 4 head groups); thread (h, c)
// owns 8 output dims of one head.  All splits' maxima are read first (one
// round of independent loads), then all partial rows.
constexpr int kCombineUnroll = 8;

__global__ __launch_bounds__(256) void attend_combine_kernel(const float* __restrict__ part,
                                                             int nsplit, uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int row = blockIdx.x, tid = threadIdx.x;
  const int h = blockIdx.y * 16 + (tid >> 4), dc = (tid & 15) * 8;
  const int64_t sstride = 64 * kPartStride;
  const float* base = part + (static_cast<int64_t>(row) * nsplit * 64 + h) * kPartStride;
  float M = kNegInf;
  int s = 0;
  for (; s + kCombineUnroll <= nsplit; s += kCombineUnroll) {
    float mm[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) mm[u] = base[(s + u) * sstride + 128];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) M = fmaxf(M, mm[u]);
  }
  for (; s < nsplit; ++s) M = fmaxf(M, base[s * sstride + 128]);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (M != kNegInf) {
    s = 0;
    for (; s + kCombineUnroll <= nsplit; s += kCombineUnroll) {
      float4 lo[kCombineUnroll], hi[kCombineUnroll];
      float ml[kCombineUnroll], ll[kCombineUnroll];
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const float* ps = base + (s + u) * sstride;
        lo[u] = *reinterpret_cast<const float4*>(ps + dc);
        hi[u] = *reinterpret_cast<const float4*>(ps + dc + 4);
        ml[u] = ps[128];
        ll[u] = ps[129];
      }
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const float w = exp2_fast(ml[u] - M);
        L = fmaf(w, ll[u], L);
        acc[0] = fmaf(w, lo[u].x, acc[0]); acc[1] = fmaf(w, lo[u].y, acc[1]);
        acc[2] = fmaf(w, lo[u].z, acc[2]); acc[3] = fmaf(w, lo[u].w, acc[3]);
        acc[4] = fmaf(w, hi[u].x, acc[4]); acc[5] = fmaf(w, hi[u].y, acc[5]);
        acc[6] = fmaf(w, hi[u].z, acc[6]); acc[7] = fmaf(w, hi[u].w, acc[7]);
      }
    }
    for (; s < nsplit; ++s) {
      const float* ps = base + s * sstride;
      const float w = exp2_fast(ps[128] - M);
      L = fmaf(w, ps[129], L);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, ps[dc + i], acc[i]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint4 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  st16(out + (static_cast<int64_t>(row) * 64 + h) * 128 + dc, v);
  if (lse != nullptr && dc == 0)
    lse[static_cast<int64_t>(row) * 64 + h] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

bool tuned(csa_dtype_t dt, int H, int D) { return dt == CSA_BF16 && H == 64 && D == 128; }

int split_len(bool hca) { return hca ? kHcaSplit : kCsaSplit; }

template <typename T, int D, bool HCA>
void launch_generic(const AttendArgs& a, float scale_log2, hipStream_t s) {
  hipLaunchKernelGGL((attend_generic_kernel<T, D, HCA>), dim3(a.H, a.B * a.Tq), dim3(kGenThreads),
                     0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.kc),
                     static_cast<const T*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                     a.n_entries, a.Tq, a.H, a.N_max, a.m, scale_log2, static_cast<T*>(a.out),
                     a.lse);
}

template <typename T, bool HCA>
void launch_generic_d(const AttendArgs& a, float scale_log2, hipStream_t s) {
  if (a.D == 32) launch_generic<T, 32, HCA>(a, scale_log2, s);
  else if (a.D == 64) launch_generic<T, 64, HCA>(a, scale_log2, s);
  else launch_generic<T, 128, HCA>(a, scale_log2, s);
}

}  // namespace

bool attend_supported(csa_dtype_t dt, int H, int D) {
  if (dt != CSA_F32 && dt != CSA_BF16) return false;
  return H >= 1 && H <= 64 && (D == 32 || D == 64 || D == 128);
}

size_t attend_workspace_bytes(csa_dtype_t dt, bool hca, int B, int Tq, int H, int D,
                              int k_or_nmax) {
  if (!tuned(dt, H, D)) return 0;
  const int sl = split_len(hca);
  const int nsplit = (k_or_nmax + sl - 1) / sl;
  return static_cast<size_t>(B) * Tq * (nsplit < 1 ? 1 : nsplit) * 64 * kPartStride * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a, csa_dtype_t dt, bool hca, hipStream_t s) {
  const float scale_log2 = a.scale * kLog2e;
  if (!tuned(dt, a.H, a.D)) {
    if (dt == CSA_F32) {
      if (hca) launch_generic_d<float, true>(a, scale_log2, s);
      else launch_generic_d<float, false>(a, scale_log2, s);
    } else {
      if (hca) launch_generic_d<uint16_t, true>(a, scale_log2, s);
      else launch_generic_d<uint16_t, false>(a, scale_log2, s);
    }
    return hipGetLastError();
  }
  const int sl = split_len(hca);
  const int n = hca ? a.N_max : a.topk;
  int nsplit = (n + sl - 1) / sl;
  if (nsplit < 1) nsplit = 1;
  float* part = static_cast<float*>(a.ws);
  const dim3 grid(nsplit, a.B * a.Tq);
  if (hca)
    hipLaunchKernelGGL(attend_split_kernel<true>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                       a.n_entries, a.Tq, a.N_max, a.m, scale_log2, sl, nsplit, part);
  else
    hipLaunchKernelGGL(attend_split_kernel<false>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                       a.n_entries, a.Tq, a.N_max, a.m, scale_log2, sl, nsplit, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(a.B * a.Tq, 4), dim3(256), 0, s, part, nsplit,
                     static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace csa
