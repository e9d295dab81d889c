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
//     S^T[j, h] = K[j] . q[h]           (A = K rows from LDS, B = q^T in registers)
//     O^T[d, h] += V^T[d, j] P^T[j, h]  (A = V^T from LDS, B = P^T)
// With that orientation each lane owns one head column, so the online
// softmax is lane-local (plus one exchange with lane l^32) and the softmax
// probabilities leave the S accumulator already in the B-operand layout of
// the PV product.  K and V rows are staged row-major in LDS (double
// buffered); V^T is read with transposing loads.
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
    const int32_t* __restrict__ n_entries, int Tq, int H, int N_max, int m, int win,
    float scale_log2, T* __restrict__ out, float* __restrict__ lse) {
  __shared__ float qs[D];
  __shared__ float p_s[kGenThreads];
  __shared__ int j_s[kGenThreads];
  __shared__ float red[kGenThreads / 64];
  const int h = blockIdx.x, row = blockIdx.y, b = row / Tq, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const T* qh = q + (static_cast<int64_t>(row) * H + h) * D;
  for (int d = tid; d < D; d += kGenThreads) qs[d] = ldf<T>(qh + d) * scale_log2;
  const int n_ent = min(n_entries[b], N_max);
  const int nv = HCA ? visible_count(q_pos[row], m, n_entries[b], N_max) : kk;
  const int lo = HCA && win > 0 ? max(0, nv - win) : 0;   // window: the last win entries
  const int n = nv - lo;
  const T* Kb = K + b * kv_sb;
  const T* Vb = Vc + b * kv_sb;
  __syncthreads();
  float m_run = kNegInf, l_run = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < n; c0 += kGenThreads) {
    const int i = c0 + tid;
    int j = -1;
    if (i < n) {
      j = HCA ? lo + i : idx[static_cast<int64_t>(row) * kk + i];
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
constexpr int kCsaSplit = 128;     // entries of the top-k list per workgroup
constexpr int kCsaGroups = 2;      // key groups per CSA workgroup (4 waves)
constexpr int kHcaSplit = 1024;    // visible entries per workgroup
constexpr int kSwaSplit = 512;     // window entries per workgroup (HCA with a window)
constexpr int kHcaGroups = 4;      // key groups per HCA workgroup (8 waves)
// Partial of one (query, split): 66 rows of 64 32-bit words, O^T as bf16
// pairs of dims (row d / 2 holds dims d, d + 1 of the 64 heads), then the
// running maximum m and sum l in fp32.
constexpr int kPartRows = 66;
constexpr int kVPitch = 160;       // bf16 per V row in LDS (256 B + 64 B pad)
constexpr int kKPitch = 136;       // bf16 per K row in LDS (256 B + 16 B pad)
constexpr float kRescaleLog2 = 8.f; // probabilities stay below 2^8 between rescales

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_f32;

template <int KG>
struct __attribute__((aligned(16))) AttnSmem {
  uint16_t v[2][KG][32 * kVPitch];   // [buffer][key group][entry][d], row-major V tiles
  uint16_t k[2][KG][32 * kKPitch];   // [buffer][key group][entry][d], row-major K tiles
};

// Per-round loads of one thread: four 16-byte chunks of its key group's K
// tile and four of its V tile (chunk c = t128 + 128 i: tile row c / 16,
// 16-byte column c % 16), so every load instruction reads whole rows.
struct RoundRegs {
  uint4 kv[4];
  uint4 vv[4];
  uint32_t vmask;                    // bit j: tile row j holds a valid entry
};

// ea: the cache row this lane's tile row jl reads (lanes 0..31 and 32..63
// agree; 0 <= ea < N_max); a chunk's row takes it from lane (row) by a
// shuffle.  Only the loads: the validity mask is set by the caller.
__device__ __forceinline__ void issue_round(const uint16_t* __restrict__ Kb,
                                            const uint16_t* __restrict__ Vb, int64_t kv_sn, int ea,
                                            int t128, RoundRegs& rr) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int pair = t128 + 128 * it;
    const int vr = pair >> 4, ch = pair & 15;
    const int64_t off = static_cast<int64_t>(__shfl(ea, vr, 64)) * kv_sn + 8 * ch;
    rr.kv[it] = ld16(Kb + off);
    rr.vv[it] = ld16(Vb + off);
  }
}
// The same for rows base + r of tile row r, clamped into the cache: no
// cross-lane step (its LDS wait would also wait for scalar loads in flight).
__device__ __forceinline__ void issue_round_rows(const uint16_t* __restrict__ Kb,
                                                 const uint16_t* __restrict__ Vb, int64_t kv_sn,
                                                 int base, int N_max, int t128, RoundRegs& rr) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int pair = t128 + 128 * it;
    const int vr = pair >> 4, ch = pair & 15;
    const int64_t off = static_cast<int64_t>(min(base + vr, N_max - 1)) * kv_sn + 8 * ch;
    rr.kv[it] = ld16(Kb + off);
    rr.vv[it] = ld16(Vb + off);
  }
}
// ej: this lane's entry for tile row jl, -1 if none.  Every load is issued:
// a row without an entry reads row 0 (in bounds, as N_max is at least 1);
// its V chunk is zeroed when it is staged (probability 0 times a non-finite
// value would not be 0) and its K chunk only feeds a score that the mask
// drops.  Branch-free loads whose values are first used at staging keep the
// compiler's count of loads in flight exact, so that waiting for one round
// never waits for the round after it.
__device__ __forceinline__ void load_round(const uint16_t* __restrict__ Kb,
                                           const uint16_t* __restrict__ Vb, int64_t kv_sn, int ej,
                                           int t128, RoundRegs& rr) {
  rr.vmask = static_cast<uint32_t>(__ballot(ej >= 0));
  issue_round(Kb, Vb, kv_sn, ej < 0 ? 0 : ej, t128, rr);
}

// One key group of the workgroup processes one 32-entry tile per round:
//   stage_round: K and V rows -> LDS (row-major, 16-byte writes);
//   compute_round: barrier,
//   S^T = K q^T (8 MFMA 32x32x16, K rows read back in the A-operand layout),
//   online softmax per lane (each lane owns one head column),
//   O^T += V^T P^T with V^T read from LDS by transposing loads
//   (ds_read_b64_tr_b16) and P^T straight from the S accumulator.
__device__ __forceinline__ void stage_round(const RoundRegs& rr, lds_u16* vt, lds_u16* kt,
                                            int t128) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int pair = t128 + 128 * it;
    const int vr = pair >> 4, ch = pair & 15;
    const uint4 x = rr.kv[it];
    *(lds_u32x4*)(kt + vr * kKPitch + 8 * ch) = u32x4{x.x, x.y, x.z, x.w};
    const uint4 y = rr.vv[it];
    const u32x4 yv = ((rr.vmask >> vr) & 1u) ? u32x4{y.x, y.y, y.z, y.w} : u32x4{0, 0, 0, 0};
    *(lds_u32x4*)(vt + vr * kVPitch + 8 * ch) = yv;
  }
}

__device__ __forceinline__ void compute_round(uint32_t vmask, bool active, const lds_u16* vt,
                                              const lds_u16* kt, int jl, int g,
                                              const bf16x8_t (&bq)[8], float scale_log2,
                                              float& m_run, float& l_run, f32x16_t (&o)[4]) {
  __syncthreads();
  if (!active) return;
  f32x16_t sacc = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 w = *(const lds_u32x4*)(kt + jl * kKPitch + 16 * s + 8 * g);
    bf16x8_t a;
    __builtin_memcpy(&a, &w, 16);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], sacc, 0, 0, 0);
  }
  float x[16];
  float tmax = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = 8 * (i >> 2) + 4 * g + (i & 3);
    x[i] = ((vmask >> j) & 1u) ? sacc[i] * scale_log2 : kNegInf;
    tmax = fmaxf(tmax, x[i]);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  // Lazy rescaling: the reference maximum m_run only moves when the tile's
  // maximum exceeds it by more than kRescaleLog2, so probabilities stay
  // below 2^kRescaleLog2 and O is rescaled only when some lane moved.
  float alpha = 1.f;
  if (tmax > m_run + kRescaleLog2) {
    alpha = exp2_fast(m_run - tmax);            // 0 when m_run is -inf
    m_run = tmax;
  }
  uint32_t pb[8];
  float psum = 0.f;
  if (m_run != kNegInf) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      pb[i >> 1] = pack_bf16x2(exp2_fast(x[i] - m_run), exp2_fast(x[i + 1] - m_run));
      psum += __uint_as_float(pb[i >> 1] << 16) + __uint_as_float(pb[i >> 1] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = 0;
  }
  l_run = l_run * alpha + psum;
  if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
  }
  // A operand lane l: row d = 32 dt + l % 32, k-slots e -> entries
  // 16 s2 + 8 (e / 4) + 4 g + e % 4 (the order of the S accumulator rows).
  // Transposing load, per 16-lane group: source lane 4r + a addresses entry
  // row jb + r at column dbase + 4a; output lane i gets column dbase + i.
  const int lg = jl >> 4, li = jl & 15;
  const int r4 = li >> 2, a4 = li & 3;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    bf16x8_t bp;
    __builtin_memcpy(&bp, &pb[4 * s2], 16);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dbase = 32 * dt + 16 * lg;
      const int jb = 16 * s2 + 4 * g;
      const lds_u16* p0 = vt + (jb + r4) * kVPitch + dbase + 4 * a4;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 8 * kVPitch));
      bf16x8_t a;
      __builtin_memcpy(&a, &lo, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[dt], 0, 0, 0);
    }
  }
}

// ---- merge of the split partials inside the split kernel
// The splits of a row meet at a barrier in global memory: each workgroup,
// once its partial is stored (device-scope stores, completed before it
// arrives), adds one to the row's arrival counter and waits until every
// split has arrived; then split s merges its own slice of the output dims
// over all splits, in split order (the result does not depend on which
// workgroup finishes first).  Counters: one 128-byte line per query row at
// the front of the workspace (separate lines keep the rows' atomics apart),
// holding the row's arrivals, departures and a count of waits that gave up;
// zero before the first call, and every call leaves them zero (the last
// workgroup of a row to depart, after its merge, resets the row's two
// counters).
// The wait is bounded so that a kernel always ends.  The splits of a row are
// consecutive workgroups and dispatch follows workgroup order, so a waiting
// workgroup only ever waits for workgroups that are already running.
constexpr int kSpinLimit = 1 << 22;               // about 0.1 s of polling
constexpr int kSyncStride = 32;                   // int32 words per row's counters

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void row_barrier(int32_t* sync, int row, int n) {
  __builtin_amdgcn_s_waitcnt(0);                  // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* arrive = sync + kSyncStride * row;     // one 128-byte line per row
    __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n; ++it) {
      if (it == kSpinLimit) {
        __hip_atomic_fetch_add(arrive + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}
// Departure, issued by thread 0 right after the barrier (no barrier follows
// it, so its round trip overlaps the merge) and checked after the merge: the
// row's last workgroup to depart resets the two counters.
__device__ __forceinline__ int row_depart_issue(int32_t* sync, int row) {
  return threadIdx.x == 0
             ? __hip_atomic_fetch_add(sync + kSyncStride * row + 1, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)
             : 0;
}
__device__ __forceinline__ void row_depart_finish(int32_t* sync, int row, int n, int departed) {
  if (threadIdx.x == 0 && departed == n - 1) {
    int32_t* arrive = sync + kSyncStride * row;
    __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(arrive + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Split s of nsplit merges output dims [d0, d1), d0 = s * Ld, Ld = ceil(128 /
// nsplit) rounded up to a multiple of 4.  Thread (h, grp) owns dims
// db .. db + 3 of head h for db = d0 + 4 grp, d0 + 4 (grp + NT / 64), ...:
// every load is a coalesced 64-word row of a partial (two bf16 dims per
// word, or m or l).  Splits are taken in groups of eight, every load of a
// group issued before its arithmetic, and the running maximum rescales what
// is already summed.
template <int NT>
__device__ __forceinline__ void merge_splits(const float* __restrict__ prow, int nsplit, int split,
                                             uint16_t* __restrict__ orow, float* __restrict__ lrow) {
  constexpr int NG = NT / 64;
  constexpr int U = 8;
  const int h = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int per = (128 + nsplit - 1) / nsplit;
  const int Ld = (per + 3) & ~3;
  const int d0 = split * Ld, d1 = min(128, d0 + Ld);
  const int64_t sstride = static_cast<int64_t>(kPartRows) * 64;
  for (int db = d0 + 4 * grp; db < d1; db += 4 * NG) {
    float M = kNegInf, L = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += U) {
      float v[U][4], ms[U], ls[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = s0 + u < nsplit;
        const float* ps = prow + static_cast<int64_t>(ok ? s0 + u : s0) * sstride + h;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t w = __float_as_uint(ld_coherent(ps + (db / 2 + i) * 64));
          v[u][2 * i] = __uint_as_float(w << 16);
          v[u][2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        }
        const float mu = ld_coherent(ps + 64 * 64);
        ms[u] = ok ? mu : kNegInf;
        ls[u] = ld_coherent(ps + 65 * 64);
      }
      float mg = M;
#pragma unroll
      for (int u = 0; u < U; ++u) mg = fmaxf(mg, ms[u]);
      if (mg == kNegInf) continue;
      const float a = M == kNegInf ? 0.f : exp2_fast(M - mg);
      L *= a;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= a;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = ms[u] == kNegInf ? 0.f : exp2_fast(ms[u] - mg);
        L = fmaf(wu, ls[u], L);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wu, v[u][i], acc[i]);
      }
      M = mg;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint2 w2;
    w2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    w2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(orow + h * 128 + db) = w2;
    if (lrow != nullptr && db == 0) lrow[h] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
  }
}

// One workgroup per (split, query row); 2 KG waves = KG key groups x 2 head
// halves.  Key group kg takes tiles KG r + kg in round r.  Round r is staged
// into LDS and its registers are reloaded with round r + 2 before it
// computes, so two rounds of K/V loads are in flight during the compute; CSA
// entry indices are read two rounds ahead of their loads.  CSA runs 2 key groups (two workgroups per
// compute unit), HCA 4 (one workgroup of 8 waves per compute unit, so that a
// split covers twice the entries for the same loads in flight and the
// partials to merge are halved).  Output: the split's unnormalised O^T,
// running maximum m and sum l (base-2 logits) in d-major rows, written with
// coalesced stores.
// Entry sources: the entry index at position p of a query row's list.
struct GlobalIdxSrc {              // CSA: the caller's top-k list in global memory
  const int32_t* __restrict__ irow;
  int kk;
  __device__ __forceinline__ int raw(int p) const { return irow[min(p, kk - 1)]; }
};
template <bool HCA, int KG, bool WIN, typename Src>
__device__ __forceinline__ void split_attention(
    AttnSmem<KG>& sm, const Src& src, int split, int row, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vc, int64_t kv_sb, int64_t kv_sn,
    int kk, int qp, int ne, int Tq, int N_max, int m, int win, float scale_log2, int split_len,
    int nsplit, float* __restrict__ part, int32_t* __restrict__ sync, int rows,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = wave & 1, kg = wave >> 1;
  const int jl = lane & 31, g = lane >> 5;
  const int t128 = hh * 64 + lane;
  const int h = 32 * hh + jl;        // this lane's head (S^T / O^T column)
  const int s0 = split * split_len;
  const uint16_t* Kb = K + b * kv_sb;
  const uint16_t* Vb = Vc + b * kv_sb;

  // Loads that need no scalar value from memory go out first: q, then the
  // first two rounds' index-list entries (CSA) or, without a window, their
  // cache rows (HCA: a position is its entry, so the rows are known; rows
  // clamped into the cache, validity applied once q_pos and n_entries are
  // in).  The scheduling barrier keeps the loads of those two values, and
  // every wait for them, behind these loads.
  // B operand: q^T for this wave's 32 heads, 8 k-steps; dims 16s + 8g + e
  const uint16_t* qrow = q + static_cast<int64_t>(row) * 64 * 128;
  constexpr int kNT = 128 * KG;
  constexpr int kQC = 64 * 128 / 8 / kNT;          // 16-byte chunks of q per thread
  constexpr int kQPitch = 136;                     // bf16 per head row in LDS (padded)
  static_assert(64 * kQPitch * 2 <= sizeof(sm.v[1]), "q staging area");
  uint4 qc[kQC];
#pragma unroll
  for (int i = 0; i < kQC; ++i) qc[i] = ld16(qrow + 8 * (tid + kNT * i));
  // Two register sets, rounds taken in pairs (an odd count ends with an
  // empty round).  Loads, including those of rounds past the end (no
  // entries), are issued on every path, with no branch around them: the
  // compiler then counts the loads in flight exactly and waiting for one
  // round never waits for a later one.
  RoundRegs ra, rb;
  const int p0 = s0 + 32 * kg + jl, p1 = p0 + 32 * KG;   // tile row jl of rounds 0 and 1
  int ea = 0, eb = 0;
  if constexpr (HCA && !WIN) {
    issue_round_rows(Kb, Vb, kv_sn, s0 + 32 * kg, N_max, t128, ra);
    issue_round_rows(Kb, Vb, kv_sn, s0 + 32 * (KG + kg), N_max, t128, rb);
  } else if constexpr (!HCA) {
    ea = src.raw(p0);
    eb = src.raw(p1);
  }
  __builtin_amdgcn_sched_barrier(0);

  const int n_ent = min(ne, N_max);
  const int nv = HCA ? visible_count(qp, m, ne, N_max) : kk;
  // HCA with a window: positions count from lo, the first of the last win
  // visible entries (splits laid over the window, not the whole cache)
  const int lo = HCA && WIN ? max(0, nv - win) : 0;
  const int n = nv - lo;
  const int s_end = min(n, s0 + split_len);
  const int ntiles = s_end > s0 ? (s_end - s0 + 31) / 32 : 0;
  const int nrounds = (ntiles + KG - 1) / KG;

  f32x16_t o[4] = {};
  float m_run = kNegInf, l_run = 0.f;
  lds_u16* const vt0 = (lds_u16*)&sm.v[0][kg][0];
  lds_u16* const kt0 = (lds_u16*)&sm.k[0][kg][0];
  lds_u16* const vt1 = (lds_u16*)&sm.v[1][kg][0];
  lds_u16* const kt1 = (lds_u16*)&sm.k[1][kg][0];

  // Entry of tile row jl in round rr: entry_raw reads the index list without
  // a condition (position clamped into the list), entry_ok validates it when
  // the round's loads are issued (-1: none).  A load under a branch, or a
  // check right after it, would make the compiler wait for every load in
  // flight, the next round's included.
  auto entry_raw = [&](int rr) -> int {
    const int p_ = s0 + 32 * (KG * rr + kg) + jl;
    return HCA ? lo + p_ : src.raw(p_);
  };
  auto entry_ok = [&](int rr, int e) -> int {
    const int t_ = KG * rr + kg, p_ = s0 + 32 * t_ + jl;
    // bitwise, not short-circuit: no branch that the index load could sink into
    const bool ok = (t_ < ntiles) & (p_ < s_end) & (e >= 0) & (e < n_ent);
    return ok ? e : -1;
  };

  if constexpr (HCA && !WIN) {
    ra.vmask = static_cast<uint32_t>(__ballot(entry_ok(0, p0) >= 0));
    rb.vmask = static_cast<uint32_t>(__ballot(entry_ok(1, p1) >= 0));
  } else {
    if constexpr (HCA) {
      ea = lo + p0;
      eb = lo + p1;
    }
    load_round(Kb, Vb, kv_sn, entry_ok(0, ea), t128, ra);
    load_round(Kb, Vb, kv_sn, entry_ok(1, eb), t128, rb);
  }
  ea = entry_raw(2);
  eb = entry_raw(3);
  // q read once per workgroup and shared through the second tile buffer
  // (not written until round 1 is staged, after the first barrier below)
  lds_u16* qs = (lds_u16*)&sm.v[1][0][0];
#pragma unroll
  for (int i = 0; i < kQC; ++i) {
    const int c = tid + kNT * i;                   // chunk c: head c / 16, dims 8 (c % 16)
    *(lds_u32x4*)(qs + (c >> 4) * kQPitch + 8 * (c & 15)) = u32x4{qc[i].x, qc[i].y, qc[i].z, qc[i].w};
  }
  __syncthreads();
  bf16x8_t bq[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 w = *(const lds_u32x4*)(qs + h * kQPitch + 16 * s + 8 * g);
    __builtin_memcpy(&bq[s], &w, 16);
  }
  // q resident before the loop (rounds 0 and 1 stay in flight), so that no
  // wait inside the loop is computed as if it were still loading; the loop
  // runs at least once so that the loads above stay ahead of this point
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(bq[s]));
  int r = 0;
  do {
    stage_round(ra, vt0, kt0, t128);
    const uint32_t vma = ra.vmask;
    load_round(Kb, Vb, kv_sn, entry_ok(r + 2, ea), t128, ra);
    ea = entry_raw(r + 4);
    compute_round(vma, KG * r + kg < ntiles, vt0, kt0, jl, g, bq, scale_log2, m_run, l_run, o);
    stage_round(rb, vt1, kt1, t128);
    const uint32_t vmb = rb.vmask;
    load_round(Kb, Vb, kv_sn, entry_ok(r + 3, eb), t128, rb);
    eb = entry_raw(r + 5);
    compute_round(vmb, KG * (r + 1) + kg < ntiles, vt1, kt1, jl, g, bq, scale_log2, m_run, l_run,
                  o);
    r += 2;
  } while (r < nrounds);

  // Merge the KG key groups of each head half through LDS (reuses the tile
  // buffers): key group kg finishes the d-tiles dt with dt % KG == kg and
  // hands the others its accumulators, running maximum and sum.
  l_run = l_run + __shfl_xor(l_run, 32, 64);
  __syncthreads();
  constexpr int kX = 67;                           // floats per lane: 64 + m + l, odd pitch
  static_assert(KG * 2 * 64 * kX * sizeof(float) <= sizeof(AttnSmem<KG>), "merge area");
  lds_f32* xo = (lds_f32*)&sm.v[0][0][0];          // [kg][hh][lane][kX]
  {
    lds_f32* dst = xo + ((kg * 2 + hh) * 64 + lane) * kX;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      if (dt % KG != kg)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[16 * dt + i] = o[dt][i];
    dst[64] = m_run;
    dst[65] = l_run;
  }
  __syncthreads();
  {
    float mk[KG], lk[KG], ak[KG];
    float M = kNegInf;
#pragma unroll
    for (int k2 = 0; k2 < KG; ++k2) {
      const lds_f32* src = xo + ((k2 * 2 + hh) * 64 + lane) * kX;
      mk[k2] = k2 == kg ? m_run : src[64];
      lk[k2] = k2 == kg ? l_run : src[65];
      M = fmaxf(M, mk[k2]);
    }
    float L = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < KG; ++k2) {
      ak[k2] = M == kNegInf ? 0.f : exp2_fast(mk[k2] - M);
      L = fmaf(ak[k2], lk[k2], L);
    }
    // this key group's d-tiles, merged over the key groups
    float vals[4][16];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      if (dt % KG != kg) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < KG; ++k2) {
          const float x = k2 == kg ? o[dt][i] : xo[((k2 * 2 + hh) * 64 + lane) * kX + 16 * dt + i];
          v = fmaf(ak[k2], x, v);
        }
        vals[dt][i] = v;
      }
    }
    if (nsplit == 1) {
      // the only split: normalise and write the output directly
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* orow = out + (static_cast<int64_t>(row) * 64 + h) * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        if (dt % KG != kg) continue;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w2;
          w2.x = pack_bf16x2(vals[dt][4 * q4] * inv, vals[dt][4 * q4 + 1] * inv);
          w2.y = pack_bf16x2(vals[dt][4 * q4 + 2] * inv, vals[dt][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4 + 4 * g) = w2;
        }
      }
      if (lse != nullptr && kg == 0 && g == 0)
        lse[static_cast<int64_t>(row) * 64 + h] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
      return;
    }
    // partial of this split, stored coherently at device scope (read by the
    // other workgroups of the row): O^T d-major as bf16 pairs (rounded to
    // nearest even: the merge's output is bf16 too, and halving the bytes
    // every split stores and every split reads back shortens the row's
    // tail), then m and l in fp32
    float* pr = part + (static_cast<int64_t>(row) * nsplit + split) * kPartRows * 64;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      if (dt % KG != kg) continue;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int d = 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3);   // even
        st_coherent(pr + (d / 2) * 64 + h, __uint_as_float(pack_bf16x2(vals[dt][i], vals[dt][i + 1])));
      }
    }
    if (kg == 0 && g == 0) {
      st_coherent(pr + 64 * 64 + h, M);
      st_coherent(pr + 65 * 64 + h, L);
    }
  }
  row_barrier(sync, row, nsplit);
  const int departed = row_depart_issue(sync, row);
  merge_splits<128 * KG>(part + static_cast<int64_t>(row) * nsplit * kPartRows * 64, nsplit, split,
                         out + static_cast<int64_t>(row) * 64 * 128,
                         lse != nullptr ? lse + static_cast<int64_t>(row) * 64 : nullptr);
  row_depart_finish(sync, row, nsplit, departed);
}

// One workgroup per (split, query row): CSA over the caller's top-k lists, or
// HCA / a sliding window over the visible entries.
template <bool HCA, int KG, bool WIN>
__global__ __launch_bounds__(128 * KG, 4 / KG) void attend_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vc, int64_t kv_sb, int64_t kv_sn, const int32_t* __restrict__ idx,
    int kk, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq,
    int N_max, int m, int win, float scale_log2, int split_len, int nsplit,
    float* __restrict__ part, int32_t* __restrict__ sync, int rows, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ AttnSmem<KG> sm;
  const int row = blockIdx.y;
  // Every argument goes into registers before its first use, so that the
  // argument loads go out together (one round trip instead of one per first
  // use); then the two values read from memory.
  asm volatile("" ::"s"(q), "s"(K), "s"(Vc), "s"(kv_sb), "s"(kv_sn), "s"(idx), "s"(kk), "s"(q_pos),
               "s"(n_entries), "s"(Tq), "s"(N_max), "s"(m), "s"(win), "s"(scale_log2),
               "s"(split_len), "s"(nsplit), "s"(part), "s"(sync), "s"(rows), "s"(out), "s"(lse));
  const int qp = HCA ? q_pos[row] : 0;
  const int ne = n_entries[row / Tq];
  const GlobalIdxSrc src{HCA ? idx : idx + static_cast<int64_t>(row) * kk, kk};
  split_attention<HCA, KG, WIN>(sm, src, blockIdx.x, row, q, K, Vc, kv_sb, kv_sn, kk, qp, ne, Tq,
                                N_max, m, win, scale_log2, split_len, nsplit, part, sync, rows,
                                out, lse);
}



// ---------------------------------------------------------------- merging two branches
// Attention results over disjoint key sets (a sliding window and the
// compressed entries, say), each as (o, lse) under the same softmax scale,
// give the attention over the union: lse = log(e^lse_a + e^lse_b) and
// o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.  One thread per 8 output
// dims of one (row, head); elementwise, so out may be o_a or o_b itself.
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const T* __restrict__ oa, const float* __restrict__ la,
                                                    const T* __restrict__ ob, const float* __restrict__ lb,
                                                    T* out, float* __restrict__ lse_out, int64_t rows_h,
                                                    int D) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per = D / 8;
  if (i >= rows_h * per) return;
  const int64_t rh = i / per;
  const int64_t off = rh * D + (i - rh * per) * 8;
  const float a = la[rh], b = lb[rh];
  const float mx = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, l = kNegInf;
  if (mx != kNegInf) {
    const float ea = a == kNegInf ? 0.f : expf(a - mx);
    const float eb = b == kNegInf ? 0.f : expf(b - mx);
    const float sum = ea + eb;
    wa = ea / sum;
    wb = eb / sum;
    l = mx + logf(sum);
  }
  float x[8], y[8];
  if constexpr (sizeof(T) == 2) {
    const uint4 u = ld16(oa + off), v = ld16(ob + off);
    const uint32_t uu[4] = {u.x, u.y, u.z, u.w}, vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[2 * c] = __uint_as_float(uu[c] << 16);
      x[2 * c + 1] = __uint_as_float(uu[c] & 0xffff0000u);
      y[2 * c] = __uint_as_float(vv[c] << 16);
      y[2 * c + 1] = __uint_as_float(vv[c] & 0xffff0000u);
    }
    uint4 r;
    r.x = pack_bf16x2(wa * x[0] + wb * y[0], wa * x[1] + wb * y[1]);
    r.y = pack_bf16x2(wa * x[2] + wb * y[2], wa * x[3] + wb * y[3]);
    r.z = pack_bf16x2(wa * x[4] + wb * y[4], wa * x[5] + wb * y[5]);
    r.w = pack_bf16x2(wa * x[6] + wb * y[6], wa * x[7] + wb * y[7]);
    st16(out + off, r);
  } else {
#pragma unroll
    for (int c = 0; c < 8; c += 4) {
      const float4 u = *reinterpret_cast<const float4*>(oa + off + c);
      const float4 v = *reinterpret_cast<const float4*>(ob + off + c);
      *reinterpret_cast<float4*>(out + off + c) =
          make_float4(wa * u.x + wb * v.x, wa * u.y + wb * v.y, wa * u.z + wb * v.z,
                      wa * u.w + wb * v.w);
    }
  }
  if (lse_out != nullptr && i - rh * per == 0) lse_out[rh] = l;
}

bool tuned(csa_dtype_t dt, int H, int D) { return dt == CSA_BF16 && H == 64 && D == 128; }

// Entries per workgroup.  A window caps the entries of a row, so windowed
// calls take shorter splits to fill the chip at decode batch sizes; the
// length depends on the call's mode only, never on its batch, so a row's
// result does not change with the batch it is computed in.
int split_len(bool hca, int win) { return hca ? (win > 0 ? kSwaSplit : kHcaSplit) : kCsaSplit; }

template <typename T, int D, bool HCA>
void launch_generic(const AttendArgs& a, float scale_log2, hipStream_t s) {
  hipLaunchKernelGGL((attend_generic_kernel<T, D, HCA>), dim3(a.H, a.B * a.Tq), dim3(kGenThreads),
                     0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.kc),
                     static_cast<const T*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                     a.n_entries, a.Tq, a.H, a.N_max, a.m, a.win, scale_log2,
                     static_cast<T*>(a.out), a.lse);
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

// Workspace of the tuned path: a fixed block of merge counters at the front
// (one 128-byte line per row for up to kAttendMaxRows rows), then the split
// partials.  The block has the same size and place for every
// call, and calls leave it zero, so a workspace zero-filled once serves calls
// of any shape.
size_t attend_sync_block_bytes(int rows) {
  return (static_cast<size_t>(kSyncStride) * rows * sizeof(int32_t) + 255) / 256 * 256;
}

size_t attend_part_bytes(csa_dtype_t dt, bool hca, int B, int Tq, int H, int D, int k_or_nmax,
                         int win) {
  if (!tuned(dt, H, D)) return 0;
  const int sl = split_len(hca, win);
  const int nsplit = (k_or_nmax + sl - 1) / sl;
  return static_cast<size_t>(B) * Tq * (nsplit < 1 ? 1 : nsplit) * kPartRows * 64 * sizeof(float);
}

size_t attend_workspace_bytes(csa_dtype_t dt, bool hca, int B, int Tq, int H, int D,
                              int k_or_nmax, int win) {
  if (!tuned(dt, H, D)) return 0;
  return attend_sync_block_bytes(kAttendMaxRows) +
         attend_part_bytes(dt, hca, B, Tq, H, D, k_or_nmax, win);
}

bool attend_rows_ok(int B, int Tq) {
  return static_cast<long long>(B) * Tq <= kAttendMaxRows;
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
  const int sl = split_len(hca, a.win);
  const int n = hca ? (a.win > 0 ? min(a.win, a.N_max) : a.N_max) : a.topk;
  int nsplit = (n + sl - 1) / sl;
  if (nsplit < 1) nsplit = 1;
  const int rows = a.B * a.Tq;
  int32_t* sync = a.sync != nullptr ? a.sync : static_cast<int32_t*>(a.ws);
  float* part = a.part != nullptr ? a.part
                                  : reinterpret_cast<float*>(static_cast<char*>(a.ws) +
                                                             attend_sync_block_bytes(kAttendMaxRows));
  uint16_t* out = static_cast<uint16_t*>(a.out);
  const dim3 grid(nsplit, rows);
  if (hca && a.win > 0)
    hipLaunchKernelGGL((attend_split_kernel<true, kHcaGroups, true>), grid, dim3(128 * kHcaGroups),
                       0, s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                       a.n_entries, a.Tq, a.N_max, a.m, a.win, scale_log2, sl, nsplit, part, sync, rows,
                       out, a.lse);
  else if (hca)
    hipLaunchKernelGGL((attend_split_kernel<true, kHcaGroups, false>), grid, dim3(128 * kHcaGroups),
                       0, s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                       a.n_entries, a.Tq, a.N_max, a.m, a.win, scale_log2, sl, nsplit, part, sync, rows,
                       out, a.lse);
  else
    hipLaunchKernelGGL((attend_split_kernel<false, kCsaGroups, false>), grid, dim3(128 * kCsaGroups), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.kv_sb, a.kv_sn, a.idx, a.topk, a.q_pos,
                       a.n_entries, a.Tq, a.N_max, a.m, a.win, scale_log2, sl, nsplit, part, sync, rows,
                       out, a.lse);
  return hipGetLastError();
}


hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb,
                        csa_dtype_t dt, int rows, int H, int D, void* out, float* lse_out,
                        hipStream_t s) {
  const int64_t rows_h = static_cast<int64_t>(rows) * H;
  const int64_t threads = rows_h * (D / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dt == CSA_F32)
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(oa),
                       la, static_cast<const float*>(ob), lb, static_cast<float*>(out), lse_out,
                       rows_h, D);
  else
    hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(oa), la, static_cast<const uint16_t*>(ob), lb,
                       static_cast<uint16_t*>(out), lse_out, rows_h, D);
  return hipGetLastError();
}

}  // namespace csa
