// Lightning Indexer scores ("DeepSeek V4 技术解读", §2.1: per query token,
// 64 indexer heads of dim 128 score the compressed entries; §5: the indexer
// QK path may run in FP4 E2M1 dequantised to FP8 E4M3).
//
//   s(t, j) = sum_h w[t, h] * max(0, q_I[t, h] . k_I[j])   for j < V(t)
//
// Decode is HBM-bound: every key row (256 B in bf16) is read once and costs
// 64 x 128 MACs, 64 FLOP/B, above the fp32 VALU ridge, so the dot products
// run on MFMA with the 64 heads of one query as the M dimension and keys as
// N.  In the 32x32 accumulator layout a lane holds one key and 16 heads, so
// ReLU, head weight and the head sum stay in registers, followed by a single
// exchange between lanes l and l^32.  K rows are loaded straight into the B
// operand (lane l%32 = key row, 16 contiguous bytes per lane per k-step),
// two tiles ahead of the MFMAs.
//
// The MFMA k-slot order does not matter for a dot product as long as A and
// B use the same one, so slot (lane/32, e) of k-step s holds dimension
// 16*s + 8*(lane/32) + e for both operands.
#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

// ---------------------------------------------------------------- generic (VALU)
template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T, int D>
__global__ __launch_bounds__(256) void score_generic_kernel(
    const T* __restrict__ q, const float* __restrict__ w, const T* __restrict__ k, int64_t k_sb,
    int64_t k_sn, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int Tq,
    int N_max, int m, int H, float* __restrict__ scores, int64_t s_rs) {
  __shared__ float qs[64 * D];
  __shared__ float ws[64];
  const int row = blockIdx.y, b = row / Tq, tid = threadIdx.x;
  const T* qrow = q + static_cast<int64_t>(row) * H * D;
  for (int i = tid; i < H * D; i += blockDim.x) qs[i] = ld_elem<T>(qrow + i);
  for (int i = tid; i < H; i += blockDim.x) ws[i] = w[static_cast<int64_t>(row) * H + i];
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + tid;
  if (j >= N_max) return;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  float* srow = scores + row * s_rs;
  if (j >= V) {
    srow[j] = kNegInf;
    return;
  }
  const T* kr = k + b * k_sb + static_cast<int64_t>(j) * k_sn;
  float kv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) kv[d] = ld_elem<T>(kr + d);
  float s = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) dot = fmaf(qs[h * D + d], kv[d], dot);
    s = fmaf(ws[h], fmaxf(dot, 0.f), s);
  }
  srow[j] = s;
}

// ---------------------------------------------------------------- selection bound
// Each wave also reports, for the scores it produced (its chunk of
// kBoundChunk keys, held as NV scores by each of 16 or 32 lanes), a value
// that c of them reach, c = bound_c_row(V, k) for the row: the c-th largest
// of the per-lane maxima (c lanes hold an entry at or above it; a little
// below the exact c-th largest, for a fraction of its cost), and the
// largest score.  Every chunk that reports a finite value holds c entries at
// or above it, and the floor(V / kBoundChunk) full chunks all do (every lane
// holds valid entries, c <= 16), so the ceil(k / c)-th largest report is at
// most the row's k-th largest score.  The top-k kernels use that bound to
// drop most entries before selecting, and the largest report as the top of
// the survivors' range.  A chunk with fewer than c lanes holding valid
// entries reports +inf (-inf as its largest when it has none); rows with no
// bound (c = 0) write nothing.
constexpr float kPosInf = __builtin_inff();

template <int NV>
__device__ float2 wave_chunk_report(const float (&vals)[NV], bool active, int c) {
  const int lane = threadIdx.x & 63;
  float lm = kNegInf;
#pragma unroll
  for (int i = 0; i < NV; ++i) lm = fmaxf(lm, vals[i]);
  if (!active) lm = kNegInf;
  float cur = kPosInf, top = kNegInf;
  for (int r = 0; r < c; ++r) {
    const float wm = wave_max(lm);
    if (r == 0) top = wm;
    if (wm == kNegInf) {
      cur = kPosInf;
      break;
    }
    const unsigned long long msk = __ballot(lm == wm);
    if (lane == __ffsll(msk) - 1) lm = kNegInf;
    cur = wm;
  }
  return make_float2(cur, top);
}

// ---------------------------------------------------------------- bf16, 64 heads x 128
constexpr int kWavesPerWg = 4;
constexpr int kTilesPerWave = 8;                  // tiles of 32 keys
constexpr int kKeysPerWave = 32 * kTilesPerWave;  // one selection chunk
constexpr int kKeysPerWg = kWavesPerWg * kKeysPerWave;
static_assert(kKeysPerWave == kBoundChunk, "one bound chunk per wave");

// Straight-line code over the wave's 8 tiles of 32 keys with a 3-deep ring of
// registers: the loads of tile t+2 are issued before the MFMAs of tile t and
// no register is copied, so two tiles (16 KB per wave) stay in flight behind
// the math; the epilogue of tile t-1 runs while the MFMAs of tile t do.  Loads are coalesced and non-temporal (instruction i of a tile
// reads key rows 4i .. 4i+3 whole, 16 lanes per row); each tile then passes
// through a wave-private LDS buffer to reach the MFMA B-operand layout (lane
// (j, g) holds dims 16s + 8g .. +7 of key j).  Rows past the visible range are
// clamped to the last visible row (in bounds, cache hits) and masked on
// output.
constexpr int kKeyPitch = 136;                    // bf16 per key row in LDS (256 B + 16 B)

template <typename SO>
__global__ __launch_bounds__(256, 2) void score_bf16_h64d128_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    int64_t k_sb, int64_t k_sn, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, SO* __restrict__ scores,
    int64_t s_rs, float2* __restrict__ chunk_rep, int n_chunks, int bound_k) {
  __shared__ __attribute__((aligned(16))) uint16_t key_lds[kWavesPerWg][32 * kKeyPitch];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[64 * kKeyPitch];
  const int row = blockIdx.y, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int jl = lane & 31, g = lane >> 5;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int chunk = blockIdx.x * kWavesPerWg + wave;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  // q_I rows (heads) of this query go to LDS and are read back per tile as
  // the A operand (the registers hold the accumulators of two tiles instead)
  const uint16_t* qrow = q + static_cast<int64_t>(row) * 64 * 128;
  u32x4_t qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qv[i] = *reinterpret_cast<const u32x4_t*>(qrow + 8 * (static_cast<int>(threadIdx.x) + 256 * i));
  const int key0 = chunk * kKeysPerWave;
  const int key_end = min(key0 + kKeysPerWave, N_max);
  const int vis_end = min(key_end, V);
  // The first two key tiles are requested before the query is staged and
  // the barrier passed, so that their latency overlaps the query's (the
  // empty asm with a memory clobber keeps the compiler from sinking them
  // below).  Every wave issues them, also one that exits below: rows are
  // clamped to [0, vis_end - 1] (row 0 when nothing is visible; N_max >= 1).
  const uint16_t* kb = k + b * k_sb + 8 * (lane & 15);
  const int lrow = lane >> 4;                     // row within each 4-row load
  const int jmax = max(vis_end - 1, 0);
  u32x4_t kt[3][8];
  auto load_tile = [&](int t, u32x4_t (&dst)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(key0 + 32 * t + 4 * i + lrow, jmax);
      dst[i] = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    }
  };
  load_tile(0, kt[0]);
  load_tile(1, kt[1]);
  asm volatile("" ::"s"(k) : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;       // 16-byte chunk: head c / 16
    *(lds_u32x4*)((lds_u16*)q_lds + (c >> 4) * kKeyPitch + 8 * (c & 15)) = qv[i];
  }
  __syncthreads();                                // the only barrier: early exits follow
  if (key0 >= N_max) return;
  SO* srow = scores + row * s_rs;
  for (int j = max(key0, V) + lane; j < key_end; j += 64) put_score(&srow[j], kNegInf);
  if (key0 >= vis_end) {
    if (chunk_rep != nullptr && lane == 0)
      chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = make_float2(kPosInf, kNegInf);
    return;
  }

  lds_u16* kl = (lds_u16*)&key_lds[wave][0];
  const lds_u16* ql = (const lds_u16*)q_lds + jl * kKeyPitch + 8 * g;
  // head weights in accumulator-row order: row = 8*(r/4) + 4*g + r%4
  const float* wrow = w + static_cast<int64_t>(row) * 64;
  float w0[16], w1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = 8 * (r >> 2) + 4 * g + (r & 3);
    w0[r] = wrow[h];
    w1[r] = wrow[32 + h];
  }

  float sc[kTilesPerWave];
  // epilogue of tile t from its accumulators: sum_h w[h] ReLU(s_h), then the
  // two lane halves (32 heads each) add up
  auto epilogue = [&](int t, const f32x16_t& c0, const f32x16_t& c1) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(w0[r], relu_f32(c0[r]), sum);
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(w1[r], relu_f32(c1[r]), sum);
    const float other = __shfl_xor(sum, 32, 64);
    const float tot = sum + other;     // commutative: both halves get the same bits
    const int j = key0 + 32 * t + jl;
    const bool ok = j < vis_end;
    if (g == 0 && ok) put_score(&srow[j], tot);
    sc[t] = ok ? tot : kNegInf;
  };
  // Iteration t: loads of tile t+2, tile t through LDS into the MFMAs, and
  // the epilogue of tile t-1 while those MFMAs run (two accumulator sets).
  // sched_barrier(0) keeps the scheduler from sinking the prefetch loads
  // below the MFMAs of the current tile (it would, to shorten live ranges).
  f32x16_t acc[2][2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    if (t + 2 < kTilesPerWave) load_tile(t + 2, kt[(t + 2) % 3]);
    __builtin_amdgcn_sched_barrier(0);
    // tile t: registers -> LDS (rows 4i + lrow) -> B operand (row jl)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(lds_u32x4*)(kl + (4 * i + lrow) * kKeyPitch + 8 * (lane & 15)) = kt[t % 3][i];
    bf16x8_t cur[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4_t x = *(const lds_u32x4*)(kl + jl * kKeyPitch + 16 * s + 8 * g);
      __builtin_memcpy(&cur[s], &x, 16);
    }
    f32x16_t (&c)[2] = acc[t & 1];
    c[0] = f32x16_t{};
    c[1] = f32x16_t{};
    __atomic_signal_fence(__ATOMIC_SEQ_CST);     // re-read the A operands from LDS
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8_t a0, a1;
      const u32x4_t x0 = *(const lds_u32x4*)(ql + 16 * s);
      const u32x4_t x1 = *(const lds_u32x4*)(ql + 32 * kKeyPitch + 16 * s);
      __builtin_memcpy(&a0, &x0, 16);
      __builtin_memcpy(&a1, &x1, 16);
      c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, cur[s], c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, cur[s], c[1], 0, 0, 0);
    }
    if (t > 0) epilogue(t - 1, acc[(t - 1) & 1][0], acc[(t - 1) & 1][1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  epilogue(kTilesPerWave - 1, acc[(kTilesPerWave - 1) & 1][0], acc[(kTilesPerWave - 1) & 1][1]);
  const int thr_c = bound_c_row(V, bound_k);
  if (chunk_rep != nullptr && thr_c > 0) {
    const float2 rep = wave_chunk_report<kTilesPerWave>(sc, g == 0, thr_c);
    if (lane == 0) chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = stored_report<SO>(rep);
  }
}

// ---------------------------------------------------------------- bf16 prefill (many queries)
// With many query tokens per sequence the score is a GEMM with the (query,
// head) pairs as rows, keys as columns and the 128 dims as the reduction,
// followed by the per-query epilogue sum_h w[h] ReLU(.).  One workgroup of
// 8 waves takes 8 queries of one sequence (one per wave: two 32-row A tiles
// of q_I held in registers) against 2048 keys.  Key tiles of 32 rows are read
// once per workgroup with coalesced loads (one 16-byte load per thread per
// tile), kept four tiles ahead in registers, staged through a triple-buffered
// LDS tile shared by the waves (one barrier per tile) and multiplied by all 8
// queries: 16 MFMA 32x32x16 per wave per 8 KB tile.  Two waves per SIMD let
// one wave's epilogue overlap the other's MFMAs.  The selection bounds are
// produced per 256-key chunk exactly as in the decode kernel.
constexpr int kPfQueries = 8;
constexpr int kPfThreads = 64 * kPfQueries;
constexpr int kPfKeys = 2048;
constexpr int kPfStages = 4;

template <typename SO>
__global__ __launch_bounds__(kPfThreads, 2) void score_prefill_bf16_h64d128_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    int64_t k_sb, int64_t k_sn, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, SO* __restrict__ scores,
    int64_t s_rs, float2* __restrict__ chunk_rep, int n_chunks, int bound_k) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  __shared__ __attribute__((aligned(16))) uint16_t tile_lds[3][32 * kKeyPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jl = lane & 31, g = lane >> 5;
  const int groups = (Tq + kPfQueries - 1) / kPfQueries;
  const int kblk = blockIdx.x, qgrp = blockIdx.y;
  const int b = qgrp / groups;
  const int t0 = (qgrp % groups) * kPfQueries;
  const int j0 = kblk * kPfKeys;
  const int j1 = min(j0 + kPfKeys, N_max);
  const int n_ent = n_entries[b];
  // visible counts of the workgroup's queries (invalid query: 0)
  int vmax = 0, vq = 0;
#pragma unroll
  for (int u = 0; u < kPfQueries; ++u) {
    const int t = t0 + u;
    const int v = t < Tq ? visible_count(q_pos[b * Tq + t], m, n_ent, N_max) : 0;
    vmax = max(vmax, v);
    if (u == wave) vq = v;
  }
  // wave-uniform values, made visibly uniform so their branches stay scalar
  vmax = __builtin_amdgcn_readfirstlane(vmax);
  vq = __builtin_amdgcn_readfirstlane(vq);
  const int rowq = __builtin_amdgcn_readfirstlane(t0 + wave < Tq ? b * Tq + t0 + wave : -1);
  const int je = min(j1, vmax);                   // keys past je are masked for all queries
  const int ntiles = __builtin_amdgcn_readfirstlane(je > j0 ? (je - j0 + 31) / 32 : 0);

  // -inf for every key this workgroup covers but does not compute
  if (rowq >= 0) {
    SO* srow = scores + rowq * s_rs;
    for (int j = j0 + 32 * ntiles + lane; j < j1; j += 64) put_score(&srow[j], kNegInf);
  }
  const uint16_t* kb = k + b * k_sb + 8 * (tid & 15);
  const int jcap = max(vmax, 1) - 1;              // clamp rows to visible ones (in bounds)
  const int lrow = tid >> 4;                      // tile row this thread loads
  // Key tile loads are issued on every path (rows clamped, so tiles past
  // the end read visible rows again): with no branch around them the
  // compiler counts the loads in flight exactly and waiting for one tile
  // never waits for the tiles behind it.
  u32x4_t ring[kPfStages];
#pragma unroll
  for (int u = 0; u < kPfStages; ++u)
    ring[u] = *reinterpret_cast<const u32x4_t*>(kb + static_cast<int64_t>(min(j0 + 32 * u + lrow, jcap)) * k_sn);

  // A operand: q_I rows of the wave's query (an invalid query reads row 0
  // and its results are never stored)
  bf16x8_t a[2][8];
  float wv[2][16];
  {
    const uint16_t* qrow = q + static_cast<int64_t>(max(rowq, 0)) * 64 * 128;
    const float* wrow = w + static_cast<int64_t>(max(rowq, 0)) * 64;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        a[hf][s2] = ld_bf16x8(qrow + (32 * hf + jl) * 128 + 16 * s2 + 8 * g);
#pragma unroll
      for (int r = 0; r < 16; ++r) wv[hf][r] = wrow[32 * hf + 8 * (r >> 2) + 4 * g + (r & 3)];
    }
  }
  const int cq = __builtin_amdgcn_readfirstlane(chunk_rep != nullptr && rowq >= 0 ? bound_c_row(vq, bound_k) : 0);
  float sc[kTilesPerWave];
  lds_u16* const st_ptr0 = (lds_u16*)&tile_lds[0][0] + lrow * kKeyPitch + 8 * (tid & 15);
  const lds_u16* const ld_ptr0 = (const lds_u16*)&tile_lds[0][0] + jl * kKeyPitch + 8 * g;
  constexpr int kBufElems = 32 * kKeyPitch;
  // MFMAs of one key tile from LDS buffer `buf` into acc
  auto mfma_tile = [&](int buf, f32x16_t (&acc)[2]) {
    const lds_u16* src = ld_ptr0 + buf * kBufElems;
    acc[0] = f32x16_t{};
    acc[1] = f32x16_t{};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const u32x4_t x = *(const lds_u32x4*)(src + 16 * s2);
      bf16x8_t bb;
      __builtin_memcpy(&bb, &x, 16);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s2], bb, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s2], bb, acc[1], 0, 0, 0);
    }
  };
  auto load_tile = [&](int t) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(kb + static_cast<int64_t>(min(j0 + 32 * t + lrow, jcap)) * k_sn);
  };
  f32x16_t acc[2][2];

  // Software pipeline, one barrier per tile.  Iteration tt: stage tile tt+2
  // into LDS buffer (tt+2)%3, load tile tt+6 into the freed register slot,
  // issue the MFMAs of tile tt+1, then the epilogue of tile tt (whose MFMAs
  // were issued one iteration earlier) while they run.
  *(lds_u32x4*)st_ptr0 = ring[0];
  *(lds_u32x4*)(st_ptr0 + kBufElems) = ring[1];
  ring[0] = load_tile(4);
  ring[1] = load_tile(5);
  __syncthreads();
  if (ntiles > 0) mfma_tile(0, acc[0]);
  for (int t = 0; t < ntiles; t += kTilesPerWave) {   // one 256-key chunk per pass
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
      const int tt = t + u;
      if (tt < ntiles) {
        __syncthreads();
        if (tt + 2 < ntiles) *(lds_u32x4*)(st_ptr0 + ((tt + 2) % 3) * kBufElems) = ring[(u + 2) % kPfStages];
      }
      ring[(u + 2) % kPfStages] = load_tile(tt + 6);
      if (tt < ntiles) {
        // the MFMAs of tile tt+1 (past the last tile they read a stale
        // buffer and are discarded: unconditional, so they share one
        // scheduling region with the epilogue of tile tt) interleaved with
        // that epilogue's VALU work
        mfma_tile((tt + 1) % 3, acc[(u + 1) & 1]);
        const f32x16_t (&c)[2] = acc[u & 1];
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum = fmaf(wv[0][r], relu_f32(c[0][r]), sum);
#pragma unroll
        for (int r = 0; r < 16; ++r) sum = fmaf(wv[1][r], relu_f32(c[1][r]), sum);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // B-operand LDS reads
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); // four VALU
        }
        const float tot = sum + __shfl_xor(sum, 32, 64);
        const int j = j0 + 32 * tt + jl;
        const bool ok = j < vq;
        if (g == 0 && rowq >= 0 && j < j1) put_score(&scores[rowq * s_rs + j], ok ? tot : kNegInf);
        sc[u] = ok ? tot : kNegInf;
        // after each 256-key chunk (or the last computed tile): its bound
        if (cq > 0 && (u == kTilesPerWave - 1 || tt == ntiles - 1)) {
#pragma unroll
          for (int v = u + 1; v < kTilesPerWave; ++v) sc[v] = kNegInf;
          const float2 rep = wave_chunk_report<kTilesPerWave>(sc, g == 0, cq);
          if (lane == 0)
            chunk_rep[static_cast<int64_t>(rowq) * n_chunks + (j0 + 32 * tt) / kBoundChunk] = stored_report<SO>(rep);
        }
      }
    }
  }
  // chunks with no computed key: no bound
  if (cq > 0 && lane == 0) {
    for (int ch = (j0 + 32 * ntiles + kBoundChunk - 1) / kBoundChunk; ch * kBoundChunk < j1; ++ch)
      chunk_rep[static_cast<int64_t>(rowq) * n_chunks + ch] = make_float2(kPosInf, kNegInf);
  }
}

// ---------------------------------------------------------------- FP4, 64 heads x 128
// gfx950's block-scaled MFMA (16x16x128, f8f6f4 with both operands E2M1)
// multiplies the E2M1 codes directly: lane l supplies row / column l % 16 and
// the 32 elements k = 32 (l / 16) .. +31, i.e. scale block l / 16, as 16 bytes
// in memory order (element 2i in the low nibble of byte i).  Its E8M0 block
// scales hold only powers of two, so they stay at 1 and the fp32 scales of
// the pages' recipe are applied in the epilogue: each block's partial dot
// product comes from an MFMA whose B operand keeps only that block's lanes
// (the others zero), so every partial is exact (products of E2M1 values are
// multiples of 1/4 below 36, 32 of them summed in fp32).  A wave covers 256
// keys as 16 tiles of 16 keys; lane (key n, block g) loads its 16 bytes of
// codes directly in the operand layout (a tile's 1 KB of codes is one
// coalesced 16-byte load per lane) and its key's four scales, two tiles ahead.
typedef int v8i32_t __attribute__((ext_vector_type(8)));
constexpr int kFp4Tiles = kKeysPerWave / 16;

__global__ __launch_bounds__(256) void score_fp4_h64d128_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale, int64_t k_sb, int64_t k_sn,
    int64_t ks_sb, int64_t ks_sn, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, float* __restrict__ scores,
    int64_t s_rs, float2* __restrict__ chunk_rep, int n_chunks, int bound_k) {
  const int row = blockIdx.y, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int chunk = blockIdx.x * kWavesPerWg + wave;
  const int key0 = chunk * kKeysPerWave;
  if (key0 >= N_max) return;
  const int key_end = min(key0 + kKeysPerWave, N_max);
  const int vis_end = min(key_end, V);
  float* srow = scores + row * s_rs;
  for (int j = max(key0, V) + lane; j < key_end; j += 64) srow[j] = kNegInf;
  if (key0 >= vis_end) {
    if (chunk_rep != nullptr && lane == 0)
      chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = make_float2(kPosInf, kNegInf);
    return;
  }

  // keys past the visible range are clamped to the last visible one (in
  // bounds, masked on output)
  const uint8_t* kb = k + b * k_sb + 16 * g;
  const float* ksb = k_scale + b * ks_sb;
  u32x4_t kc[3], ks[3];
  auto load_tile = [&](int t, u32x4_t& c, u32x4_t& sc4) {
    const int j = min(key0 + 16 * t + nl, vis_end - 1);
    c = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    sc4 = ld16_stream(ksb + static_cast<int64_t>(j) * ks_sn);
  };
  load_tile(0, kc[0], ks[0]);
  load_tile(1, kc[1], ks[1]);

  // A operand per head tile mt: head 16 mt + n, block g (16 bytes of codes)
  const uint8_t* qrow = q + static_cast<int64_t>(row) * 64 * 64;
  const float* qsrow = q_scale + static_cast<int64_t>(row) * 64 * 4;
  v8i32_t qa[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(qrow + (16 * mt + nl) * 64 + 16 * g);
    qa[mt] = v8i32_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]),
                     static_cast<int>(c[3]), 0, 0, 0, 0};
  }
  // accumulator rows: head = 16*mt + 4*g + r
  float sq[4][4][4];   // [mt][r][blk]
  float wv[4][4];
  const float* wrow = w + static_cast<int64_t>(row) * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * mt + 4 * g + r;
      wv[mt][r] = wrow[h];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) sq[mt][r][blk] = qsrow[h * 4 + blk];
    }

  float scv[kFp4Tiles];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < kFp4Tiles; ++t) {
    if (t + 2 < kFp4Tiles) load_tile(t + 2, kc[(t + 2) % 3], ks[(t + 2) % 3]);
    __builtin_amdgcn_sched_barrier(0);
    const u32x4_t c = kc[t % 3];
    const u32x4_t skr = ks[t % 3];
    const float skv[4] = {__uint_as_float(skr[0]), __uint_as_float(skr[1]),
                          __uint_as_float(skr[2]), __uint_as_float(skr[3])};
    f32x4_t p[4][4];     // [mt][blk]
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const bool mine = g == blk;
      const v8i32_t bm = {mine ? static_cast<int>(c[0]) : 0, mine ? static_cast<int>(c[1]) : 0,
                          mine ? static_cast<int>(c[2]) : 0, mine ? static_cast<int>(c[3]) : 0,
                          0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4_t z = {};
        p[mt][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], bm, z, 4, 4, 0, 127,
                                                                        0, 127);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float tv = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) tv = fmaf(sq[mt][r][blk] * skv[blk], p[mt][blk][r], tv);
        sum = fmaf(wv[mt][r], relu_f32(tv), sum);
      }
    // heads are spread over the four 16-lane groups of the key's column
    sum = sum + __shfl_xor(sum, 16, 64);
    sum = sum + __shfl_xor(sum, 32, 64);
    const int jj = key0 + 16 * t + nl;
    const bool ok = jj < vis_end;
    if (g == 0 && ok) srow[jj] = sum;
    scv[t] = ok ? sum : kNegInf;
    __builtin_amdgcn_sched_barrier(0);
  }
  const int thr_c = bound_c_row(V, bound_k);
  if (chunk_rep != nullptr && thr_c > 0) {
    const float2 rep = wave_chunk_report<kFp4Tiles>(scv, g == 0, thr_c);
    if (lane == 0) chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = rep;
  }
}

// ---------------------------------------------------------------- MX FP4 (E8M0 scales), 64 x 128
// The same operand layout with power-of-two block scales: lane (row / column
// l % 16, block l / 16) hands the MFMA its block's E8M0 byte, the hardware
// scales each block partial exactly, and one MFMA per 16-head tile gives the
// whole 128-dim dot product.  The epilogue is ReLU and w only (2 VALU
// operations per head and entry), so the kernel streams: a wave keeps
// kMxAhead tiles of codes (16 bytes per lane) and scale words (the key's four
// scale bytes, read by all four block lanes) in flight.
constexpr int kMxAhead = 3;

__global__ __launch_bounds__(256) void score_mx4_h64d128_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ k_scale, int64_t k_sb, int64_t k_sn, int64_t ks_sb,
    int64_t ks_sn, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries,
    int Tq, int N_max, int m, float* __restrict__ scores, int64_t s_rs,
    float2* __restrict__ chunk_rep, int n_chunks, int bound_k) {
  const int row = blockIdx.y, b = row / Tq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int V = visible_count(q_pos[row], m, n_entries[b], N_max);
  const int chunk = blockIdx.x * kWavesPerWg + wave;
  const int key0 = chunk * kKeysPerWave;
  if (key0 >= N_max) return;
  const int key_end = min(key0 + kKeysPerWave, N_max);
  const int vis_end = min(key_end, V);
  float* srow = scores + row * s_rs;
  for (int j = max(key0, V) + lane; j < key_end; j += 64) srow[j] = kNegInf;
  if (key0 >= vis_end) {
    if (chunk_rep != nullptr && lane == 0)
      chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = make_float2(kPosInf, kNegInf);
    return;
  }

  // keys past the visible range are clamped to the last visible one (in
  // bounds, masked on output)
  const uint8_t* kb = k + b * k_sb + 16 * g;
  const uint8_t* ksb = k_scale + b * ks_sb;
  u32x4_t kc[kMxAhead + 1];
  uint32_t ks[kMxAhead + 1];
  auto load_tile = [&](int t, u32x4_t& c, uint32_t& sw) {
    const int j = min(key0 + 16 * t + nl, vis_end - 1);
    c = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    sw = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ksb + static_cast<int64_t>(j) * ks_sn));
  };
#pragma unroll
  for (int t = 0; t < kMxAhead; ++t) load_tile(t, kc[t], ks[t]);

  // A operand per head tile mt: head 16 mt + n, block g (16 bytes of codes)
  // and that block's scale byte
  const uint8_t* qrow = q + static_cast<int64_t>(row) * 64 * 64;
  const uint8_t* qsrow = q_scale + static_cast<int64_t>(row) * 64 * 4;
  v8i32_t qa[4];
  int sa[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(qrow + (16 * mt + nl) * 64 + 16 * g);
    qa[mt] = v8i32_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]),
                     static_cast<int>(c[3]), 0, 0, 0, 0};
    sa[mt] = qsrow[(16 * mt + nl) * 4 + g];
  }
  // accumulator rows: head = 16*mt + 4*g + r
  float wv[4][4];
  const float* wrow = w + static_cast<int64_t>(row) * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wrow[16 * mt + 4 * g + r];

  float scv[kFp4Tiles];
#pragma unroll
  for (int t = 0; t < kFp4Tiles; ++t) {
    if (t + kMxAhead < kFp4Tiles)
      load_tile(t + kMxAhead, kc[(t + kMxAhead) % (kMxAhead + 1)], ks[(t + kMxAhead) % (kMxAhead + 1)]);
    const u32x4_t c = kc[t % (kMxAhead + 1)];
    const int sb = static_cast<int>((ks[t % (kMxAhead + 1)] >> (8 * g)) & 0xffu);
    const v8i32_t bc = {static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]),
                        static_cast<int>(c[3]), 0, 0, 0, 0};
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4_t z = {};
      const f32x4_t p =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], bc, z, 4, 4, 0, sa[mt], 0, sb);
#pragma unroll
      for (int r = 0; r < 4; ++r) sum = fmaf(wv[mt][r], relu_f32(p[r]), sum);
    }
    // heads are spread over the four 16-lane groups of the key's column
    sum = sum + __shfl_xor(sum, 16, 64);
    sum = sum + __shfl_xor(sum, 32, 64);
    const int jj = key0 + 16 * t + nl;
    const bool ok = jj < vis_end;
    if (g == 0 && ok) srow[jj] = sum;
    scv[t] = ok ? sum : kNegInf;
  }
  const int thr_c = bound_c_row(V, bound_k);
  if (chunk_rep != nullptr && thr_c > 0) {
    const float2 rep = wave_chunk_report<kFp4Tiles>(scv, g == 0, thr_c);
    if (lane == 0) chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = rep;
  }
}

template <typename T, int D>
void launch_generic(const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((a.N_max + 255) / 256, a.B * a.Tq);
  hipLaunchKernelGGL((score_generic_kernel<T, D>), grid, dim3(256), 0, s,
                     static_cast<const T*>(a.q), a.w, static_cast<const T*>(a.k), a.k_sb, a.k_sn,
                     a.q_pos, a.n_entries, a.Tq, a.N_max, a.m, a.H, static_cast<float*>(a.scores),
                     a.s_rs);
}

}  // namespace

bool score_tuned(csa_dtype_t dt, int H, int D) {
  return (dt == CSA_FP4_E2M1 || dt == CSA_FP4_E2M1_E8M0 || dt == CSA_BF16) && H == 64 &&
         D == 128;
}

int score_chunk_keys() { return kKeysPerWave; }

bool score16_supported(csa_dtype_t dt, int H, int D) { return dt == CSA_BF16 && H == 64 && D == 128; }

bool score_supported(csa_dtype_t dt, int H, int D) {
  if (dt == CSA_FP4_E2M1 || dt == CSA_FP4_E2M1_E8M0) return H == 64 && D == 128;
  if (dt != CSA_F32 && dt != CSA_BF16) return false;
  return H >= 1 && H <= 64 && (D == 32 || D == 64 || D == 128);
}

hipError_t launch_score(const ScoreArgs& a, csa_dtype_t dt, hipStream_t s) {
  if (dt == CSA_FP4_E2M1) {
    const dim3 grid((a.N_max + kKeysPerWg - 1) / kKeysPerWg, a.B * a.Tq);
    hipLaunchKernelGGL(score_fp4_h64d128_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(a.q), static_cast<const float*>(a.q_scale),
                       a.w, static_cast<const uint8_t*>(a.k),
                       static_cast<const float*>(a.k_scale), a.k_sb, a.k_sn, a.ks_sb, a.ks_sn,
                       a.q_pos, a.n_entries, a.Tq, a.N_max, a.m, static_cast<float*>(a.scores),
                       a.s_rs, a.chunk_rep, a.n_chunks, a.bound_k);
  } else if (dt == CSA_FP4_E2M1_E8M0) {
    const dim3 grid((a.N_max + kKeysPerWg - 1) / kKeysPerWg, a.B * a.Tq);
    hipLaunchKernelGGL(score_mx4_h64d128_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.q_scale),
                       a.w, static_cast<const uint8_t*>(a.k),
                       static_cast<const uint8_t*>(a.k_scale), a.k_sb, a.k_sn, a.ks_sb, a.ks_sn,
                       a.q_pos, a.n_entries, a.Tq, a.N_max, a.m, static_cast<float*>(a.scores),
                       a.s_rs, a.chunk_rep, a.n_chunks, a.bound_k);
  } else if (dt == CSA_BF16 && a.H == 64 && a.D == 128 && a.Tq >= kPfQueries) {
    const int groups = (a.Tq + kPfQueries - 1) / kPfQueries;
    const dim3 grid((a.N_max + kPfKeys - 1) / kPfKeys, a.B * groups);
    if (a.score16)
      hipLaunchKernelGGL(score_prefill_bf16_h64d128_kernel<uint16_t>, grid, dim3(kPfThreads), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<uint16_t*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k);
    else
      hipLaunchKernelGGL(score_prefill_bf16_h64d128_kernel<float>, grid, dim3(kPfThreads), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<float*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k);
  } else if (dt == CSA_BF16 && a.H == 64 && a.D == 128) {
    const dim3 grid((a.N_max + kKeysPerWg - 1) / kKeysPerWg, a.B * a.Tq);
    if (a.score16)
      hipLaunchKernelGGL(score_bf16_h64d128_kernel<uint16_t>, grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<uint16_t*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k);
    else
      hipLaunchKernelGGL(score_bf16_h64d128_kernel<float>, grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<float*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k);
  } else if (dt == CSA_BF16) {
    if (a.D == 32) launch_generic<uint16_t, 32>(a, s);
    else if (a.D == 64) launch_generic<uint16_t, 64>(a, s);
    else launch_generic<uint16_t, 128>(a, s);
  } else {
    if (a.D == 32) launch_generic<float, 32>(a, s);
    else if (a.D == 64) launch_generic<float, 64>(a, s);
    else launch_generic<float, 128>(a, s);
  }
  return hipGetLastError();
}

}  // namespace csa
