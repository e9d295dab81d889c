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
// exchange between lanes l and l^32.  K rows are read with whole-row
// coalesced loads, one tile ahead of the MFMAs, and reach the B operand
// (lane l%32 = key row, 16 contiguous bytes per lane per k-step) through a
// wave-private LDS tile.
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
// below the exact c-th largest, for a fraction of its cost; the valid lanes
// are among lanes 0..31), and the largest score.  Every chunk that reports a finite value holds c entries at
// or above it, and the floor(V / kBoundChunk) full chunks all do (every lane
// holds valid entries, c <= 16), so the ceil(k / c)-th largest report is at
// most the row's k-th largest score.  The top-k kernels use that bound to
// drop most entries before selecting, and the largest report as the top of
// the survivors' range.  A chunk with fewer than c lanes holding valid
// entries reports +inf (-inf as its largest when it has none); rows with no
// bound (c = 0) write nothing.
constexpr float kPosInf = __builtin_inff();

// The value of lane l ^ j (j = 1, 2, 4, 8, 16) for the sorting network
// below: DPP inside a 16-lane row for j < 16 (quad permutes; for j = 4 the
// half-row mirror 8h + 7 - i followed by the quad reversal 4q + 3 - i, which
// together give 8h + 4(1 - a) + i = l ^ 4 for l = 8h + 4a + i; the row
// rotation by 8), a lane swizzle for j = 16.  j is a constant after unrolling.
__device__ __forceinline__ float lane_xor(float v, int j) {
  const int x = __float_as_int(v);
  if (j == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  if (j == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if (j == 4) {
    const int m = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
    return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false));
  }
  if (j == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  return __shfl_xor(v, 16, 64);
}

template <int NV>
__device__ float2 wave_chunk_report(const float (&vals)[NV], bool active, int c) {
  const int lane = threadIdx.x & 63;
  float v = kNegInf;
#pragma unroll
  for (int i = 0; i < NV; ++i) v = fmaxf(v, vals[i]);
  if (!active) v = kNegInf;
  // Bitonic sort of the 32 lane maxima of lanes 0..31 into descending order
  // (15 compare-exchange stages, all in registers; lanes 32..63 sort their
  // own values, unused).  Before it, c rounds of a full-wave maximum and
  // removal took 2 us of a 23 us launch.
#pragma unroll
  for (int k = 2; k <= 32; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float o = lane_xor(v, j);
      const bool want_max = ((lane & j) == 0) == ((lane & k) == 0);
      v = want_max ? fmaxf(v, o) : fminf(v, o);
    }
  }
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const int cu = __builtin_amdgcn_readfirstlane(c);
  const float cth = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), cu - 1));
  return make_float2(cth == kNegInf ? kPosInf : cth, top);
}

// ---------------------------------------------------------------- bf16, 64 heads x 128
constexpr int kWavesPerWg = 4;
constexpr int kTilesPerWave = 8;                  // tiles of 32 keys
constexpr int kKeysPerWave = 32 * kTilesPerWave;  // one selection chunk
constexpr int kKeysPerWg = kWavesPerWg * kKeysPerWave;
static_assert(kKeysPerWave == kBoundChunk, "one bound chunk per wave");

// Tile order: a row's keys are read as tiles of 32 (8 KB); chunk c of the row
// (0 <= c < nch = ceil(N_max / 256)) is the strided set of tiles c, c + nch,
// c + 2 nch, ...  At each step the waves of a row therefore read one
// contiguous stretch of the key cache together, instead of every wave
// streaming its own region: HBM serves the stretch at about 6.4 TB/s, the
// per-wave regions at about 5.6 (the chunk reports only need disjoint sets
// of keys).  In the decode kernel a wave takes two chunks, w and w + nw (nw
// waves per row), one after the other: half the waves, each amortising its
// query staging over twice the keys (4 % faster than one chunk per wave;
// four chunks per wave leave half the compute units idle at 128K).  At 128K
// that is one 4-wave workgroup per compute unit, one wave per SIMD, which
// leaves the registers to hold the query heads (the A operand) for the whole
// wave instead of re-reading them from LDS every tile.
// Straight-line code over the wave's 16 tiles with a 2-deep ring of
// registers: the loads of tile t+1 are issued before tile t is staged and
// multiplied and no register is copied, so one tile (8 KB per wave) stays in
// flight behind the math (two in flight measured slower: more requests
// queued at HBM at once); the epilogue of tile t-1 runs while the MFMAs of
// tile t do.
// Loads are coalesced and non-temporal (instruction i of a tile reads key
// rows 4i .. 4i+3 whole, 16 lanes per row); each tile then passes through a
// wave-private LDS buffer to reach the MFMA B-operand layout (lane (j, g)
// holds dims 16s + 8g .. +7 of key j).  Rows past the visible range are
// clamped to the last visible row (in bounds, cache hits) and masked on
// output.
constexpr int kKeyPitch = 136;                    // bf16 per key row in LDS (256 B + 16 B)
constexpr int kChunksPerWave = 2;                 // 256-key chunks per wave (decode kernel)
constexpr int kDecodeTiles = kTilesPerWave * kChunksPerWave;

template <typename SO>
__global__ __launch_bounds__(256, 1) void score_bf16_h64d128_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    int64_t k_sb, int64_t k_sn, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, SO* __restrict__ scores,
    int64_t s_rs, float2* __restrict__ chunk_rep, int n_chunks, int bound_k) {
  __shared__ __attribute__((aligned(16))) uint16_t key_lds[kWavesPerWg][32 * kKeyPitch];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[64 * kKeyPitch];
  const int row = blockIdx.y, b = row / Tq;
  // Every argument in registers before its first use (the argument loads go
  // out together, one round trip); then the two values read from memory,
  // whose loads go out ahead of the query and key loads below and which
  // only the masking waits for.
  asm volatile("" ::"s"(q), "s"(w), "s"(k), "s"(k_sb), "s"(k_sn), "s"(q_pos), "s"(n_entries),
               "s"(Tq), "s"(N_max), "s"(m), "s"(scores), "s"(s_rs), "s"(chunk_rep), "s"(n_chunks),
               "s"(bound_k));
  const int qp = q_pos[row], ne = n_entries[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int jl = lane & 31, g = lane >> 5;
  const int wid = blockIdx.x * kWavesPerWg + wave;    // this wave within the row
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  // q_I rows (heads) of this query are staged in LDS by the whole workgroup
  // (coalesced 16-byte loads) and read back by every wave in the A-operand
  // layout
  const uint16_t* qrow = q + static_cast<int64_t>(row) * 64 * 128;
  u32x4_t qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qv[i] = *reinterpret_cast<const u32x4_t*>(qrow + 8 * (static_cast<int>(threadIdx.x) + 256 * i));
  const int nch = (N_max + kKeysPerWave - 1) / kKeysPerWave;
  const int nw = (nch + kChunksPerWave - 1) / kChunksPerWave;   // waves per row
  // tile t of the wave: tile t % 8 of its chunk wid + (t / 8) nw
  auto chunk_of = [&](int t) { return wid + (t / kTilesPerWave) * nw; };
  auto tile_key0 = [&](int t) { return 32 * ((t % kTilesPerWave) * nch + chunk_of(t)); };
  // The first key tile is requested before the query is staged and the
  // barrier passed, so that its latency overlaps the query's (the
  // empty asm with a memory clobber keeps the compiler from sinking them
  // below).  Every wave issues it, also one that exits below, with rows
  // clamped into the cache (N_max >= 1): it needs neither q_pos nor
  // n_entries, and the keys past the visible ones are masked in the
  // epilogue.  Later tiles are clamped to [0, vis - 1] (row 0 when nothing
  // is visible), so that a partly visible row reads no more than it shows.
  const uint16_t* kb = k + b * k_sb + 8 * (lane & 15);
  const int lrow = lane >> 4;                     // row within each 4-row load
  u32x4_t kt[2][8];
  auto load_tile_clamped = [&](int t, u32x4_t (&dst)[8], int jcap) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(tile_key0(t) + 4 * i + lrow, jcap);
      dst[i] = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    }
  };
  load_tile_clamped(0, kt[0], N_max - 1);
  asm volatile("" ::"s"(k) : "memory");
  const int V = visible_count(qp, m, ne, N_max);
  const int vis = min(V, N_max);
  const int jmax = max(vis - 1, 0);
  auto load_tile = [&](int t, u32x4_t (&dst)[8]) { load_tile_clamped(t, dst, jmax); };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = static_cast<int>(threadIdx.x) + 256 * i;       // 16-byte chunk: head c / 16
    *(lds_u32x4*)((lds_u16*)q_lds + (c >> 4) * kKeyPitch + 8 * (c & 15)) = qv[i];
  }
  __syncthreads();                                // the only barrier: early exits follow
  if (wid >= nw) return;                          // past the row
  SO* srow = scores + row * s_rs;
  if (tile_key0(0) >= vis) {                      // the wave's smallest key: nothing visible
    for (int t = 0; t < kDecodeTiles; ++t) {
      const int j = tile_key0(t) + jl;
      if (g == 0 && chunk_of(t) < nch && j < N_max) put_score(&srow[j], kNegInf);
    }
    for (int x = 0; x < kChunksPerWave; ++x)
      if (chunk_rep != nullptr && lane == 0 && chunk_of(kTilesPerWave * x) < nch)
        chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk_of(kTilesPerWave * x)] =
            make_float2(kPosInf, kNegInf);
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

  // the A operand (32 heads x 128 dims per 32x32 tile, two tiles) read from
  // LDS once into registers: one wave per SIMD leaves room for it
  bf16x8_t qa0[8], qa1[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4_t x0 = *(const lds_u32x4*)(ql + 16 * s);
    const u32x4_t x1 = *(const lds_u32x4*)(ql + 32 * kKeyPitch + 16 * s);
    __builtin_memcpy(&qa0[s], &x0, 16);
    __builtin_memcpy(&qa1[s], &x1, 16);
  }
  float sc[kChunksPerWave][kTilesPerWave];
  const int thr_c = bound_c_row(V, bound_k);
  // epilogue of tile t from its accumulators: sum_h w[h] ReLU(s_h), then the
  // two lane halves (32 heads each) add up; after a chunk's last tile, its
  // report
  auto epilogue = [&](int t, const f32x16_t& c0, const f32x16_t& c1) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(w0[r], relu_f32(c0[r]), sum);
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(w1[r], relu_f32(c1[r]), sum);
    const float other = __shfl_xor(sum, 32, 64);
    const float tot = sum + other;     // commutative: both halves get the same bits
    const int j = tile_key0(t) + jl;
    const bool mine = chunk_of(t) < nch;
    const bool ok = mine && j < vis;
    if (g == 0 && mine && j < N_max) put_score(&srow[j], ok ? tot : kNegInf);
    sc[t / kTilesPerWave][t % kTilesPerWave] = ok ? tot : kNegInf;
    if (t % kTilesPerWave == kTilesPerWave - 1 && chunk_rep != nullptr && thr_c > 0 && mine) {
      const float2 rep = wave_chunk_report<kTilesPerWave>(sc[t / kTilesPerWave], g == 0, thr_c);
      if (lane == 0)
        chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk_of(t)] = stored_report<SO>(rep);
    }
  };
  // Iteration t: loads of tile t+1, tile t through LDS into the MFMAs, and
  // the epilogue of tile t-1 while those MFMAs run (two accumulator sets).
  // sched_barrier(0) keeps the scheduler from sinking the prefetch loads
  // below the MFMAs of the current tile (it would, to shorten live ranges).
  f32x16_t acc[2][2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < kDecodeTiles; ++t) {
    if (t + 1 < kDecodeTiles) load_tile(t + 1, kt[(t + 1) % 2]);
    __builtin_amdgcn_sched_barrier(0);
    // tile t: registers -> LDS (rows 4i + lrow) -> B operand (row jl)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(lds_u32x4*)(kl + (4 * i + lrow) * kKeyPitch + 8 * (lane & 15)) = kt[t % 2][i];
    bf16x8_t cur[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4_t x = *(const lds_u32x4*)(kl + jl * kKeyPitch + 16 * s + 8 * g);
      __builtin_memcpy(&cur[s], &x, 16);
    }
    f32x16_t (&c)[2] = acc[t & 1];
    c[0] = f32x16_t{};
    c[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa0[s], cur[s], c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa1[s], cur[s], c[1], 0, 0, 0);
    }
    if (t > 0) epilogue(t - 1, acc[(t - 1) & 1][0], acc[(t - 1) & 1][1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  epilogue(kDecodeTiles - 1, acc[(kDecodeTiles - 1) & 1][0], acc[(kDecodeTiles - 1) & 1][1]);
}

// ---------------------------------------------------------------- bf16 prefill (many queries)
// With many query tokens per sequence the score is a GEMM with the (query,
// head) pairs as rows, keys as columns and the 128 dims as the reduction,
// followed by the per-query epilogue sum_h w[h] ReLU(.).  One workgroup of
// 8 waves takes 8 queries of one sequence (one per wave: two 32-row A tiles
// of q_I held in registers) against 4096 keys, in blocks of 256 keys (one
// selection chunk, 64 KB) that go from memory straight into LDS
// (global_load_lds_dwordx4, no staging registers), double-buffered, with one
// barrier per block: the next block is requested at the top of each block,
// whose 64 KB all 8 queries then read, 16 MFMA 32x32x16 per wave per 32-key
// tile, the ReLU-w epilogue of tile u-1 running under the MFMAs of tile u.
// The kernel holds about 240 VGPRs and 128 KB of LDS, so a compute unit runs
// one workgroup (two waves per SIMD); the grid is ordered so that each XCD
// works through its own eighth of the key blocks (below).  The selection
// bounds are produced per 256-key chunk exactly as in the decode kernel.
//
// Measured on one box against the former design (32-key tiles staged
// through registers and an LDS tile, one barrier per tile, 2048 keys per
// workgroup): 4.29 -> 3.68 ms for the 4096-query chunk at 66,560 entries,
// scores bitwise identical.  Steps, each kept for what it measured: the
// stores made branch-free so the compiler's waits count exactly (the four-
// tile register ring had held two tiles in flight), 4096 keys per workgroup,
// blocks loaded straight into LDS with one barrier per block, the lane
// halves' sums added by a register swap instead of an LDS permute (whose
// wait had also waited for every B-operand read in flight).  Measured and
// dropped: B operands of the next tile read ahead under a scheduling
// barrier (8 % slower), a single accumulator set (equal), 12 waves of 168
// VGPRs (three per SIMD, equal), waves of a SIMD staggered by a sleep
// (equal), 8192 or 16384 keys per workgroup (equal, 3 % slower).

// Raw buffer stores: the hardware drops a store whose byte offset is at or
// past the record count of the buffer resource, so kOob turns a store off
// without a branch.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void buf_score(__amdgpu_buffer_rsrc_t r, uint32_t off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_score(__amdgpu_buffer_rsrc_t r, uint32_t off, float v, uint16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(bf16_rne_bits(v), r, off, 0, 0);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buf_rep(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(v.x), __float_as_uint(v.y)}, r, off, 0, 0);
}
constexpr int kPfQueries = 8;
constexpr int kPfThreads = 64 * kPfQueries;
constexpr int kPfKeys = 4096;

constexpr int kPbRows = kBoundChunk;             // keys per LDS block: one report chunk
constexpr int kPbBytes = kPbRows * 256;           // 64 KB of bf16 keys
constexpr int kPbTiles = kPbRows / 32;
static_assert(kPbTiles == kTilesPerWave, "a block is one chunk of tiles");

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low bits 3:0
// and high bits 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
#define CSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

template <typename SO>
__global__ __launch_bounds__(kPfThreads, 2) void score_prefill_bf16_h64d128_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    int64_t k_sb, int64_t k_sn, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_entries, int Tq, int N_max, int m, SO* __restrict__ scores,
    int64_t s_rs, float2* __restrict__ chunk_rep, int n_chunks, int bound_k, int n_qgroups) {
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  __shared__ __attribute__((aligned(1024))) uint8_t blk_lds[2][kPbBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jl = lane & 31, g = lane >> 5;
  const int groups = (Tq + kPfQueries - 1) / kPfQueries;
  // XCD-aware order (a one-dimensional grid of 8 * ceil(units / 8)
  // workgroups): the dispatcher hands workgroup i to XCD i % 8, and the
  // (key block, query group) units, in key-block-major order, are cut into
  // eight contiguous ranges, range x for the workgroups of XCD x.  Each XCD
  // then reads about an eighth of the key blocks, which stay in its L2 while
  // all query groups pass over them: 1.4 GB of L2 fills per launch on the
  // 4096-query chunk instead of 8.2 GB with the key block varying fastest
  // across the grid (same time).  Correctness does not depend on the
  // placement.
  const int nkb = (N_max + kPfKeys - 1) / kPfKeys;
  const int units = nkb * n_qgroups;
  const int per_xcd = (units + 7) / 8;
  const int unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (unit >= units) return;                      // grid padding (no barrier passed yet)
  const int kblk = unit / n_qgroups, qgrp = unit % n_qgroups;
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
  const int nblk = (ntiles + kPbTiles - 1) / kPbTiles;

  // -inf for every key this workgroup covers but does not compute
  if (rowq >= 0) {
    SO* srow = scores + rowq * s_rs;
    for (int j = j0 + 32 * ntiles + lane; j < j1; j += 64) put_score(&srow[j], kNegInf);
  }
  const uint16_t* kb = k + b * k_sb;
  const int jcap = max(vmax, 1) - 1;              // clamp rows to visible ones (in bounds)

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
  // A block of 256 keys goes straight from memory into LDS buffer `buf`,
  // laid out by k-slice: the 32 bytes of dims 16 s .. 16 s + 15 of block row
  // r sit at 8192 s + 32 r, their two 16-byte halves swapped in rows with
  // (r / 8) odd, so that 16 lanes reading one half of rows r0 .. r0 + 15
  // touch 64 distinct 4-byte banks (measured as fast as an XOR-swizzled
  // row-major layout, whose reads need a per-slice address).  Each 16-byte load
  // writes LDS byte 16 l of its kilobyte for lane l, so instruction i of
  // wave v (kilobyte 8 v + i: slice v, rows 32 i .. 32 i + 31) has lane l
  // fetch row 32 i + l / 2, the half that belongs at position l % 2.  Rows
  // past the visible ones are clamped (in bounds; their scores are masked).
  auto load_block = [&](int blk, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 8 * wave + i;                  // kilobyte of the buffer
      const int s2 = kk >> 3;                       // its k-slice
      const int r = 32 * (kk & 7) + (lane >> 1);    // block row
      const int c = 2 * s2 + ((lane & 1) ^ ((r >> 3) & 1));   // 16-byte chunk of the row
      const int j = min(j0 + kPbRows * blk + r, jcap);
      const uint16_t* gp = kb + static_cast<int64_t>(j) * k_sn + 8 * c;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gp,
                                       (void __attribute__((address_space(3)))*)&blk_lds[buf][1024 * (8 * wave + i)],
                                       16, 0, 0);
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  load_block(0, 0);
  const int cq = __builtin_amdgcn_readfirstlane(chunk_rep != nullptr && rowq >= 0 ? bound_c_row(vq, bound_k) : 0);
  // store windows: the query's scores of this key block, its chunk reports
  // (empty for an invalid query or without reports)
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(
      scores + static_cast<int64_t>(max(rowq, 0)) * s_rs + j0,
      rowq >= 0 ? static_cast<uint32_t>(j1 - j0) * static_cast<uint32_t>(sizeof(SO)) : 0u);
  const __amdgpu_buffer_rsrc_t rrs = make_rsrc(
      chunk_rep + (chunk_rep != nullptr ? static_cast<int64_t>(max(rowq, 0)) * n_chunks : 0),
      chunk_rep != nullptr && rowq >= 0 ? static_cast<uint32_t>(n_chunks) * 8u : 0u);
  // B operand of tile u, k-slice s: block row 32 u + jl, dims 16 s + 8 g .. +7
  auto mfma_tile = [&](int buf, int u, f32x16_t (&acc)[2]) {
    const lds_u8* rowp = (const lds_u8*)&blk_lds[buf][(32 * u + jl) * 32 + 16 * (g ^ ((jl >> 3) & 1))];
    acc[0] = f32x16_t{};
    acc[1] = f32x16_t{};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const u32x4_t x = *(const lds_u32x4*)(rowp + 8192 * s2);
      bf16x8_t bb;
      __builtin_memcpy(&bb, &x, 16);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s2], bb, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s2], bb, acc[1], 0, 0, 0);
    }
  };
  float sc[kTilesPerWave];
  // epilogue of tile u of block blk from its accumulators: the score store
  // (dropped past the last computed tile or the key block) and sc[u]
  auto epilogue = [&](int blk, int u, const f32x16_t (&c)[2]) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(wv[0][r], relu_f32(c[0][r]), sum);
#pragma unroll
    for (int r = 0; r < 16; ++r) sum = fmaf(wv[1][r], relu_f32(c[1][r]), sum);
    // the two lane halves' sums added by a register swap of the halves (no
    // LDS instruction, so no wait on the B-operand reads in flight)
    const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    const float tot = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
    const int tt = kPbTiles * blk + u;
    const bool live = tt < ntiles;
    const bool ok = live && j0 + 32 * tt + jl < vq;
    const uint32_t so = static_cast<uint32_t>(32 * tt + jl) * static_cast<uint32_t>(sizeof(SO));
    buf_score(srs, g == 0 && live ? so : kOob, ok ? tot : kNegInf, (SO*)nullptr);
    sc[u] = ok ? tot : kNegInf;
  };
  f32x16_t acc[2][2];

  // One barrier per block.  At the top of block blk its loads have landed
  // (each thread waits for its own, the barrier for everybody's) and every
  // wave is done with block blk - 1, whose buffer then takes block blk + 1.
  // Inside a block the MFMAs of tile u run under the epilogue of tile u - 1.
  // The waits count exactly: after a block's loads come, on every path, the
  // eight score stores and one report store of the block before it.
  CSA_WAIT_VMCNT(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    if (blk > 0) {
      CSA_WAIT_VMCNT(kPbTiles + 1);
      __syncthreads();
    }
    if (blk + 1 < nblk) load_block(blk + 1, buf ^ 1);
    // the next block's loads stay ahead of this block's stores (the wait at
    // the top of the next block counts the stores issued after them)
    __builtin_amdgcn_sched_barrier(0);
    mfma_tile(buf, 0, acc[0]);
#pragma unroll
    for (int u = 1; u < kPbTiles; ++u) {
      mfma_tile(buf, u, acc[u & 1]);
      epilogue(blk, u - 1, acc[(u - 1) & 1]);
    }
    epilogue(blk, kPbTiles - 1, acc[(kPbTiles - 1) & 1]);
    // the block's chunk bound
    float2 rep = make_float2(0.f, 0.f);
    if (cq > 0) rep = stored_report<SO>(wave_chunk_report<kTilesPerWave>(sc, g == 0, cq));
    const uint32_t ro = static_cast<uint32_t>((j0 + kPbRows * blk) / kBoundChunk) * 8u;
    buf_rep(rrs, cq > 0 && lane == 0 ? ro : kOob, rep);
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
// product comes from an MFMA whose A operand keeps only that block's lanes
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
  const int chunk = blockIdx.x * kWavesPerWg + wave;
  // tiles of 16 keys in the interleaved order of the bf16 kernel: wave c of
  // the row takes tiles c, c + nch, c + 2 nch, ...
  // Every argument in registers before its first use (one round trip for
  // the argument loads); then q_pos and n_entries, whose loads go out ahead
  // of the key loads and which only the masking waits for.
  asm volatile("" ::"s"(q), "s"(q_scale), "s"(w), "s"(k), "s"(k_scale), "s"(k_sb), "s"(k_sn),
               "s"(ks_sb), "s"(ks_sn), "s"(q_pos), "s"(n_entries), "s"(Tq), "s"(N_max), "s"(m),
               "s"(scores), "s"(s_rs), "s"(chunk_rep), "s"(n_chunks), "s"(bound_k));
  const int nch = (N_max + kKeysPerWave - 1) / kKeysPerWave;
  if (chunk >= nch) return;
  const int qp = q_pos[row], ne = n_entries[b];
  auto tile_key0 = [&](int t) { return 16 * (t * nch + chunk); };
  const uint8_t* kb = k + b * k_sb + 16 * g;
  const float* ksb = k_scale + b * ks_sb;
  u32x4_t kc[3], ks[3];
  auto load_tile_clamped = [&](int t, u32x4_t& c, u32x4_t& sc4, int jcap) {
    const int j = min(tile_key0(t) + nl, jcap);
    c = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    sc4 = ld16_stream(ksb + static_cast<int64_t>(j) * ks_sn);
  };
  // the first two tiles with rows clamped into the cache (N_max >= 1): they
  // need neither q_pos nor n_entries; keys past the visible ones are masked
  // on output
  load_tile_clamped(0, kc[0], ks[0], N_max - 1);
  load_tile_clamped(1, kc[1], ks[1], N_max - 1);
  asm volatile("" ::"s"(k) : "memory");           // the loads above stay ahead of the exit below

  const int V = visible_count(qp, m, ne, N_max);
  const int vis = min(V, N_max);
  float* srow = scores + row * s_rs;
  if (tile_key0(0) >= vis) {                      // no visible key in this wave's tiles
    for (int t = 0; t < kFp4Tiles; ++t) {
      const int j = tile_key0(t) + nl;
      if (g == 0 && j < N_max) srow[j] = kNegInf;
    }
    if (chunk_rep != nullptr && lane == 0)
      chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = make_float2(kPosInf, kNegInf);
    return;
  }
  // later tiles: keys past the visible range clamped to the last visible one
  // (in bounds, masked on output)
  auto load_tile = [&](int t, u32x4_t& c, u32x4_t& sc4) { load_tile_clamped(t, c, sc4, vis - 1); };

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
  // the A operand of block blk keeps only the lanes of that block (the others
  // zero), built once per wave: every key tile then feeds its codes unmasked
  // (masking B per tile cost 16 VALU instructions per tile, 10 % of the time)
  v8i32_t qm[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const bool mine = g == blk;
      qm[mt][blk] = v8i32_t{mine ? qa[mt][0] : 0, mine ? qa[mt][1] : 0, mine ? qa[mt][2] : 0,
                            mine ? qa[mt][3] : 0, 0, 0, 0, 0};
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
      const v8i32_t bm = {static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]),
                          static_cast<int>(c[3]), 0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4_t z = {};
        p[mt][blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qm[mt][blk], bm, z, 4, 4, 0,
                                                                        127, 0, 127);
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
    const int jj = tile_key0(t) + nl;
    const bool ok = jj < vis;
    if (g == 0 && jj < N_max) srow[jj] = ok ? sum : kNegInf;
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
  const int chunk = blockIdx.x * kWavesPerWg + wave;
  // tiles of 16 keys in the interleaved order of the bf16 kernel: wave c of
  // the row takes tiles c, c + nch, c + 2 nch, ...
  // Every argument in registers before its first use (one round trip for
  // the argument loads); then q_pos and n_entries, whose loads go out ahead
  // of the query and key loads and which only the masking waits for.
  asm volatile("" ::"s"(q), "s"(q_scale), "s"(w), "s"(k), "s"(k_scale), "s"(k_sb), "s"(k_sn),
               "s"(ks_sb), "s"(ks_sn), "s"(q_pos), "s"(n_entries), "s"(Tq), "s"(N_max), "s"(m),
               "s"(scores), "s"(s_rs), "s"(chunk_rep), "s"(n_chunks), "s"(bound_k));
  const int nch = (N_max + kKeysPerWave - 1) / kKeysPerWave;
  if (chunk >= nch) return;
  const int qp = q_pos[row], ne = n_entries[b];
  auto tile_key0 = [&](int t) { return 16 * (t * nch + chunk); };
  const uint8_t* kb = k + b * k_sb + 16 * g;
  const uint8_t* ksb = k_scale + b * ks_sb;
  u32x4_t kc[kMxAhead + 1];
  uint32_t ks[kMxAhead + 1];
  auto load_tile_clamped = [&](int t, u32x4_t& c, uint32_t& sw, int jcap) {
    const int j = min(tile_key0(t) + nl, jcap);
    c = ld16_stream(kb + static_cast<int64_t>(j) * k_sn);
    sw = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ksb + static_cast<int64_t>(j) * ks_sn));
  };
  // the first tiles with rows clamped into the cache (N_max >= 1): they need
  // neither q_pos nor n_entries; keys past the visible ones are masked on
  // output
#pragma unroll
  for (int t = 0; t < kMxAhead; ++t) load_tile_clamped(t, kc[t], ks[t], N_max - 1);

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
  asm volatile("" ::"s"(k) : "memory");           // the loads above stay ahead of the exit below

  const int V = visible_count(qp, m, ne, N_max);
  const int vis = min(V, N_max);
  float* srow = scores + row * s_rs;
  if (tile_key0(0) >= vis) {                      // no visible key in this wave's tiles
    for (int t = 0; t < kFp4Tiles; ++t) {
      const int j = tile_key0(t) + nl;
      if (g == 0 && j < N_max) srow[j] = kNegInf;
    }
    if (chunk_rep != nullptr && lane == 0)
      chunk_rep[static_cast<int64_t>(row) * n_chunks + chunk] = make_float2(kPosInf, kNegInf);
    return;
  }
  // later tiles: keys past the visible range clamped to the last visible one
  // (in bounds, masked on output)
  auto load_tile = [&](int t, u32x4_t& c, uint32_t& sw) { load_tile_clamped(t, c, sw, vis - 1); };

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
    const int jj = tile_key0(t) + nl;
    const bool ok = jj < vis;
    if (g == 0 && jj < N_max) srow[jj] = ok ? sum : kNegInf;
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
    const int nkb = (a.N_max + kPfKeys - 1) / kPfKeys;
    const int units = nkb * a.B * groups;
    const dim3 grid(8 * ((units + 7) / 8));
    if (a.score16)
      hipLaunchKernelGGL(score_prefill_bf16_h64d128_kernel<uint16_t>, grid, dim3(kPfThreads), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<uint16_t*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k, a.B * groups);
    else
      hipLaunchKernelGGL(score_prefill_bf16_h64d128_kernel<float>, grid, dim3(kPfThreads), 0, s,
                         static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                         a.k_sb, a.k_sn, a.q_pos, a.n_entries, a.Tq, a.N_max, a.m,
                         static_cast<float*>(a.scores), a.s_rs, a.chunk_rep, a.n_chunks,
                         a.bound_k, a.B * groups);
  } else if (dt == CSA_BF16 && a.H == 64 && a.D == 128) {
    const int nch = (a.N_max + kKeysPerWave - 1) / kKeysPerWave;
    const int nw = (nch + kChunksPerWave - 1) / kChunksPerWave;
    const dim3 grid((nw + kWavesPerWg - 1) / kWavesPerWg, a.B * a.Tq);
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
