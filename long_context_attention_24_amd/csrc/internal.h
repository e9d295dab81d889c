// Host-side launchers implemented in the .hip files; called by csa_api.cpp
// after argument validation.  Each returns the HIP error of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// ---- compress.hip
hipError_t launch_compress(const void* x, int64_t x_sb, int64_t x_st, const float* z, int64_t z_sb,
                           void* out, int64_t o_sb, int64_t o_sj, csa_dtype_t dt, int B, int n,
                           int C, int m, hipStream_t s);

hipError_t launch_compress_mx4(const void* x, int64_t x_sb, int64_t x_st, const float* z,
                               int64_t z_sb, void* out, int64_t o_sb, int64_t o_sj,
                               uint8_t* codes, int64_t c_sb, int64_t c_sj, uint8_t* scales,
                               int64_t s_sb, int64_t s_sj, csa_dtype_t dt, int B, int n, int C,
                               int D_mx, int m, hipStream_t s);
hipError_t launch_compress_append(const void* x, int64_t x_sb, int64_t x_st, int x_rows,
                                  const float* z, int64_t z_sb, const int32_t* t_new, void* cache,
                                  int64_t c_sb, int64_t c_sj, int32_t* n_entries, csa_dtype_t dt,
                                  int B, int C, int m, int N_max, hipStream_t s);

// ---- quantize.hip
hipError_t launch_quantize_mx4(const void* x, int64_t x_rs, csa_dtype_t dt, int rows, int D,
                               uint8_t* codes, int64_t c_rs, uint8_t* scales, int64_t s_rs,
                               hipStream_t s);

// ---- index_score.hip
struct ScoreArgs {
  const void* q;            // [B*Tq, H_I, D_I] (FP4: codes)
  const void* q_scale;      // FP4 only: fp32 (CSA_FP4_E2M1) or E8M0 bytes
  const float* w;           // [B*Tq, H_I]
  const void* k;            // cache base
  const void* k_scale;      // FP4 only: fp32 (CSA_FP4_E2M1) or E8M0 bytes
  int64_t k_sb, k_sn, ks_sb, ks_sn;
  const int32_t* q_pos;
  const int32_t* n_entries;
  int B, Tq, N_max, H, D, m;
  void* scores;             // [B*Tq, s_rs] fp32, or bf16 when score16
  int64_t s_rs;             // row stride of scores (elements)
  float2* chunk_rep;        // [B*Tq, n_chunks] (c-th largest, largest) per chunk, or NULL
  int n_chunks, bound_k;    // bound_k: the k the bounds serve (0: none)
  bool score16;             // bf16 scores (and bf16-rounded reports); score16_supported only
};
hipError_t launch_score(const ScoreArgs& a, csa_dtype_t dt, hipStream_t s);
bool score_supported(csa_dtype_t dt, int H, int D);
bool score_tuned(csa_dtype_t dt, int H, int D);   // writes chunk bounds
bool score16_supported(csa_dtype_t dt, int H, int D);
int score_chunk_keys();                            // keys per bound chunk

// ---- topk.hip
// Selection from rows of N_max scores.  chunk_rep (nullable): per-row chunk
// reports written by the tuned score kernels (one per 256-key chunk, n_chunks
// per row, for the same k); they are used when topk_bounded_ok(N_max), with
// a workspace of topk_bounded_workspace_bytes (zero for rows that one
// workgroup per row streams) and, for few long rows, topk_sync_bytes() of
// counters at `sync` (zero before the call; every call leaves them zero).
// Otherwise the workspace is topk_workspace_bytes and sync is unused.
size_t topk_workspace_bytes(int rows, int N_max, int k);
bool topk_bounded_ok(int N_max);
size_t topk_bounded_workspace_bytes(int rows, int N_max);
size_t topk_sync_bytes();
bool topk_supported(int N_max, int k);
// score16: bf16 score rows (chunk_rep required and topk_bounded_ok(N_max)).
hipError_t launch_topk(const void* scores, bool score16, int64_t s_rs, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                       const float2* chunk_rep, int n_chunks, int32_t* idx,
                       float* out_scores, void* ws, uint32_t* sync, hipStream_t s);

// ---- attend.hip
struct AttendArgs {
  const void* q;            // [B*Tq, H, D]
  const void* kc;           // cache bases
  const void* vc;
  int64_t kv_sb, kv_sn;
  const int32_t* idx;       // CSA: [B*Tq, k]; HCA: NULL
  const int32_t* q_pos;     // HCA: [B*Tq]
  const int32_t* n_entries; // [B]
  int B, Tq, H, D, N_max, topk, m;
  int win;                  // HCA only: attend the last win visible entries (0: all)
  float scale;
  void* out;
  float* lse;
  void* ws;                 // workspace: merge counters (fixed block) then partials
  int32_t* sync = nullptr;  // or explicit counters (attend_sync_block_bytes(rows), zero)
  float* part = nullptr;    // and partials (attend_part_bytes)
};
constexpr int kAttendMaxRows = 65536;   // B * Tq of the tuned kernels (the grid's y extent)
// k_or_nmax: k (CSA), N_max (HCA) or min(window, N_max) (HCA with a window);
// win: that min(window, N_max) for a windowed call, else 0.
// The tuned path's workspace starts with merge counters that must be zero
// before a call; every call leaves them zero.
size_t attend_workspace_bytes(csa_dtype_t dt, bool hca, int B, int Tq, int H, int D, int k_or_nmax,
                              int win = 0);
bool attend_rows_ok(int B, int Tq);   // B * Tq within the tuned kernels' row limit
// Explicit layout (AttendArgs::sync / part): counters for `rows` query rows
// and the split partials of the tuned path (both 0 for the generic path).
size_t attend_sync_block_bytes(int rows);
size_t attend_part_bytes(csa_dtype_t dt, bool hca, int B, int Tq, int H, int D, int k_or_nmax,
                         int win = 0);

bool attend_supported(csa_dtype_t dt, int H, int D);
hipError_t launch_attend(const AttendArgs& a, csa_dtype_t dt, bool hca, hipStream_t s);
// (o, lse) of two disjoint key sets -> the attention over their union
hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb,
                        csa_dtype_t dt, int rows, int H, int D, void* out, float* lse_out,
                        hipStream_t s);

}  // namespace csa
