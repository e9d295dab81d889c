// C ABI of the CSA / HCA library: argument validation, workspace layout and
// dispatch to the kernels.  Every check runs on the host before anything is
// enqueued; a failed check leaves the outputs untouched.
#include <stdarg.h>
#include <atomic>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "csa.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(csa_dtype_t dt) { return dt == CSA_F32 ? 4 : 2; }

bool valid_dtype(csa_dtype_t dt) {
  return dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_FP4_E2M1 || dt == CSA_FP4_E2M1_E8M0;
}
bool is_fp4(csa_dtype_t dt) { return dt == CSA_FP4_E2M1 || dt == CSA_FP4_E2M1_E8M0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// padded row length of the score matrix kept in a workspace (16-byte rows)
int64_t score_row_stride(int N_max) { return (static_cast<int64_t>(N_max) + 3) / 4 * 4; }

#define CSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

csa_status_t check_score_args(const void* q_idx, const void* q_scale, const float* w_idx,
                              const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                              int64_t ks_sb, int64_t ks_sn, csa_dtype_t dt, const int32_t* q_pos,
                              const int32_t* n_entries, int B, int Tq, int N_max, int H_I, int D_I,
                              int m) {
  CSA_REQUIRE(q_idx && w_idx && k_idx && q_pos && n_entries, CSA_ERR_INVALID_ARGUMENT,
              "index score: NULL input pointer");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && N_max >= 1 && H_I >= 1 && D_I >= 1 && m >= 1,
              CSA_ERR_INVALID_ARGUMENT, "index score: sizes must be >= 1");
  CSA_REQUIRE(valid_dtype(dt), CSA_ERR_INVALID_ARGUMENT, "index score: unknown dtype %d", (int)dt);
  CSA_REQUIRE(csa::score_supported(dt, H_I, D_I), CSA_ERR_UNSUPPORTED,
              "index score: dtype %d with H_I=%d D_I=%d not supported", (int)dt, H_I, D_I);
  CSA_REQUIRE(aligned16(q_idx) && aligned16(k_idx) && aligned16(w_idx), CSA_ERR_INVALID_ARGUMENT,
              "index score: pointers must be 16-byte aligned");
  if (is_fp4(dt)) {
    CSA_REQUIRE(q_scale && k_scale, CSA_ERR_INVALID_ARGUMENT, "index score: FP4 needs scales");
    if (dt == CSA_FP4_E2M1)
      CSA_REQUIRE(aligned16(q_scale) && aligned16(k_scale), CSA_ERR_INVALID_ARGUMENT,
                  "index score: fp32 scale pointers must be 16-byte aligned");
    else
      CSA_REQUIRE(aligned4(q_scale) && aligned4(k_scale), CSA_ERR_INVALID_ARGUMENT,
                  "index score: E8M0 scale pointers must be 4-byte aligned");
    CSA_REQUIRE(k_sn >= D_I / 2 && k_sn % 16 == 0 && k_sb % 16 == 0 &&
                    k_sb >= static_cast<int64_t>(N_max) * k_sn,
                CSA_ERR_INVALID_ARGUMENT, "index score: bad FP4 code strides");
    CSA_REQUIRE(ks_sn >= D_I / 32 && ks_sn % 4 == 0 && ks_sb % 4 == 0 &&
                    ks_sb >= static_cast<int64_t>(N_max) * ks_sn,
                CSA_ERR_INVALID_ARGUMENT, "index score: bad FP4 scale strides");
  } else {
    const int64_t vec = 16 / static_cast<int64_t>(esize(dt));
    CSA_REQUIRE(k_sn >= D_I && k_sn % vec == 0 && k_sb % vec == 0 &&
                    (B == 1 || k_sb >= static_cast<int64_t>(N_max) * k_sn),
                CSA_ERR_INVALID_ARGUMENT, "index score: bad key strides (k_sb=%lld k_sn=%lld)",
                (long long)k_sb, (long long)k_sn);
  }
  return CSA_OK;
}

// Chunk reports written by the tuned score kernels: one per 256-key chunk of a
// row, the c-th largest and the largest score of the chunk (see topk.hip).
int bound_chunks(int N_max) {
  return (N_max + csa::score_chunk_keys() - 1) / csa::score_chunk_keys();
}
// The k the score kernel's chunk bounds serve, or 0 when no bounds are used
// (untuned score shape, or rows too long for the bounded selection).
int bound_k(csa_dtype_t dt, int H_I, int D_I, int N_max, int k) {
  return csa::score_tuned(dt, H_I, D_I) && csa::topk_bounded_ok(N_max) ? k : 0;
}

// selection counters (fixed size, zero between calls) | scores | chunk bounds
// | selection workspace
size_t sel_sync_bytes() { return round_up(csa::topk_sync_bytes()); }
size_t index_topk_ws_bytes(int B, int Tq, int N_max, size_t topk_ws, size_t score_bytes) {
  const size_t rows = static_cast<size_t>(B) * Tq;
  const size_t bws = csa::topk_bounded_workspace_bytes(static_cast<int>(rows), N_max);
  return sel_sync_bytes() + round_up(rows * score_row_stride(N_max) * score_bytes) +
         round_up(rows * bound_chunks(N_max) * sizeof(float2)) +
         round_up(topk_ws > bws ? topk_ws : bws);
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(csa_status_t st) {
  switch (st) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARGUMENT: return "CSA_ERR_INVALID_ARGUMENT";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE_TOO_SMALL: return "CSA_ERR_WORKSPACE_TOO_SMALL";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
  }
  return "CSA_ERR_UNKNOWN";
}

const char* csa_last_error(void) { return g_err; }

csa_status_t csa_compress(const void* x, int64_t x_sb, int64_t x_st, const float* logits,
                          int64_t z_sb, void* out, int64_t o_sb, int64_t o_sj, csa_dtype_t dtype,
                          int B, int n, int C, int m, hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(x && logits && out, CSA_ERR_INVALID_ARGUMENT, "compress: NULL pointer");
  CSA_REQUIRE(B >= 1 && n >= 1 && C >= 1 && m >= 1, CSA_ERR_INVALID_ARGUMENT,
              "compress: sizes must be >= 1");
  CSA_REQUIRE(m <= 4096, CSA_ERR_UNSUPPORTED, "compress: m=%d > 4096", m);
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "compress: dtype must be F32 or BF16");
  const int64_t es = static_cast<int64_t>(esize(dtype));
  CSA_REQUIRE((C * es) % 16 == 0, CSA_ERR_UNSUPPORTED, "compress: C*elem_size must be a multiple of 16");
  CSA_REQUIRE(C * es / 16 <= 256, CSA_ERR_UNSUPPORTED, "compress: C too large (%d)", C);
  CSA_REQUIRE(aligned16(x) && aligned16(out), CSA_ERR_INVALID_ARGUMENT,
              "compress: pointers must be 16-byte aligned");
  CSA_REQUIRE((x_st * es) % 16 == 0 && (x_sb * es) % 16 == 0 && (o_sj * es) % 16 == 0 &&
                  (o_sb * es) % 16 == 0,
              CSA_ERR_INVALID_ARGUMENT, "compress: strides must be multiples of 16 bytes");
  CSA_REQUIRE(x_st >= C && o_sj >= C && z_sb >= n, CSA_ERR_INVALID_ARGUMENT,
              "compress: strides smaller than the rows");
  return hip_status(csa::launch_compress(x, x_sb, x_st, logits, z_sb, out, o_sb, o_sj, dtype, B,
                                         n, C, m, stream),
                    "compress launch");
}

csa_status_t csa_compress_mx4(const void* x, int64_t x_sb, int64_t x_st, const float* logits,
                              int64_t z_sb, void* out, int64_t o_sb, int64_t o_sj, uint8_t* codes,
                              int64_t c_sb, int64_t c_sj, uint8_t* scales, int64_t s_sb,
                              int64_t s_sj, csa_dtype_t dtype, int B, int n, int C, int D_mx, int m,
                              hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(x && logits && codes && scales && (out || D_mx == C), CSA_ERR_INVALID_ARGUMENT,
              "compress mx4: NULL pointer");
  CSA_REQUIRE(B >= 1 && n >= 1 && C >= 1 && m >= 1, CSA_ERR_INVALID_ARGUMENT,
              "compress mx4: sizes must be >= 1");
  CSA_REQUIRE(D_mx >= 32 && D_mx % 32 == 0 && D_mx <= C && (C - D_mx) % 32 == 0,
              CSA_ERR_INVALID_ARGUMENT,
              "compress mx4: D_mx must be a positive multiple of 32, at most C, with C - D_mx a "
              "multiple of 32");
  CSA_REQUIRE(m <= 4096, CSA_ERR_UNSUPPORTED, "compress mx4: m=%d > 4096", m);
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "compress mx4: dtype must be F32 or BF16");
  const int64_t es = static_cast<int64_t>(esize(dtype));
  CSA_REQUIRE(C * es / 16 <= 256, CSA_ERR_UNSUPPORTED, "compress mx4: C too large (%d)", C);
  CSA_REQUIRE(aligned16(x) && (out == nullptr || aligned16(out)), CSA_ERR_INVALID_ARGUMENT,
              "compress mx4: x and out must be 16-byte aligned");
  const int64_t cw = dtype == CSA_BF16 ? 4 : 2;   // code bytes written per thread
  CSA_REQUIRE(reinterpret_cast<uintptr_t>(codes) % cw == 0 && c_sj % cw == 0 && c_sb % cw == 0,
              CSA_ERR_INVALID_ARGUMENT, "compress mx4: codes must be %lld-byte aligned",
              static_cast<long long>(cw));
  CSA_REQUIRE((x_st * es) % 16 == 0 && (x_sb * es) % 16 == 0 && (o_sj * es) % 16 == 0 &&
                  (o_sb * es) % 16 == 0,
              CSA_ERR_INVALID_ARGUMENT, "compress mx4: strides must be multiples of 16 bytes");
  CSA_REQUIRE(x_st >= C && z_sb >= n && c_sj >= D_mx / 2 && s_sj >= D_mx / 32 &&
                  (D_mx == C || o_sj >= C - D_mx),
              CSA_ERR_INVALID_ARGUMENT, "compress mx4: strides smaller than the rows");
  return hip_status(csa::launch_compress_mx4(x, x_sb, x_st, logits, z_sb, out, o_sb, o_sj, codes,
                                             c_sb, c_sj, scales, s_sb, s_sj, dtype, B, n, C, D_mx,
                                             m, stream),
                    "compress mx4 launch");
}

csa_status_t csa_compress_append(const void* x, int64_t x_sb, int64_t x_st, int x_rows,
                                 const float* logits, int64_t z_sb, const int32_t* t_new,
                                 void* cache, int64_t c_sb, int64_t c_sj, int32_t* n_entries,
                                 csa_dtype_t dtype, int B, int C, int m, int N_max,
                                 hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(x && logits && t_new && cache && n_entries, CSA_ERR_INVALID_ARGUMENT,
              "compress append: NULL pointer");
  CSA_REQUIRE(B >= 1 && C >= 1 && m >= 1 && N_max >= 1 && x_rows >= m && x_rows % m == 0,
              CSA_ERR_INVALID_ARGUMENT,
              "compress append: sizes must be >= 1 and x_rows a positive multiple of m");
  CSA_REQUIRE(m <= 4096, CSA_ERR_UNSUPPORTED, "compress append: m=%d > 4096", m);
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "compress append: dtype must be F32 or BF16");
  const int64_t es = static_cast<int64_t>(esize(dtype));
  CSA_REQUIRE((C * es) % 16 == 0 && C * es / 16 <= 256, CSA_ERR_UNSUPPORTED,
              "compress append: C*elem_size must be a multiple of 16 and at most 4096 bytes");
  CSA_REQUIRE(aligned16(x) && aligned16(cache), CSA_ERR_INVALID_ARGUMENT,
              "compress append: pointers must be 16-byte aligned");
  CSA_REQUIRE((x_st * es) % 16 == 0 && (x_sb * es) % 16 == 0 && (c_sj * es) % 16 == 0 &&
                  (c_sb * es) % 16 == 0,
              CSA_ERR_INVALID_ARGUMENT, "compress append: strides must be multiples of 16 bytes");
  CSA_REQUIRE(x_st >= C && c_sj >= C && z_sb >= x_rows, CSA_ERR_INVALID_ARGUMENT,
              "compress append: strides smaller than the rows");
  return hip_status(csa::launch_compress_append(x, x_sb, x_st, x_rows, logits, z_sb, t_new, cache,
                                                c_sb, c_sj, n_entries, dtype, B, C, m, N_max,
                                                stream),
                    "compress append launch");
}

csa_status_t csa_attend_merge(const void* o_a, const float* lse_a, const void* o_b,
                              const float* lse_b, csa_dtype_t dtype, int rows, int H, int D,
                              void* out, float* lse_out, hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(o_a && lse_a && o_b && lse_b && out, CSA_ERR_INVALID_ARGUMENT,
              "attend merge: NULL pointer");
  CSA_REQUIRE(rows >= 1 && H >= 1 && D >= 8 && D % 8 == 0, CSA_ERR_INVALID_ARGUMENT,
              "attend merge: need rows, H >= 1 and D a positive multiple of 8");
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "attend merge: dtype must be F32 or BF16");
  CSA_REQUIRE(aligned16(o_a) && aligned16(o_b) && aligned16(out), CSA_ERR_INVALID_ARGUMENT,
              "attend merge: outputs must be 16-byte aligned");
  return hip_status(csa::launch_merge(o_a, lse_a, o_b, lse_b, dtype, rows, H, D, out, lse_out,
                                      stream),
                    "attend merge launch");
}

csa_status_t csa_quantize_mx4(const void* x, int64_t x_rs, csa_dtype_t dtype, int rows, int D,
                              uint8_t* codes, int64_t c_rs, uint8_t* scales, int64_t s_rs,
                              hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(x && codes && scales, CSA_ERR_INVALID_ARGUMENT, "quantize mx4: NULL pointer");
  CSA_REQUIRE(rows >= 1 && D >= 32 && D % 32 == 0, CSA_ERR_INVALID_ARGUMENT,
              "quantize mx4: need rows >= 1 and D a positive multiple of 32");
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "quantize mx4: dtype must be F32 or BF16");
  const int64_t es = static_cast<int64_t>(esize(dtype));
  CSA_REQUIRE(aligned16(x) && aligned16(codes) && (x_rs * es) % 16 == 0 && c_rs % 16 == 0,
              CSA_ERR_INVALID_ARGUMENT, "quantize mx4: x and codes must be 16-byte aligned rows");
  CSA_REQUIRE(x_rs >= D && c_rs >= D / 2 && s_rs >= D / 32, CSA_ERR_INVALID_ARGUMENT,
              "quantize mx4: row strides smaller than the rows");
  return hip_status(csa::launch_quantize_mx4(x, x_rs, dtype, rows, D, codes, c_rs, scales, s_rs,
                                             stream),
                    "quantize mx4 launch");
}

csa_status_t csa_index_score(const void* q_idx, const void* q_scale, const float* w_idx,
                             const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                             int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                             const int32_t* q_pos, const int32_t* n_entries, int B, int Tq,
                             int N_max, int H_I, int D_I, int m, float* scores,
                             hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_score_args(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb,
                                     ks_sn, idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, m);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(scores, CSA_ERR_INVALID_ARGUMENT, "index score: NULL scores");
  csa::ScoreArgs a{q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                   q_pos, n_entries, B, Tq, N_max, H_I, D_I, m, scores, N_max,
                   nullptr, 0, 0, false};
  return hip_status(csa::launch_score(a, idx_dtype, stream), "index score launch");
}

csa_status_t csa_topk_workspace(int B, int Tq, int N_max, int k, size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "topk workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && N_max >= 1 && k >= 1, CSA_ERR_INVALID_ARGUMENT,
              "topk workspace: sizes must be >= 1");
  CSA_REQUIRE(csa::topk_supported(N_max, k), CSA_ERR_UNSUPPORTED,
              "topk: N_max=%d with k=%d not supported", N_max, k);
  *bytes = csa::topk_workspace_bytes(B * Tq, N_max, k);
  return CSA_OK;
}

csa_status_t csa_topk(const float* scores, int64_t s_rs, const int32_t* q_pos,
                      const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                      int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  g_err[0] = 0;
  CSA_REQUIRE(scores && q_pos && n_entries && topk_idx, CSA_ERR_INVALID_ARGUMENT,
              "topk: NULL pointer");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && N_max >= 1 && m >= 1 && k >= 1, CSA_ERR_INVALID_ARGUMENT,
              "topk: sizes must be >= 1");
  CSA_REQUIRE(s_rs >= N_max && s_rs % 4 == 0 && aligned16(scores), CSA_ERR_INVALID_ARGUMENT,
              "topk: score rows must be 16-byte aligned and hold N_max values");
  CSA_REQUIRE(csa::topk_supported(N_max, k), CSA_ERR_UNSUPPORTED,
              "topk: N_max=%d with k=%d not supported", N_max, k);
  const size_t need = csa::topk_workspace_bytes(B * Tq, N_max, k);
  CSA_REQUIRE(ws_bytes >= need && (need == 0 || ws), CSA_ERR_WORKSPACE_TOO_SMALL,
              "topk: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(csa::launch_topk(scores, false, s_rs, q_pos, n_entries, B, Tq, N_max, m, k,
                                     nullptr, 0, topk_idx, topk_score, ws, nullptr, stream),
                    "topk launch");
}

csa_status_t csa_index_topk_workspace(int B, int Tq, int N_max, int k, size_t* bytes) {
  g_err[0] = 0;
  size_t t = 0;
  csa_status_t st = csa_topk_workspace(B, Tq, N_max, k, &t);
  if (st != CSA_OK) return st;
  *bytes = index_topk_ws_bytes(B, Tq, N_max, t, sizeof(float));
  return CSA_OK;
}

csa_status_t csa_index_topk_bf16_workspace(int B, int Tq, int N_max, int k, size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "index topk bf16 workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && N_max >= 1 && k >= 1, CSA_ERR_INVALID_ARGUMENT,
              "index topk bf16 workspace: sizes must be >= 1");
  CSA_REQUIRE(csa::topk_bounded_ok(N_max) && csa::topk_supported(N_max, k), CSA_ERR_UNSUPPORTED,
              "index topk bf16: N_max=%d with k=%d not supported", N_max, k);
  *bytes = index_topk_ws_bytes(B, Tq, N_max, 0, sizeof(uint16_t));
  return CSA_OK;
}

}  // extern "C"

namespace {

// Workspace of the index + top-k pair: score rows | chunk reports | selection.
struct IndexWs {
  void* scores;
  int64_t srs;
  float2* bounds;                 // NULL when the score kernel writes no reports
  int n_chunks;
  void* sel_ws;
};

// Lays out the workspace after its selection counters (scores | chunk
// bounds | selection workspace from ws) and launches the score kernel (with
// chunk reports when the bounded selection will use them).
csa_status_t launch_index_scores(const void* q_idx, const void* q_scale, const float* w_idx,
                                 const void* k_idx, const void* k_scale, int64_t k_sb,
                                 int64_t k_sn, int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                                 const int32_t* q_pos, const int32_t* n_entries, int B, int Tq,
                                 int N_max, int H_I, int D_I, int m, int k, void* ws, bool score16,
                                 hipStream_t stream, IndexWs& iw) {
  const int64_t srs = score_row_stride(N_max);
  const size_t rows = static_cast<size_t>(B) * Tq;
  char* base = static_cast<char*>(ws);
  iw.scores = base;
  iw.srs = srs;
  base += round_up(rows * srs * (score16 ? sizeof(uint16_t) : sizeof(float)));
  iw.n_chunks = bound_chunks(N_max);
  const int bk = bound_k(idx_dtype, H_I, D_I, N_max, k);
  iw.bounds = bk > 0 ? reinterpret_cast<float2*>(base) : nullptr;
  base += round_up(rows * iw.n_chunks * sizeof(float2));
  iw.sel_ws = base;
  csa::ScoreArgs a{q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                   q_pos, n_entries, B, Tq, N_max, H_I, D_I, m, iw.scores, srs,
                   iw.bounds, iw.n_chunks, bk, score16};
  return hip_status(csa::launch_score(a, idx_dtype, stream), "index score launch");
}

// Shared body of csa_index_topk (fp32 score rows) and csa_index_topk_bf16.
csa_status_t index_topk_impl(const void* q_idx, const void* q_scale, const float* w_idx,
                             const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                             int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                             const int32_t* q_pos, const int32_t* n_entries, int B, int Tq,
                             int N_max, int H_I, int D_I, int m, int k, int32_t* topk_idx,
                             float* topk_score, void* ws, size_t ws_bytes, hipStream_t stream,
                             bool score16) {
  csa_status_t st = check_score_args(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb,
                                     ks_sn, idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, m);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(topk_idx && k >= 1, CSA_ERR_INVALID_ARGUMENT, "index topk: bad output / k");
  if (score16)
    CSA_REQUIRE(csa::score16_supported(idx_dtype, H_I, D_I), CSA_ERR_UNSUPPORTED,
                "index topk bf16: needs the BF16 64 x 128 indexer (dtype %d, H_I=%d, D_I=%d)",
                static_cast<int>(idx_dtype), H_I, D_I);
  size_t need = 0;
  st = score16 ? csa_index_topk_bf16_workspace(B, Tq, N_max, k, &need)
               : csa_index_topk_workspace(B, Tq, N_max, k, &need);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ws && ws_bytes >= need && aligned16(ws), CSA_ERR_WORKSPACE_TOO_SMALL,
              "index topk: workspace %zu < %zu bytes (or misaligned)", ws_bytes, need);
  IndexWs iw;
  st = launch_index_scores(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                           idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, m, k,
                           static_cast<char*>(ws) + sel_sync_bytes(), score16, stream, iw);
  if (st != CSA_OK) return st;
  return hip_status(csa::launch_topk(iw.scores, score16, iw.srs, q_pos, n_entries, B, Tq, N_max, m,
                                     k, iw.bounds, iw.n_chunks, topk_idx, topk_score, iw.sel_ws,
                                     static_cast<uint32_t*>(ws), stream),
                    "topk launch");
}

}  // namespace

extern "C" {

csa_status_t csa_index_topk(const void* q_idx, const void* q_scale, const float* w_idx,
                            const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                            int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                            const int32_t* q_pos, const int32_t* n_entries, int B, int Tq,
                            int N_max, int H_I, int D_I, int m, int k, int32_t* topk_idx,
                            float* topk_score, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  return index_topk_impl(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                         idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, m, k, topk_idx,
                         topk_score, ws, ws_bytes, stream, false);
}

csa_status_t csa_index_topk_bf16(const void* q_idx, const float* w_idx, const void* k_idx,
                                 int64_t k_sb, int64_t k_sn, const int32_t* q_pos,
                                 const int32_t* n_entries, int B, int Tq, int N_max, int m, int k,
                                 int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  g_err[0] = 0;
  return index_topk_impl(q_idx, nullptr, w_idx, k_idx, nullptr, k_sb, k_sn, 0, 0, CSA_BF16, q_pos,
                         n_entries, B, Tq, N_max, 64, 128, m, k, topk_idx, topk_score, ws,
                         ws_bytes, stream, true);
}

static csa_status_t check_attend(const void* q, const void* k_c, const void* v_c, int64_t kv_sb,
                                 int64_t kv_sn, const int32_t* n_entries, csa_dtype_t dtype, int B,
                                 int Tq, int H, int D, int N_max, void* out) {
  CSA_REQUIRE(q && k_c && v_c && n_entries && out, CSA_ERR_INVALID_ARGUMENT,
              "attend: NULL pointer");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1 && D >= 1 && N_max >= 1, CSA_ERR_INVALID_ARGUMENT,
              "attend: sizes must be >= 1");
  CSA_REQUIRE(csa::attend_rows_ok(B, Tq), CSA_ERR_UNSUPPORTED,
              "attend: B*Tq=%lld query rows exceed 65536", static_cast<long long>(B) * Tq);
  CSA_REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED,
              "attend: dtype must be F32 or BF16");
  CSA_REQUIRE(csa::attend_supported(dtype, H, D), CSA_ERR_UNSUPPORTED,
              "attend: H=%d D=%d not supported", H, D);
  CSA_REQUIRE(aligned16(q) && aligned16(k_c) && aligned16(v_c) && aligned16(out),
              CSA_ERR_INVALID_ARGUMENT, "attend: pointers must be 16-byte aligned");
  const int64_t vec = 16 / static_cast<int64_t>(esize(dtype));
  CSA_REQUIRE(kv_sn >= D && kv_sn % vec == 0 && kv_sb % vec == 0 &&
                  (B == 1 || kv_sb >= static_cast<int64_t>(N_max) * kv_sn),
              CSA_ERR_INVALID_ARGUMENT, "attend: bad cache strides");
  return CSA_OK;
}

csa_status_t csa_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int k,
                                  size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "attend workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1 && D >= 1 && k >= 1, CSA_ERR_INVALID_ARGUMENT,
              "attend workspace: sizes must be >= 1");
  *bytes = csa::attend_workspace_bytes(dtype, false, B, Tq, H, D, k);
  return CSA_OK;
}

csa_status_t csa_attend(const void* q, const void* k_c, const void* v_c, int64_t kv_sb,
                        int64_t kv_sn, const int32_t* topk_idx, const int32_t* n_entries,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int k,
                        float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_attend(q, k_c, v_c, kv_sb, kv_sn, n_entries, dtype, B, Tq, H, D, N_max,
                                 out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(topk_idx && k >= 1, CSA_ERR_INVALID_ARGUMENT, "attend: bad topk_idx / k");
  const size_t need = csa::attend_workspace_bytes(dtype, false, B, Tq, H, D, k);
  CSA_REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned16(ws))),
              CSA_ERR_WORKSPACE_TOO_SMALL, "attend: workspace %zu < %zu bytes", ws_bytes, need);
  csa::AttendArgs a{q, k_c, v_c, kv_sb, kv_sn, topk_idx, nullptr, n_entries, B, Tq, H, D,
                    N_max, k, 1, 0, scale, out, lse, ws};
  return hip_status(csa::launch_attend(a, dtype, false, stream), "attend launch");
}

csa_status_t hca_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max,
                                  size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "hca workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1 && D >= 1 && N_max >= 1, CSA_ERR_INVALID_ARGUMENT,
              "hca workspace: sizes must be >= 1");
  *bytes = csa::attend_workspace_bytes(dtype, true, B, Tq, H, D, N_max);
  return CSA_OK;
}

csa_status_t hca_attend(const void* q, const void* k_c, const void* v_c, int64_t kv_sb,
                        int64_t kv_sn, const int32_t* q_pos, const int32_t* n_entries,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int m,
                        float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_attend(q, k_c, v_c, kv_sb, kv_sn, n_entries, dtype, B, Tq, H, D, N_max,
                                 out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(q_pos && m >= 1, CSA_ERR_INVALID_ARGUMENT, "hca: bad q_pos / m");
  const size_t need = csa::attend_workspace_bytes(dtype, true, B, Tq, H, D, N_max);
  CSA_REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned16(ws))),
              CSA_ERR_WORKSPACE_TOO_SMALL, "hca: workspace %zu < %zu bytes", ws_bytes, need);
  csa::AttendArgs a{q, k_c, v_c, kv_sb, kv_sn, nullptr, q_pos, n_entries, B, Tq, H, D,
                    N_max, 0, m, 0, scale, out, lse, ws};
  return hip_status(csa::launch_attend(a, dtype, true, stream), "hca launch");
}

csa_status_t swa_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max,
                                  int window, size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "swa workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1 && D >= 1 && N_max >= 1 && window >= 1,
              CSA_ERR_INVALID_ARGUMENT, "swa workspace: sizes must be >= 1");
  const int wn = window < N_max ? window : N_max;
  *bytes = csa::attend_workspace_bytes(dtype, true, B, Tq, H, D, wn, wn);
  return CSA_OK;
}

csa_status_t swa_attend(const void* q, const void* k, const void* v, int64_t kv_sb,
                        int64_t kv_sn, const int32_t* q_pos, const int32_t* n_tokens,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int window,
                        float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_attend(q, k, v, kv_sb, kv_sn, n_tokens, dtype, B, Tq, H, D, N_max, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(q_pos && window >= 1, CSA_ERR_INVALID_ARGUMENT, "swa: bad q_pos / window");
  const int wn = window < N_max ? window : N_max;
  const size_t need = csa::attend_workspace_bytes(dtype, true, B, Tq, H, D, wn, wn);
  CSA_REQUIRE(ws_bytes >= need && (need == 0 || (ws && aligned16(ws))),
              CSA_ERR_WORKSPACE_TOO_SMALL, "swa: workspace %zu < %zu bytes", ws_bytes, need);
  csa::AttendArgs a{q, k, v, kv_sb, kv_sn, nullptr, q_pos, n_tokens, B, Tq, H, D,
                    N_max, 0, 1, wn, scale, out, lse, ws};
  return hip_status(csa::launch_attend(a, dtype, true, stream), "swa launch");
}

}  // extern "C"

// ---------------------------------------------------------------- score -> top-k -> attention
namespace {

// Intermediate buffers of one decode step: selection counters and attention
// merge counters for `sync_rows` rows (both fixed in size and place, zero
// before the call, zero after it), attention partials, top-k lists (used when
// the caller passes none), index + top-k workspace.
struct StepSizes {
  size_t sync, part, idx, index;
  size_t total() const { return sync + part + idx + index; }
};
csa_status_t step_sizes(csa_dtype_t dtype, int B, int Tq, int N_max, int H, int D, int k,
                        int sync_rows, StepSizes& z) {
  size_t t = 0;
  csa_status_t st = csa_index_topk_workspace(B, Tq, N_max, k, &t);
  if (st != CSA_OK) return st;
  z.sync = sel_sync_bytes() + round_up(csa::attend_sync_block_bytes(sync_rows));
  z.part = round_up(csa::attend_part_bytes(dtype, false, B, Tq, H, D, k));
  z.idx = round_up(static_cast<size_t>(B) * Tq * k * sizeof(int32_t));
  z.index = t;
  return CSA_OK;
}

csa_status_t check_step(const void* q_idx, const void* q_scale, const float* w_idx,
                        const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                        int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype, const void* q,
                        const void* k_c, const void* v_c, int64_t kv_sb, int64_t kv_sn,
                        csa_dtype_t dtype, const int32_t* q_pos, const int32_t* n_entries, int B,
                        int Tq, int N_max, int H_I, int D_I, int H, int D, int m, int k,
                        void* out) {
  csa_status_t st = check_score_args(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb,
                                     ks_sn, idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, m);
  if (st != CSA_OK) return st;
  st = check_attend(q, k_c, v_c, kv_sb, kv_sn, n_entries, dtype, B, Tq, H, D, N_max, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1, CSA_ERR_INVALID_ARGUMENT, "index topk attend: k must be >= 1");
  CSA_REQUIRE(csa::topk_supported(N_max, k), CSA_ERR_UNSUPPORTED,
              "index topk attend: N_max=%d with k=%d not supported", N_max, k);
  return CSA_OK;
}

// Launches the step on buffers laid out as StepSizes at base (arguments
// already validated).
csa_status_t step_impl(const void* q_idx, const void* q_scale, const float* w_idx,
                       const void* k_idx, const void* k_scale, int64_t k_sb, int64_t k_sn,
                       int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype, const void* q,
                       const void* k_c, const void* v_c, int64_t kv_sb, int64_t kv_sn,
                       csa_dtype_t dtype, const int32_t* q_pos, const int32_t* n_entries, int B,
                       int Tq, int N_max, int H_I, int D_I, int H, int D, int m, int k, float scale,
                       void* out, float* lse, int32_t* topk_idx, const StepSizes& z, char* base,
                       hipStream_t stream) {
  uint32_t* sel_sync = reinterpret_cast<uint32_t*>(base);
  int32_t* sync = reinterpret_cast<int32_t*>(base + sel_sync_bytes());
  float* part = reinterpret_cast<float*>(base + z.sync);
  int32_t* idx_buf = reinterpret_cast<int32_t*>(base + z.sync + z.part);
  void* index_ws = base + z.sync + z.part + z.idx;
  IndexWs iw;
  csa_status_t st = launch_index_scores(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb,
                                        ks_sn, idx_dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I,
                                        m, k, static_cast<char*>(index_ws) + sel_sync_bytes(),
                                        false, stream, iw);
  if (st != CSA_OK) return st;
  int32_t* idx = topk_idx != nullptr ? topk_idx : idx_buf;
  st = hip_status(csa::launch_topk(iw.scores, false, iw.srs, q_pos, n_entries, B, Tq, N_max, m, k,
                                   iw.bounds, iw.n_chunks, idx, nullptr, iw.sel_ws, sel_sync,
                                   stream),
                  "topk launch");
  if (st != CSA_OK) return st;
  csa::AttendArgs a{q, k_c, v_c, kv_sb, kv_sn, idx, nullptr, n_entries, B, Tq, H, D,
                    N_max, k, m, 0, scale, out, lse, nullptr, sync, part};
  return hip_status(csa::launch_attend(a, dtype, false, stream), "attend launch");
}

// ---- the allocation-free variant's scratch
// One file-scope device array per GPU the library runs on, held until the
// process ends.  Host code never uses its name as an address: the device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there and kept in g_scratch_addr.  The
// array is zero when the code object is loaded; the selection and attention
// merge counters at its front are the only part that must be zero before a
// call, and every call leaves them zero.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kScratchRows = 4096;                // B * Tq the counter block serves
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];

csa_status_t scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  CSA_REQUIRE(dev >= 0 && dev < kMaxDevices, CSA_ERR_UNSUPPORTED, "device %d >= %d", dev,
              kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_index_topk_attend_workspace(csa_dtype_t idx_dtype, csa_dtype_t dtype, int B,
                                             int Tq, int N_max, int H, int D, int k,
                                             size_t* bytes) {
  g_err[0] = 0;
  CSA_REQUIRE(bytes, CSA_ERR_INVALID_ARGUMENT, "index topk attend workspace: NULL result");
  CSA_REQUIRE(B >= 1 && Tq >= 1 && N_max >= 1 && H >= 1 && D >= 1 && k >= 1,
              CSA_ERR_INVALID_ARGUMENT, "index topk attend workspace: sizes must be >= 1");
  CSA_REQUIRE(valid_dtype(idx_dtype) && (dtype == CSA_F32 || dtype == CSA_BF16),
              CSA_ERR_INVALID_ARGUMENT, "index topk attend workspace: bad dtype");
  StepSizes z;
  const csa_status_t st = step_sizes(dtype, B, Tq, N_max, H, D, k, csa::kAttendMaxRows, z);
  if (st != CSA_OK) return st;
  *bytes = z.total();
  return CSA_OK;
}

csa_status_t csa_index_topk_attend(const void* q_idx, const void* q_scale, const float* w_idx,
                                   const void* k_idx, const void* k_scale, int64_t k_sb,
                                   int64_t k_sn, int64_t ks_sb, int64_t ks_sn,
                                   csa_dtype_t idx_dtype, const void* q, const void* k_c,
                                   const void* v_c, int64_t kv_sb, int64_t kv_sn,
                                   csa_dtype_t dtype, const int32_t* q_pos,
                                   const int32_t* n_entries, int B, int Tq, int N_max, int H_I,
                                   int D_I, int H, int D, int m, int k, float scale, void* out,
                                   float* lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_step(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                               idx_dtype, q, k_c, v_c, kv_sb, kv_sn, dtype, q_pos, n_entries, B,
                               Tq, N_max, H_I, D_I, H, D, m, k, out);
  if (st != CSA_OK) return st;
  StepSizes z;
  st = step_sizes(dtype, B, Tq, N_max, H, D, k, csa::kAttendMaxRows, z);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ws && ws_bytes >= z.total() && aligned16(ws), CSA_ERR_WORKSPACE_TOO_SMALL,
              "index topk attend: workspace %zu < %zu bytes (or misaligned)", ws_bytes, z.total());
  return step_impl(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn, idx_dtype, q,
                   k_c, v_c, kv_sb, kv_sn, dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, H, D,
                   m, k, scale, out, lse, topk_idx, z, static_cast<char*>(ws), stream);
}

size_t csa_index_topk_attend_noalloc_max_bytes(void) { return kScratchBytes; }

csa_status_t csa_index_topk_attend_noalloc(const void* q_idx, const void* q_scale,
                                           const float* w_idx, const void* k_idx,
                                           const void* k_scale, int64_t k_sb, int64_t k_sn,
                                           int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                                           const void* q, const void* k_c, const void* v_c,
                                           int64_t kv_sb, int64_t kv_sn, csa_dtype_t dtype,
                                           const int32_t* q_pos, const int32_t* n_entries, int B,
                                           int Tq, int N_max, int H_I, int D_I, int H, int D,
                                           int m, int k, float scale, void* out, float* lse,
                                           int32_t* topk_idx, hipStream_t stream) {
  g_err[0] = 0;
  csa_status_t st = check_step(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn,
                               idx_dtype, q, k_c, v_c, kv_sb, kv_sn, dtype, q_pos, n_entries, B,
                               Tq, N_max, H_I, D_I, H, D, m, k, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(static_cast<long long>(B) * Tq <= kScratchRows, CSA_ERR_UNSUPPORTED,
              "index topk attend noalloc: B*Tq=%lld > %d query rows", static_cast<long long>(B) * Tq,
              kScratchRows);
  StepSizes z;
  st = step_sizes(dtype, B, Tq, N_max, H, D, k, kScratchRows, z);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(z.total() <= kScratchBytes, CSA_ERR_UNSUPPORTED,
              "index topk attend noalloc: needs %zu bytes of scratch, the maximum is %zu",
              z.total(), kScratchBytes);
  void* base = nullptr;
  st = scratch_address(&base);
  if (st != CSA_OK) return st;
  return step_impl(q_idx, q_scale, w_idx, k_idx, k_scale, k_sb, k_sn, ks_sb, ks_sn, idx_dtype, q,
                   k_c, v_c, kv_sb, kv_sn, dtype, q_pos, n_entries, B, Tq, N_max, H_I, D_I, H, D,
                   m, k, scale, out, lse, topk_idx, z, static_cast<char*>(base), stream);
}

}  // extern "C"
