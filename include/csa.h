/*
 * csa.h - Compressed Sparse Attention (CSA) and Heavily Compressed Attention
 * (HCA) on AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * The method is the one described in the technical review
 * "DeepSeek V4 技术解读" (takeshell.com):
 *   §2.1 CSA  - merge the KV entries of every m tokens into one compressed
 *               entry by weighted aggregation; a Lightning Indexer scores each
 *               query token's indexer queries against the compressed entries
 *               and keeps the top-k; core attention runs over those k only.
 *               V4-Pro: m = 4, 64 indexer heads x 128 dims, top-k = 1024.
 *   §2.2 HCA  - m' = 128 tokens per entry, dense attention over all entries.
 *   §5        - the indexer QK path may run in FP4 E2M1, dequantised to
 *               FP8 E4M3 without loss.
 *   §6.2      - kernels are batch invariant: a token's result is bitwise the
 *               same wherever it sits in a batch; no floating-point atomics.
 *
 * Readings of points the pages leave open (all implemented exactly so):
 *   - pooling weights: softmax of one fp32 logit per raw token within its
 *     block; the same weights pool every channel of the row (K, V, K_I).
 *   - one shared KV head (K and V separate arrays) for all query heads; one
 *     shared indexer key per compressed entry.
 *   - index score s(t,j) = sum_h w[t,h] * max(0, q_I[t,h] . k_I[j]), unscaled,
 *     fp32 accumulation.
 *   - causality: entry j is visible to a query at position t iff
 *     m * (j + 1) <= t + 1, i.e. V(t) = min(n_entries[b], floor((t+1)/m)).
 *   - top-k: order (score descending, index ascending), -0.0 == +0.0, keep
 *     min(k, V(t)); indices returned ascending, padded with -1.  One set per
 *     query token, shared by all heads.
 *   - attention: softmax(scale * q . k) over the set; an empty set gives
 *     output 0 and lse -inf.  lse is the natural-log log-sum-exp.
 *   - FP4: E2M1 codes, element 2i in the low nibble of byte i, one fp32
 *     scale per 32 consecutive elements of a vector.
 *   - MX FP4 (a variant of §5's FP4 path): the same codes with one E8M0
 *     scale byte per 32 elements, as in the OCP Microscaling formats; such
 *     power-of-two scales keep FP4 -> FP8 E4M3 exact (the pages' condition
 *     that the scale stay within range) and gfx950's block-scaled MFMA
 *     applies them itself.
 *
 * Conventions for every call
 *   - All data pointers are DEVICE memory owned by the caller.  The library
 *     allocates and frees nothing and keeps no state between calls besides
 *     loaded kernel code; calls are thread-safe.
 *   - Calls only enqueue work on `stream` and return; results are valid once
 *     the stream has reached that point.  No call synchronises.
 *   - Tensors are row-major with the last dimension contiguous.  Strides are
 *     given in ELEMENTS of the tensor's storage type (bytes for FP4 codes).
 *     Pointers and row strides must be 16-byte aligned.
 *   - Validation happens on the host before anything is enqueued; a failed
 *     check returns a status, enqueues nothing and leaves outputs untouched.
 *     A failed launch returns CSA_ERR_HIP.  csa_last_error() gives a message
 *     for the calling thread's last failure.  Nothing aborts or throws.
 *   - Outputs must not alias inputs.  Overlapping calls on one stream are
 *     ordered by the stream; workspaces must not be shared by calls that may
 *     run concurrently.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad size, misalignment   */
  CSA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (shape/dtype) */
  CSA_ERR_WORKSPACE_TOO_SMALL = 3,
  CSA_ERR_HIP = 4                 /* a HIP launch failed                     */
} csa_status_t;

typedef enum {
  CSA_F32 = 0,        /* float32                                           */
  CSA_BF16 = 1,       /* bfloat16 (uint16 bit patterns)                    */
  CSA_FP4_E2M1 = 2,   /* packed E2M1 codes + one fp32 scale per 32 values  */
  CSA_FP4_E2M1_E8M0 = 3 /* packed E2M1 codes + one E8M0 scale byte per 32
                           values (MX FP4: value = code * 2^(byte - 127))  */
} csa_dtype_t;

int csa_abi_version(void);
const char* csa_status_string(csa_status_t status);
/* Message of the calling thread's most recent non-OK status ("" if none). */
const char* csa_last_error(void);

/*
 * csa_compress - token-dimension compression (§2.1 "KV cache compression",
 * §2.2 with m' = 128).
 *
 *   out[b, j, c] = sum_{i<m} w_i x[b, m*j + i, c],
 *   w = softmax(logits[b, m*j .. m*j+m-1])       for j < n / m, every c < C.
 *
 * x       [B, n, C] dtype, strides (x_sb, x_st) elements, channel stride 1.
 * logits  [B, n] fp32, batch stride z_sb, token stride 1.
 * out     [B, n/m, C] dtype, strides (o_sb, o_sj).
 * dtype   CSA_F32 or CSA_BF16 (x and out).  Math in fp32; bf16 output is
 *         rounded to nearest even.
 * Only complete blocks are produced; a tail of n % m tokens is ignored.
 * Requires B, n, C, m >= 1, m <= 4096, C * sizeof(dtype) a multiple of 16.
 */
csa_status_t csa_compress(const void* x, int64_t x_sb, int64_t x_st,
                          const float* logits, int64_t z_sb,
                          void* out, int64_t o_sb, int64_t o_sj,
                          csa_dtype_t dtype, int B, int n, int C, int m,
                          hipStream_t stream);

/*
 * csa_compress_mx4 - csa_compress with the trailing D_mx channels of every
 * entry (the indexer key) stored as MX FP4 instead of dtype (§2.1
 * compression and §5's FP4 indexer QK path in one pass: the key is encoded
 * from its fp32 pooled value, the format CSA_FP4_E2M1_E8M0 consumes).
 *
 *   channels c < C - D_mx: out[b, j, c] as csa_compress writes it;
 *   channels C - D_mx .. C - 1: the pooled fp32 values v encoded per block of
 *   32 as csa_quantize_mx4 encodes them (shared exponent e from the block's
 *   largest |v|, codes = nearest E2M1 of v / 2^e): codes[b, j, D_mx/2]
 *   (element 2i in the low nibble of byte i), scales[b, j, D_mx/32] (e + 127).
 *
 * x, logits, dtype, B, n, C, m and their strides as in csa_compress; out
 * [B, n/m, C - D_mx] (strides o_sb, o_sj; NULL allowed when D_mx == C);
 * codes with strides (c_sb, c_sj) bytes, 4-byte aligned (2 for CSA_F32);
 * scales with strides (s_sb, s_sj) bytes.  D_mx and C - D_mx multiples of 32.
 */
csa_status_t csa_compress_mx4(const void* x, int64_t x_sb, int64_t x_st,
                              const float* logits, int64_t z_sb,
                              void* out, int64_t o_sb, int64_t o_sj,
                              uint8_t* codes, int64_t c_sb, int64_t c_sj,
                              uint8_t* scales, int64_t s_sb, int64_t s_sj,
                              csa_dtype_t dtype, int B, int n, int C, int D_mx, int m,
                              hipStream_t stream);

/*
 * csa_compress_append - incremental compression during decoding (§2.1 KV
 * cache compression applied as tokens arrive: a compressed entry is formed
 * once its m tokens are all present).
 *
 * For each sequence b, token t = t_new[b] (0-based position) has just been
 * added.  When it completes a block, (t + 1) % m == 0, entry
 * j = (t + 1) / m - 1 is pooled exactly as csa_compress pools it,
 *   cache[b, j, c] = sum_{i<m} w_i x_token(m*j + i)[c],
 *   w = softmax(logits of tokens m*j .. m*j + m - 1),
 * and n_entries[b] is set to j + 1 (device memory, updated in place).
 * Otherwise (or when t < 0, or j >= N_max) nothing is written.
 * x        [B, x_rows, C] dtype, strides (x_sb, x_st): token s at row s mod
 *          x_rows; x_rows a positive multiple of m (x_rows = m: a ring of the
 *          latest block; x_rows >= sequence length: the whole sequence).
 * logits   [B, x_rows] fp32 (batch stride z_sb), token s at column s mod x_rows.
 * cache    [B, N_max, C] dtype with strides (c_sb, c_sj).
 * Requirements on dtype, C, m and alignment as csa_compress.
 */
csa_status_t csa_compress_append(const void* x, int64_t x_sb, int64_t x_st, int x_rows,
                                 const float* logits, int64_t z_sb, const int32_t* t_new,
                                 void* cache, int64_t c_sb, int64_t c_sj, int32_t* n_entries,
                                 csa_dtype_t dtype, int B, int C, int m, int N_max,
                                 hipStream_t stream);

/*
 * csa_quantize_mx4 - MX FP4 encoding of indexer vectors (§5: the indexer QK
 * path in FP4; the input format of CSA_FP4_E2M1_E8M0).  Per block of 32
 * consecutive elements of a row (OCP Microscaling encoding):
 *   e = floor(log2(max |x|)) - 2, clamped to [-127, 127] (-127 for an
 *   all-zero block); scale byte e + 127;
 *   code = the E2M1 magnitude nearest to |x| / 2^e (a tie to the code with an
 *   even mantissa bit; above 5 saturates to 6) with x's sign bit.
 * x       [rows, D] dtype (CSA_F32 or CSA_BF16), row stride x_rs elements.
 * codes   [rows, D/2] bytes, element 2i in the low nibble of byte i, row
 *         stride c_rs bytes.
 * scales  [rows, D/32] E8M0 bytes, row stride s_rs bytes.
 * Requires rows >= 1, D a multiple of 32, x and codes 16-byte aligned with
 * row strides of whole 16-byte units, c_rs >= D/2, s_rs >= D/32, x_rs >= D.
 * Inputs must be finite.
 */
csa_status_t csa_quantize_mx4(const void* x, int64_t x_rs, csa_dtype_t dtype, int rows, int D,
                              uint8_t* codes, int64_t c_rs, uint8_t* scales, int64_t s_rs,
                              hipStream_t stream);

/*
 * csa_index_score - Lightning Indexer scores (§2.1), every entry of the cache.
 *
 *   scores[b, t, j] = sum_h w_idx[b,t,h] * max(0, q_idx[b,t,h,:] . k_idx[b,j,:])
 *                     for j < V(b,t), and -inf for V(b,t) <= j < N_max.
 *
 * q_idx     [B, Tq, H_I, D_I] contiguous (idx_dtype); for the FP4 dtypes the
 *           codes [B, Tq, H_I, D_I/2] bytes plus q_scale [B, Tq, H_I, D_I/32]
 *           contiguous: fp32 (CSA_FP4_E2M1) or E8M0 bytes (CSA_FP4_E2M1_E8M0).
 * w_idx     [B, Tq, H_I] fp32 contiguous.
 * k_idx     [B, N_max, D_I] with strides (k_sb, k_sn) (FP4: bytes of codes);
 *           k_scale [B, N_max, D_I/32] with strides (ks_sb, ks_sn) in scale
 *           elements (fp32 or bytes) for the FP4 dtypes, else NULL.  Scale
 *           pointers and strides: 16-byte aligned for fp32 scales, 4-byte
 *           aligned for E8M0 bytes.
 * q_pos     [B, Tq] int32 device: position of each query token.
 * n_entries [B] int32 device: valid cache rows per sequence (<= N_max).
 * scores    [B, Tq, N_max] fp32 contiguous.
 * Supported: F32 / BF16 with H_I <= 64 and D_I in {32, 64, 128};
 *            both FP4 dtypes with H_I = 64, D_I = 128.  Tuned: BF16 and FP4
 *            64 x 128.
 */
csa_status_t csa_index_score(const void* q_idx, const void* q_scale, const float* w_idx,
                             const void* k_idx, const void* k_scale,
                             int64_t k_sb, int64_t k_sn, int64_t ks_sb, int64_t ks_sn,
                             csa_dtype_t idx_dtype,
                             const int32_t* q_pos, const int32_t* n_entries,
                             int B, int Tq, int N_max, int H_I, int D_I, int m,
                             float* scores, hipStream_t stream);

/*
 * csa_topk - top-k selection of compressed entries per query token (§2.1).
 *
 * scores    [B, Tq, *] fp32 with row stride s_rs (>= N_max); only the first
 *           V(b,t) entries of a row are considered; they must be finite.
 * topk_idx  [B, Tq, k] int32: the min(k, V) entries with the largest scores,
 *           ties to the lower index, in ascending index order, then -1.
 * topk_score [B, Tq, k] fp32 or NULL: the score of each returned entry
 *           (-inf for padding).
 * ws        workspace of at least csa_topk_workspace(...) bytes (may be NULL
 *           when that size is 0).
 * Supported: 1 <= k <= 2048, ceil(N_max / 32768) * k <= 32768.
 */
csa_status_t csa_topk(const float* scores, int64_t s_rs,
                      const int32_t* q_pos, const int32_t* n_entries,
                      int B, int Tq, int N_max, int m, int k,
                      int32_t* topk_idx, float* topk_score,
                      void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t csa_topk_workspace(int B, int Tq, int N_max, int k, size_t* bytes);

/*
 * csa_index_topk - csa_index_score followed by csa_topk, with the score
 * matrix kept in the workspace.  Arguments as in those two calls.
 * ws        csa_index_topk_workspace bytes, 16-byte aligned, ZERO-FILLED before
 *           its first use: it starts with counters through which the
 *           workgroups that share a long row hand its survivors to the last
 *           of them (tuned indexers, at most 64 rows).  Every call leaves
 *           them zero, so a workspace is cleared once and then reused by
 *           calls of any shape; calls that may run concurrently need
 *           separate workspaces.
 */
csa_status_t csa_index_topk(const void* q_idx, const void* q_scale, const float* w_idx,
                            const void* k_idx, const void* k_scale,
                            int64_t k_sb, int64_t k_sn, int64_t ks_sb, int64_t ks_sn,
                            csa_dtype_t idx_dtype,
                            const int32_t* q_pos, const int32_t* n_entries,
                            int B, int Tq, int N_max, int H_I, int D_I, int m, int k,
                            int32_t* topk_idx, float* topk_score,
                            void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t csa_index_topk_workspace(int B, int Tq, int N_max, int k, size_t* bytes);

/*
 * csa_index_topk_bf16 - csa_index_topk with the score matrix held in BF16
 * ("DeepSeek-V4 点评总结", 主要观点, the FP4 quantisation-aware-training
 * point: index scores stored in BF16 instead of FP32, reported as 2x faster
 * inference at 99.7 % KV recall).
 *
 *   Each fp32 score is rounded to BF16 (nearest, ties to even) when it is
 *   stored; the selection is the exact top-k of the rounded scores (ties to
 *   the lower index, ascending index order, -1 padding), so it can differ
 *   from the fp32 selection only where rounding merges or reorders scores.
 * Arguments as in csa_index_topk for the BF16 64 x 128 indexer (q_idx
 * [B, Tq, 64, 128], k_idx [B, N_max, 128] with strides (k_sb, k_sn)); no
 * scale arguments.  topk_score returns the rounded scores (fp32) or is NULL.
 * Workspace: csa_index_topk_bf16_workspace bytes, 16-byte aligned, ZERO-FILLED
 * before its first use (as for csa_index_topk).
 * Supported: N_max <= 262144 and k as for csa_topk; else CSA_ERR_UNSUPPORTED.
 */
csa_status_t csa_index_topk_bf16(const void* q_idx, const float* w_idx, const void* k_idx,
                                 int64_t k_sb, int64_t k_sn,
                                 const int32_t* q_pos, const int32_t* n_entries,
                                 int B, int Tq, int N_max, int m, int k,
                                 int32_t* topk_idx, float* topk_score,
                                 void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t csa_index_topk_bf16_workspace(int B, int Tq, int N_max, int k, size_t* bytes);

/*
 * csa_attend - core attention over the selected entries only (§2.1).
 *
 *   o[b,t,h,:] = sum_{j in S} softmax_j(scale * q[b,t,h,:] . K[b,j,:]) V[b,j,:]
 *   S = { topk_idx[b,t,i] : 0 <= topk_idx[b,t,i] < n_entries[b] }.
 *   lse[b,t,h] = log sum_{j in S} exp(scale * q . K[b,j]).  Empty S: o = 0,
 *   lse = -inf.  Repeated indices count repeatedly.
 *
 * q         [B, Tq, H, D] contiguous (dtype).
 * k_c, v_c  [B, N_max, D] sharing strides (kv_sb, kv_sn).
 * topk_idx  [B, Tq, k] int32.
 * out       [B, Tq, H, D] (dtype); lse [B, Tq, H] fp32 or NULL.
 * ws        csa_attend_workspace bytes, 16-byte aligned (NULL when that is 0).
 *           The tuned path splits the entry list over several workgroups
 *           that merge their partial results through synchronisation words
 *           at the front of the workspace: the workspace must be ZERO-FILLED
 *           before its first use (for example with hipMemsetAsync).  Every
 *           call leaves those words zero again, so a workspace is cleared
 *           once and then reused by any number of calls of any shape (this
 *           holds for hca_attend and swa_attend workspaces too).  Calls that
 *           may run concurrently need separate workspaces.
 * Supported: F32 / BF16 with H <= 64, D in {32, 64, 128}, B * Tq <= 65536;
 *            tuned BF16 64 x 128.
 */
csa_status_t csa_attend(const void* q, const void* k_c, const void* v_c,
                        int64_t kv_sb, int64_t kv_sn,
                        const int32_t* topk_idx, const int32_t* n_entries,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int k,
                        float scale, void* out, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t csa_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int k,
                                  size_t* bytes);

/*
 * hca_attend - HCA (§2.2): attention over every visible compressed entry,
 * S = { j : j < V(b,t) } with V as above for pooling factor m.  Other
 * arguments and outputs as in csa_attend.
 */
csa_status_t hca_attend(const void* q, const void* k_c, const void* v_c,
                        int64_t kv_sb, int64_t kv_sn,
                        const int32_t* q_pos, const int32_t* n_entries,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int m,
                        float scale, void* out, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t hca_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max,
                                  size_t* bytes);

/*
 * csa_attend_merge - attention over the union of two disjoint key sets from
 * the two partial results ("DeepSeek V4 技术解读", §2.3: a local sliding
 * window kept next to the compressed global entries; e.g. the outputs of
 * swa_attend and csa_attend for the same queries, same softmax scale).
 *
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   out = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b     (per row and head;
 *   both sets empty, lse_a = lse_b = -inf: out 0, lse -inf).
 *
 * o_a, o_b, out [rows, H, D] contiguous (dtype F32 or BF16), lse_a, lse_b,
 * lse_out [rows, H] fp32 (lse_out may be NULL).  out may be o_a or o_b
 * itself (elementwise); no other overlap.  Requires D a multiple of 8.
 */
csa_status_t csa_attend_merge(const void* o_a, const float* lse_a, const void* o_b,
                              const float* lse_b, csa_dtype_t dtype, int rows, int H, int D,
                              void* out, float* lse_out, hipStream_t stream);

/*
 * csa_index_topk_attend - one CSA decode step: Lightning Indexer scores,
 * top-k selection and core attention over the selected entries, in one call
 * ("DeepSeek V4 技术解读", §2.1, the three steps of the CSA flow: compressed
 * KV cache -> Lightning Indexer -> core attention).
 *
 *   Results equal csa_index_topk followed by csa_attend on the same inputs:
 *   out (and lse) as csa_attend computes them over the top-k set of each
 *   query token; topk_idx (NULL: not returned) as csa_index_topk returns it.
 *
 * Indexer arguments as in csa_index_topk (q_idx .. idx_dtype, H_I, D_I);
 * attention arguments as in csa_attend (q, k_c, v_c, kv_sb, kv_sn, dtype, H,
 * D, scale, out, lse); q_pos, n_entries, B, Tq, N_max, m, k as in both.
 * ws        csa_index_topk_attend_workspace bytes, 16-byte aligned, ZERO-FILLED
 *           before its first use (it starts with the selection's and the
 *           attention's synchronisation words; every call leaves them zero).
 * The step runs the score kernel, the selection kernel(s) and the split
 * attention kernel (which merges its splits itself) back to back on
 * `stream`, with the index lists in the workspace when topk_idx is NULL.
 * Supported: as csa_index_topk and csa_attend together.
 */
csa_status_t csa_index_topk_attend(const void* q_idx, const void* q_scale, const float* w_idx,
                                   const void* k_idx, const void* k_scale,
                                   int64_t k_sb, int64_t k_sn, int64_t ks_sb, int64_t ks_sn,
                                   csa_dtype_t idx_dtype,
                                   const void* q, const void* k_c, const void* v_c,
                                   int64_t kv_sb, int64_t kv_sn, csa_dtype_t dtype,
                                   const int32_t* q_pos, const int32_t* n_entries,
                                   int B, int Tq, int N_max, int H_I, int D_I, int H, int D,
                                   int m, int k, float scale,
                                   void* out, float* lse, int32_t* topk_idx,
                                   void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t csa_index_topk_attend_workspace(csa_dtype_t idx_dtype, csa_dtype_t dtype, int B,
                                             int Tq, int N_max, int H, int D, int k,
                                             size_t* bytes);

/*
 * csa_index_topk_attend_noalloc - csa_index_topk_attend for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same results.
 *
 * The intermediate buffers live in a library-owned scratch array of
 * csa_index_topk_attend_noalloc_max_bytes() bytes (32 MiB) per GPU, held
 * until the process ends; the call allocates nothing.  Every call on a GPU
 * uses that GPU's one array, so calls that may overlap on one GPU (other
 * streams, other threads) race and must not be issued.  The stream must
 * belong to the calling thread's current device.  Limits: B * Tq <= 4096 and
 * the step's buffers within the scratch size: csa_index_topk_attend_workspace
 * less 7.5 MiB (its attention counters serve 65536 rows in 8 MiB, the
 * scratch's 4096 rows in 0.5 MiB) at most 32 MiB, else CSA_ERR_UNSUPPORTED.
 */
csa_status_t csa_index_topk_attend_noalloc(const void* q_idx, const void* q_scale,
                                           const float* w_idx, const void* k_idx,
                                           const void* k_scale, int64_t k_sb, int64_t k_sn,
                                           int64_t ks_sb, int64_t ks_sn, csa_dtype_t idx_dtype,
                                           const void* q, const void* k_c, const void* v_c,
                                           int64_t kv_sb, int64_t kv_sn, csa_dtype_t dtype,
                                           const int32_t* q_pos, const int32_t* n_entries,
                                           int B, int Tq, int N_max, int H_I, int D_I, int H,
                                           int D, int m, int k, float scale,
                                           void* out, float* lse, int32_t* topk_idx,
                                           hipStream_t stream);
size_t csa_index_topk_attend_noalloc_max_bytes(void);

/*
 * swa_attend - sliding-window attention over uncompressed tokens ("DeepSeek
 * V4 技术解读", §2.3: the first layers attend a sliding window of recent
 * tokens at full resolution; the window size is not given there and is an
 * argument here).
 *
 *   o[b,t,h,:] = sum_{j in S} softmax_j(scale * q[b,t,h,:] . K[b,j,:]) V[b,j,:]
 *   S = { j : max(0, P - window) <= j < P },  P = min(q_pos[b,t] + 1,
 *   n_tokens[b], N_max): the query's own token and the window - 1 before it.
 *   lse as in csa_attend (S is never empty for q_pos >= 0).
 * q [B, Tq, H, D] contiguous; k, v [B, N_max, D] token caches sharing strides
 * (kv_sb, kv_sn); q_pos [B, Tq], n_tokens [B] int32 device (tokens cached).
 * window >= 1.  Workspace: swa_attend_workspace bytes (16-byte aligned).
 * Supported: as csa_attend; tuned BF16 64 x 128.
 */
csa_status_t swa_attend(const void* q, const void* k, const void* v,
                        int64_t kv_sb, int64_t kv_sn,
                        const int32_t* q_pos, const int32_t* n_tokens,
                        csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max, int window,
                        float scale, void* out, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream);
csa_status_t swa_attend_workspace(csa_dtype_t dtype, int B, int Tq, int H, int D, int N_max,
                                  int window, size_t* bytes);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
