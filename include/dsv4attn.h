/*
 * libdsv4attn -- the CSA / HCA attention hot path of DeepSeek-V4 for AMD
 * Instinct MI355X (gfx950), as a plain C ABI.
 *
 * Sources (cited by page title and section):
 *   digest = ai-papers-daily page "DeepSeek-V4: Towards Highly Efficient
 *            Million-Token Context Intelligence", 子模块实现, 模块 B (CSA,
 *            eq 9-19), 模块 C (HCA, eq 20-26), 模块 D (sliding window,
 *            attention sink), 模块 F (KV precisions, FP4 indexer).
 *   blog   = jsqmd page "DeepSeek V4大模型算法解析", 二、核心算法, 1.) CSA
 *            (第一/二/三阶段) and 2.) HCA.
 *   news   = 智能計算芯世界 page on DeepSeek-V4, 三、全棧基建優化 (batch-invariant,
 *            deterministic kernels).
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer unless it is marked "host".
 *     The caller owns every buffer (inputs, outputs, workspaces); the library
 *     allocates nothing and keeps no mutable global state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every kernel is
 *     enqueued on it and the call returns without synchronising.
 *   - Return value: DSV4_OK, or an error status.  Argument checks run on the
 *     host before any HIP call; on any error nothing is launched and no output
 *     is written.  dsv4_last_error() gives a message for the calling thread.
 *   - Tensors are row-major, last dimension contiguous.  Weights use the
 *     [out, in] layout, so a projection is C = H W^T.
 *   - Positions: query i of batch b sits at absolute position q_pos0[b] + i.
 *     Compressed-cache row s of a batch is absolute block s.  Entry s is
 *     visible to position p iff ratio*(s+1) <= p+1 (every token it pools is at
 *     or before p; digest 模块 D: a query attends only to earlier blocks).
 *   - Results are deterministic and batch invariant: a sequence's outputs do
 *     not depend on the batch it is in, and repeated calls are bitwise equal
 *     (news, 批不變 + 確定性內核).
 */
#ifndef DSV4ATTN_H
#define DSV4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DSV4_OK                   0
#define DSV4_ERR_INVALID_ARG      1 /* null pointer, bad size, uncovered window ... */
#define DSV4_ERR_UNSUPPORTED      2 /* dtype / layout / shape combination not built */
#define DSV4_ERR_HIP              3 /* a HIP launch failed */
#define DSV4_ERR_WORKSPACE        4 /* workspace smaller than the size query returns */

/* activation dtypes (hidden states, queries, weights, attention outputs) */
#define DSV4_F32                  0
#define DSV4_BF16                 1

/* row layouts of compressed entries, window rows and indexer keys.
 * ROW_FP8_ROPE_BF16: dims [0, c-64) as OCP E4M3 bytes (no scale) followed by
 *   dims [c-64, c) as bf16 -- the last 64 dims carry RoPE and stay bf16
 *   (digest 模块 D partial RoPE, 模块 F mixed-precision KV); c + 64 bytes.
 * ROW_MXFP4: c/2 bytes of OCP E2M1 codes (element 2j in the low nibble of byte
 *   j) plus a separate scales array of c/32 E8M0 bytes per row (one per 32
 *   consecutive dims); used for the indexer keys (digest 模块 F FP4 indexer). */
#define DSV4_ROW_F32              0
#define DSV4_ROW_BF16             1
#define DSV4_ROW_FP8_ROPE_BF16    2
#define DSV4_ROW_MXFP4            3

/* Bytes of one stored row of width c in `layout` (MXFP4: codes only). 0 if invalid. */
size_t dsv4_row_bytes(int layout, int c);

/*
 * CSA token-level compressor (digest 模块 B eq 9-12; blog 第一阶段).
 *   C^a, C^b, Z^a, Z^b = H W_{aKV}^T, H W_{bKV}^T, H W_{aZ}^T, H W_{bZ}^T.
 *   Entry i, channel j: softmax over the logits Z^a[m i + r, j] + B^a[r, j] and
 *   Z^b[m (i-1) + r, j] + B^b[r, j] (r < m; the b-part is absent for entry 0),
 *   then the matching weighted sum of C^a / C^b rows.  Windows of successive
 *   entries overlap by m tokens.
 *
 * H        [n_left + n, d] act_dtype.  Row n_left is the token at absolute
 *          position m*block0; the n_left rows before it are left context.
 * W        [4c, d] act_dtype = W_aKV | W_bKV | W_aZ | W_bZ stacked by rows.
 * bias_ab  [2, m, c] float = B^a, B^b.
 * block0   absolute index of the first emitted entry.  If block0 > 0 the first
 *          entry's b-window needs n_left >= m (else DSV4_ERR_INVALID_ARG).
 * comp_out [n/m rows] in comp_layout (F32, BF16, FP8_ROPE_BF16 or MXFP4);
 *          comp_scales [n/m, c/32] bytes for MXFP4, else ignored (may be NULL).
 *          An incomplete final block (n % m tokens) emits no entry.
 * raw_out  [n rows] of C^a in raw_layout (F32, BF16 or FP8_ROPE_BF16), the
 *          uncompressed sliding-window KV of the chunk; NULL to skip.
 * Row layouts FP8_ROPE_BF16 need c >= 64 and c % 32 == 0; MXFP4 needs c % 32 == 0.
 */
int dsv4_csa_compress(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype,
                      const void* W, const float* bias_ab, int m, int c, int64_t block0,
                      void* comp_out, void* comp_scales, int comp_layout,
                      void* raw_out, int raw_layout, void* stream);

/*
 * HCA compressor (digest 模块 C eq 20-23; blog 2.) HCA): C = H W_KV^T,
 * Z = H W_Z^T; entry i, channel j = softmax_r(Z[m' i + r, j] + B[r, j]) weighted
 * sum of C[m' i + r, j] over r < m' (no overlap).
 * H [n, d]; W [2c, d] = W_KV | W_Z; bias [m', c] float.
 * comp_out [n/m' rows] in comp_layout; raw_out [n rows] of C in raw_layout or NULL.
 */
int dsv4_hca_compress(const void* H, int64_t n, int64_t d, int act_dtype,
                      const void* W, const float* bias, int m_prime, int c,
                      void* comp_out, void* comp_scales, int comp_layout,
                      void* raw_out, int raw_layout, void* stream);

/*
 * The compressors of one chunk together (digest 核心思路: CSA and HCA layers
 * alternate, and both, with the indexer keys, compress the same hidden states
 * H of the chunk): the results are those of
 *   dsv4_csa_compress(H, n_left, n, ..., csa_kv ...),
 *   dsv4_csa_compress(H, n_left, n, ..., csa_keys ...) and
 *   dsv4_hca_compress(H + n_left rows, n, ..., hca ...),
 * bit for bit.  Any of the three may be NULL (skipped).  Each is validated as
 * its own call would be, all before anything is launched.  When every given
 * compressor takes the pipelined MFMA path (bf16 H, d % 64 == 0, c % 64 == 0,
 * m = 4, m' = 128, no MXFP4 window rows, MXFP4 entries for CSA only) they run
 * in one launch over the same 256-token tiles of H; otherwise one after the
 * other.
 */
typedef struct {
  const void* W;         /* CSA: [4c, d] = W_aKV | W_bKV | W_aZ | W_bZ; HCA: [2c, d] = W_KV | W_Z */
  const float* bias;     /* CSA: [2, m, c] = B^a, B^b; HCA: [m', c] */
  int c;
  void* comp_out;        /* entries in comp_layout; comp_scales for MXFP4 (else may be NULL) */
  void* comp_scales;
  int comp_layout;
  void* raw_out;         /* window rows in raw_layout, or NULL */
  int raw_layout;
} dsv4_compressor_t;

int dsv4_compress_chunk(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                        int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                        int m_prime, const dsv4_compressor_t* hca, void* stream);

/*
 * Lightning-indexer scores (digest 模块 B eq 16; blog 第二阶段):
 *   I[b, t, s] = sum_h wI[b, t, h] * ReLU(qI[b, t, h, :] . K[b, s, :])
 * for entries visible to the query (m*(s+1) <= p+1), -inf otherwise.  No scale.
 * qI     [B, nq, hI, cI] q_dtype;  wI [B, nq, hI] float.
 * keys   [B, S, row] in k_layout (F32, BF16 or MXFP4); k_scales [B, S, cI/32]
 *        bytes for MXFP4 (else ignored).
 * q_pos0 host [B].   scores [B, nq, S] float (output).
 * The float accumulation is fp32; bf16 and MXFP4 inputs are decoded exactly.
 */
int dsv4_indexer_score(const void* qI, int q_dtype, const float* wI,
                       const void* keys, const uint8_t* k_scales, int k_layout,
                       int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                       const int64_t* q_pos0, float* scores, void* stream);

/*
 * Index scores with the indexer's QK product in FP4 (digest 模块 F: the
 * lightning indexer computes its attention in FP4).  Each query head's c_I
 * values are quantised to MXFP4 exactly as the keys are stored (blocks of 32
 * along c_I, E8M0 scale 2^(floor(log2 amax) - 2), E2M1 elements rounded to
 * nearest even, saturating), then
 *   I[b, t, s] = sum_h wI[b, t, h] * ReLU(Q4[b, t, h, :] . K4[b, s, :])
 * for visible entries, -inf otherwise, with the products of FP4 values exact
 * and the sums in fp32.  Same arguments as dsv4_indexer_score with MXFP4 keys:
 * k_codes [B, S, cI/2] (element 2j in the low nibble of byte j), k_scales
 * [B, S, cI/32].  cI must be a multiple of 32.
 */
int dsv4_indexer_score_fp4q(const void* qI, int q_dtype, const float* wI,
                            const uint8_t* k_codes, const uint8_t* k_scales,
                            int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                            const int64_t* q_pos0, float* scores, void* stream);

/*
 * Index scores with the queries in FP8: as dsv4_indexer_score_fp4q, but each
 * query head's 32-value blocks along c_I are quantised to MXFP8 (OCP MX: E8M0
 * scale 2^(floor(log2 amax) - 8), E4M3 elements rounded to nearest even and
 * saturated at 448) and multiplied with the stored MXFP4 keys on the scaled
 * MFMA (E4M3 x E2M1 products exact, sums in fp32).  The FP8 side of the
 * pages' low-precision indexer (digest 模块 F); same arguments and limits.
 */
int dsv4_indexer_score_fp8q(const void* qI, int q_dtype, const float* wI,
                            const uint8_t* k_codes, const uint8_t* k_scales,
                            int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                            const int64_t* q_pos0, float* scores, void* stream);

/*
 * Top-k selector (digest 模块 B eq 17; blog 第二阶段 Top-k稀疏选择).
 * For each row (b, t): the k visible entries with the largest score; ties go
 * to the lower index; order (score descending, index ascending); fewer than
 * k visible entries -> all of them, then -1 padding.  Only entries with
 * m*(s+1) <= p+1 and s < S are candidates (the score values of other entries
 * are never read).  -0.0 and +0.0 compare equal.  Scores must not be NaN.
 * scores [B, nq, S] float; idx_out [B, nq, k] int32.  k <= 4096.
 * ws: workspace of dsv4_topk_workspace_size() bytes (may be 0 -> NULL ok).
 */
size_t dsv4_topk_workspace_size(int64_t B, int64_t nq, int64_t S, int k);
int dsv4_topk_select(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                     const int64_t* q_pos0, int k, int32_t* idx_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Index scores and top-k in one call (digest 模块 B eq 16 then eq 17): idx_out
 * is bit for bit what dsv4_indexer_score into a [B, nq, S] buffer followed by
 * dsv4_topk_select with the same k would give (same arguments, same limits as
 * those two calls; k <= 4096), without the caller holding the score rows.
 * For bf16 queries with 32 heads, cI in {32, 64, 128}, BF16 or MXFP4 keys and
 * k <= 1024 the scores are not stored: every 32nd key is scored first, each
 * row's threshold is a value at or below its ks-th best sample score (ks
 * about k/32 plus six standard deviations), the full pass keeps only the
 * visible scores at or above it, and a per-row select takes the k best of
 * those.  A row that kept fewer than min(k, visible) scores, or more than its
 * lists hold, has its scores recomputed in full and selected by the top-k
 * pass, so the result never depends on the sample.  Other shapes run the two
 * calls in sequence through the workspace.
 * ws: workspace of dsv4_indexer_topk_workspace_size() bytes (the same
 * arguments); it holds a full score row for each query of up to 64 sequences,
 * written only for rows the threshold does not settle.  A smaller workspace
 * fails with DSV4_ERR_WORKSPACE before anything is launched.
 */
size_t dsv4_indexer_topk_workspace_size(int q_dtype, int k_layout, int64_t B, int64_t nq, int hI, int cI,
                                        int64_t S, int k);
int dsv4_indexer_topk(const void* qI, int q_dtype, const float* wI,
                      const void* keys, const uint8_t* k_scales, int k_layout,
                      int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                      const int64_t* q_pos0, int k, int32_t* idx_out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * dsv4_topk_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and results as
 * dsv4_topk_select.  Its workspace is a static device array of
 * DSV4_TOPK_SCRATCH_BYTES per GPU, held until the process ends; a shape whose
 * dsv4_topk_workspace_size() exceeds it fails with DSV4_ERR_UNSUPPORTED
 * before anything runs.  The call allocates nothing (no hipMalloc, no
 * hipFree).  Every call on one GPU shares that array: calls that overlap on
 * one GPU (concurrent streams, other threads) race and must be serialised by
 * the caller.
 */
#define DSV4_TOPK_SCRATCH_BYTES ((size_t)16 << 20)
int dsv4_topk_select_noalloc(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                             const int64_t* q_pos0, int k, int32_t* idx_out, void* stream);

/*
 * CSA core: shared-KV multi-query attention over the selected compressed
 * entries plus the sliding window, with an attention sink (digest 模块 B
 * eq 18-19, 模块 D; blog 第三阶段).  For query (b, t) at position p and head h:
 *   keys = { kv_comp[b, s] : s in idx[b, t], 0 <= s < S }  ++
 *          { window row of position u : max(0, p-n_win+1) <= u <= p }
 *   l_x = scale * q[b,t,h] . key_x;  M = max(max_x l_x, sink[h])
 *   out[b,t,h] = sum_x e^{l_x-M} key_x / (sum_x e^{l_x-M} + e^{sink[h]-M})
 * Each key is also its value.  Entries of idx outside [0, S) are padding.
 * scale must be finite and > 0 (1/sqrt(c) in the pages' reading).
 * sink NULL -> no sink term.  An empty key set gives a zero output.
 * q [B, nq, nh, c] q_dtype; out the same shape and dtype.
 * kv_comp [B, S, row] and kv_win [B, W, row] in kv_layout (F32 with F32
 * queries; BF16 or FP8_ROPE_BF16 with BF16 queries).  Window row w of batch b
 * holds position win_pos0[b] + w (host array); every query's window must be
 * covered, else DSV4_ERR_INVALID_ARG.  idx [B, nq, k] int32.
 * ws: workspace of dsv4_attn_workspace_size() bytes, where dense is 0 for this
 * call and 1 for dsv4_hca_dense_fwd, and max_keys bounds the compressed
 * entries plus window rows of any query (k + n_win here; S + n_win for HCA);
 * the exact need of a call is dsv4_attn_plan()'s workspace_bytes.  A smaller
 * workspace fails with DSV4_ERR_WORKSPACE before anything is launched.
 */
size_t dsv4_attn_workspace_size(int dense, int64_t B, int64_t nq, int nh, int c, int64_t max_keys);

/*
 * Launch plan of an attention call (host only, no HIP call): the kernel that
 * runs, how many queries share a block, and how a block's key slots are split
 * across blocks (splits > 1: per-split {m, l} in fp32 and output rows in bf16
 * in the workspace, merged in split order).  workspace_bytes is exactly what the call with these arguments
 * needs; dsv4_attn_workspace_size() bounds it from above.  Arguments as for
 * the calls themselves: dense 0 is dsv4_sparse_mqa_fwd (k used), dense 1 is
 * dsv4_hca_dense_fwd (m_prime used); q_pos0 is a host array [B].  Returns
 * DSV4_OK, DSV4_ERR_INVALID_ARG or DSV4_ERR_UNSUPPORTED (as the call would).
 */
typedef struct {
  int path;                /* 0 generic fp32-math kernel, 1 bf16-row MFMA (c = 128), 2 FP8-row MFMA (c = 512) */
  int queries_per_block;
  int splits;              /* key-slot splits of a query group (blocks per group) */
  int split_slots;         /* key slots per split (splits > 1) */
  size_t workspace_bytes;
} dsv4_attn_plan_t;
int dsv4_attn_plan(int dense, int q_dtype, int kv_layout, int64_t B, int64_t nq, int nh, int c, int64_t S,
                   int k, int m_prime, int n_win, const int64_t* q_pos0, dsv4_attn_plan_t* plan);
int dsv4_sparse_mqa_fwd(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                        const void* kv_comp, int kv_layout, int64_t S,
                        const int32_t* idx, int k,
                        const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                        const int64_t* q_pos0, const float* sink, float scale,
                        void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * HCA core: as dsv4_sparse_mqa_fwd but over every visible compressed entry
 * (m'*(s+1) <= p+1, s < S) instead of an index list (digest 模块 C eq 24-26;
 * blog 2.) HCA 融合与计算).
 */
int dsv4_hca_dense_fwd(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                       const void* kv_comp, int kv_layout, int64_t S, int m_prime,
                       const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                       const int64_t* q_pos0, const float* sink, float scale,
                       void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * The two attention cores with the output rotation (dsv4_out_rope; digest
 * 模块 D: each entry is key and value, so the output's RoPE dims are rotated
 * back by the query's position) done in the same launch: out is bit for bit
 * what the call without _rope followed by dsv4_out_rope(out, ..., theta,
 * rope_dims, q_pos0) leaves, without the second pass over out.  rope_dims and
 * c multiples of 8, rope_dims <= min(c, 512), theta > 0 (else
 * DSV4_ERR_UNSUPPORTED / DSV4_ERR_INVALID_ARG before anything is launched);
 * rope_dims 0 is the plain call.  Other arguments, the workspace and the
 * limits as for dsv4_sparse_mqa_fwd / dsv4_hca_dense_fwd.
 */
int dsv4_sparse_mqa_fwd_rope(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                             const void* kv_comp, int kv_layout, int64_t S,
                             const int32_t* idx, int k,
                             const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                             const int64_t* q_pos0, const float* sink, float scale,
                             float theta, int rope_dims,
                             void* out, void* ws, size_t ws_bytes, void* stream);
int dsv4_hca_dense_fwd_rope(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                            const void* kv_comp, int kv_layout, int64_t S, int m_prime,
                            const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                            const int64_t* q_pos0, const float* sink, float scale,
                            float theta, int rope_dims,
                            void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Query-side RMSNorm and partial RoPE (digest 模块 D: each query head is
 * RMS-normalised before core attention; RoPE acts on the last dims only).
 * For every row x = q[b, t, h, :] of width c, at position p = q_pos0[b] + t:
 *   y = x / sqrt(mean(x^2) + eps) * gamma          (gamma NULL: 1)
 *   then the last rope_dims dims are rotated as interleaved pairs
 *   (c - R + 2j, c - R + 2j + 1), j < R/2, by p * theta^(-2j/R).
 * q and q_out [B, nq, nh, c] in q_dtype (F32 or BF16, 16-byte aligned); they
 * may be the same buffer.  c a multiple of 8 up to 4096; rope_dims a multiple
 * of 8 up to min(c, 512) (64 in the pages); eps >= 0 (1e-6 in this library's
 * reading), theta > 0 (10000).  q_pos0: host array [B].
 */
int dsv4_q_norm_rope(const void* q, int q_dtype, void* q_out, int64_t B, int64_t nq, int nh, int c,
                     const float* gamma, float eps, float theta, int rope_dims,
                     const int64_t* q_pos0, void* stream);

/*
 * KV-side RMSNorm and partial RoPE, with the storage pack (digest 模块 D; 模块 F
 * for the FP8 + bf16-RoPE rows).  Row i of batch entry b, rows[b, i, :] in
 * in_layout (F32 or BF16), sits at position pos0[b] + pos_stride * i (host
 * array pos0): window rows use their token positions (stride 1), compressed
 * entries the newest token they pool, m (s + 1) - 1 (stride m).  The row is
 * normalised and rotated as in dsv4_q_norm_rope and stored to rows_out[b, i]
 * in out_layout (F32, BF16 or FP8_ROPE_BF16).  In place only when the two
 * layouts have the same row size.  Same limits on c, rope_dims, eps and theta
 * as dsv4_q_norm_rope; FP8 rows need c >= 64 and c % 16 == 0.
 */
int dsv4_kv_norm_rope(const void* rows, int in_layout, int64_t B, int64_t n, int c,
                      const float* gamma, float eps, float theta, int rope_dims,
                      const int64_t* pos0, int64_t pos_stride,
                      void* rows_out, int out_layout, void* stream);

/*
 * Output rotation (digest 模块 D: since each KV entry is key and value, the
 * output carries the entries' absolute positions; rotating it back by the
 * query's position leaves relative ones).  In place on o [B, nq, nh, c]
 * (F32 or BF16): the last rope_dims dims of row (b, t, h) are rotated by
 * -(q_pos0[b] + t), as pairs like dsv4_q_norm_rope; the other dims are not
 * touched.  rope_dims == 0 is a no-op.
 */
int dsv4_out_rope(void* o, int o_dtype, int64_t B, int64_t nq, int nh, int c, float theta, int rope_dims,
                  const int64_t* q_pos0, void* stream);

/*
 * bf16 GEMM, C = A B^T with fp32 accumulation, for the projections around the
 * core (digest 模块 B: the low-rank query path and the grouped output
 * projection).  A [M, K] and B [N, K] are bf16, K-contiguous with row strides
 * lda, ldb (elements, multiples of 8, 16-byte aligned bases); C [M, N] in
 * c_dtype (F32 or BF16, round to nearest even) with row stride ldc.  batch
 * products run with element strides stride_a, stride_b, stride_c (multiples
 * of 8 for A and B when batch > 1).  K a multiple of 64.
 */
int dsv4_gemm_bf16_nt(const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b,
                      void* C, int c_dtype, int64_t ldc, int64_t stride_c, int64_t M, int64_t N, int64_t K,
                      int64_t batch, void* stream);

/*
 * Low-rank query path (digest 模块 B eq 13-15 and 18): for h [n, d] bf16,
 *   c^Q = h W_DQ^T          [n, d_c], stored bf16 in ws
 *   q   = c^Q W_UQ^T        [n, nh * c]   bf16  (the heads of MQA)
 *   q^I = c^Q W_IUQ^T       [n, hI * cI]  bf16  (the indexer heads)
 *   w^I = h W_w^T           [n, hI]       fp32  (the indexer head weights)
 * Weights in the [out, in] layout, bf16: W_DQ [d_c, d], W_UQ [nh c, d_c],
 * W_IUQ [hI cI, d_c], W_w [hI, d].  q, qI or wI may be NULL to skip them (the
 * HCA layer has no indexer).  d and d_c multiples of 64.  ws: at least
 * dsv4_query_proj_workspace_size(n, d_c) bytes, 16-byte aligned.
 */
size_t dsv4_query_proj_workspace_size(int64_t n, int d_c);
int dsv4_query_proj(const void* h, int64_t n, int d, const void* W_DQ, int d_c,
                    const void* W_UQ, int nh, int c, const void* W_IUQ, int hI, int cI, const void* W_w,
                    void* q, void* qI, float* wI, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped output projection (digest 模块 B): the nh head outputs o [n, nh, c]
 * form g groups of consecutive heads; group j's rows (nh/g heads, flattened
 * head-major) are projected by W_O1[j] [d_g, (nh/g) c] into columns
 * [j d_g, (j+1) d_g) of z [n, g d_g] (stored bf16 in ws), then
 * out = z W_O2^T [n, d] bf16 with W_O2 [d, g d_g].  All bf16; (nh/g) c and
 * g d_g multiples of 64.  ws: dsv4_output_proj_workspace_size(n, g, d_g) bytes.
 */
size_t dsv4_output_proj_workspace_size(int64_t n, int g, int d_g);
int dsv4_output_proj(const void* o, int64_t n, int nh, int c, int g, int d_g, const void* W_O1,
                     const void* W_O2, int d, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Streaming cache maintenance for decode (digest 模块 F: every compressed
 * entry is persisted and a reused prefix computes only its incomplete
 * trailing block again; the uncompressed window rows are cached, checkpointed
 * or recomputed.  Pooling as dsv4_csa_compress / dsv4_hca_compress: 模块 B
 * eq 9-12, 模块 C eq 20-23; blog 第一阶段 for the b-window).
 *
 * State: per sequence a caller-owned buffer of dsv4_stream_state_bytes()
 * bytes (sequence b at state + b * that size): per channel an online-softmax
 * accumulator (running maximum, sum of weights, weighted sum) of the entry of
 * the current block and, with overlap = 1 (CSA), one of the next entry's
 * b-part (the current block's b-rows), each tagged with its entry and the
 * number of rows it holds.  overlap = 0 is HCA (no b-window).
 * dsv4_stream_state_reset() marks both accumulators empty (a fill kernel, so
 * it can sit in a captured graph).
 */
size_t dsv4_stream_state_bytes(int overlap, int m, int c);
int dsv4_stream_state_reset(void* state, int64_t B, int overlap, int m, int c, void* stream);

/* RMSNorm and partial RoPE applied to a row before it is packed (as in
 * dsv4_kv_norm_rope).  norm 0 skips the RMSNorm; rope_dims 0 the rotation. */
typedef struct {
  int norm;             /* 1: x / sqrt(mean(x^2) + eps) * gamma */
  const float* gamma;   /* [c] device, or NULL for 1 */
  float eps;            /* >= 0 */
  int rope_dims;        /* last dims rotated as pairs, multiple of 8, <= min(c, 512) */
  float theta;          /* > 0 */
} dsv4_norm_rope_t;

/*
 * dsv4_compress_chunk with the KV RMSNorm and partial RoPE of the pages
 * (digest 模块 D: the compressed KV head is RMS-normalised before core
 * attention and its last rope_dims dims carry RoPE) applied in the same call
 * to what the CSA KV compressor (kv_nr) and the HCA compressor (hca_nr; each
 * layer has its own gamma) emit, entries and window rows; a NULL descriptor
 * leaves that compressor as dsv4_compress_chunk has it.  The results are
 * those of dsv4_compress_chunk with F32 rows followed by
 * dsv4_kv_norm_rope(F32 rows -> the caller's layout), bit for bit, for
 *   CSA entries at positions m (s + 1) - 1 (s absolute, from block0),
 *   HCA entry i of the chunk at m block0 + m' (i + 1) - 1,
 *   window rows of chunk token i at m block0 + i
 * (the chunk starts at token m block0).  norm 0: rotation only.  The indexer
 * keys are not normalised.  The compressors' 64-channel tiles split a row
 * across blocks, so the fp32 rows pass through the workspace
 * (dsv4_compress_chunk_nr_workspace_size(n, m, c of the normalised CSA KV or
 * 0, m', c of the normalised HCA or 0) bytes) to a second kernel of the call.
 * Normalised outputs in F32, BF16 or FP8_ROPE_BF16.
 */
size_t dsv4_compress_chunk_nr_workspace_size(int64_t n, int m, int c_kv, int m_prime, int c_hca);
int dsv4_compress_chunk_nr(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                           int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                           int m_prime, const dsv4_compressor_t* hca, const dsv4_norm_rope_t* kv_nr,
                           const dsv4_norm_rope_t* hca_nr, void* ws, size_t ws_bytes, void* stream);

/*
 * Feed n_new tokens of each of B sequences: H [B, n_new, d] (act_dtype) holds
 * the hidden states of positions pos0[b] + i (host array, >= 0).  W and bias
 * as the batch compressors (CSA, overlap = 1: W [4c, d] = W^{aKV} | W^{bKV} |
 * W^{aZ} | W^{bZ}, bias [2, m, c]; HCA, overlap = 0: W [2c, d], bias [m, c]).
 * For every token, in order:
 *   - its logits and values enter the accumulators;
 *   - its C^a (CSA) / C (HCA) row, normalised and rotated at its position
 *     when nr != NULL, is packed into the window ring when ring != NULL:
 *     ring [B, 2 ring_w, row] in ring_layout (F32, BF16, FP8_ROPE_BF16), rows
 *     x mod ring_w and x mod ring_w + ring_w.  The attention calls read it as
 *     kv_win with W = 2 ring_w and win_pos0[b] = dsv4_swa_ring_pos0(p, ring_w)
 *     for a query at p, provided n_win <= ring_w;
 *   - if it completes block s (position m (s + 1) - 1) and
 *     emit_from[b] <= s < S (emit_from: host array, or NULL for 0), entry s
 *     (the accumulated weighted sum over the sum of weights, per channel),
 *     normalised and rotated at position
 *     m (s + 1) - 1 when nr != NULL, and packed into cache[b, s] (cache
 *     [B, S, row] in cache_layout; MXFP4 also cache_scales [B, S, c/32];
 *     cache NULL: no entries).
 * Resuming after P persisted tokens: reset the state, then feed positions
 * from m floor(P/m) (HCA) or m max(floor(P/m) - 1, 0) (CSA: the b-window)
 * with emit_from = floor(P/m).  An entry whose rows were not all fed since
 * the reset is written as the layout's NaN (F32 / BF16 NaN, E4M3 0x7F, MXFP4
 * scale 0xFF).
 * c even and <= 512 (FP8 rows: c >= 64, c % 16 == 0; MXFP4: c % 32 == 0);
 * bf16 needs d % 8 == 0.  ws: dsv4_stream_workspace_size() bytes, 16-byte
 * aligned.  Results for a sequence do not depend on B or on the other rows.
 */
size_t dsv4_stream_workspace_size(int64_t B, int64_t n_new, int64_t d, int overlap, int c);
int dsv4_stream_compress(const void* H, int64_t B, int64_t n_new, int64_t d, int act_dtype,
                         const void* W, const float* bias, int overlap, int m, int c,
                         const int64_t* pos0, const int64_t* emit_from, void* state,
                         void* cache, void* cache_scales, int cache_layout, int64_t S,
                         void* ring, int64_t ring_w, int ring_layout, const dsv4_norm_rope_t* nr,
                         void* ws, size_t ws_bytes, void* stream);

/* Position held by row 0 of a window ring whose newest position is p_last:
 * floor((p_last - ring_w + 1) / ring_w) * ring_w (may be negative).  Host only. */
int64_t dsv4_swa_ring_pos0(int64_t p_last, int64_t ring_w);

/* Status text, and the last error message of the calling thread. */
const char* dsv4_status_string(int status);
const char* dsv4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSV4ATTN_H */
