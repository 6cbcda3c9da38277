// Host-side launchers of the libdsv4attn kernels (internal; the public C ABI
// is include/dsv4attn.h).  Every launcher assumes validated arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define DSV4_HD __host__ __device__
#else
#define DSV4_HD
#endif

namespace dsv4 {

enum { ACT_F32 = 0, ACT_BF16 = 1 };
enum { ROW_F32 = 0, ROW_BF16 = 1, ROW_FP8 = 2, ROW_MXFP4 = 3 };
constexpr int ROPE_DIMS = 64;   // the last 64 dims of a KV row stay bf16

// number of entries visible at position p for ratio m: entries s < floor((p+1)/m)
// satisfy m*(s+1) <= p+1
DSV4_HD inline int64_t visible_count(int64_t p, int64_t m, int64_t S) {
  int64_t v = (p + 1) / m;
  if (v < 0) v = 0;
  return v < S ? v : S;
}

struct CompressArgs {
  const void* H;        // [n_left + n, d]
  int64_t n_left, n, d;
  int act;              // ACT_F32 / ACT_BF16
  const void* W;        // [nmat * c, d]
  const float* bias;    // CSA [2, m, c]; HCA [m', c]
  int m, c;
  int64_t block0;       // CSA: absolute index of the first emitted entry
  void* comp;           // [n/m rows]
  uint8_t* comp_scales; // MXFP4 scales [n/m, c/32]
  int comp_layout;
  void* raw;            // [n rows] or null
  int raw_layout;
};

hipError_t launch_csa_compress(const CompressArgs& a, hipStream_t s);
hipError_t launch_hca_compress(const CompressArgs& a, hipStream_t s);
// the compressors of one chunk in one launch (any pointer may be null)
bool compress_fused_ok(const CompressArgs* kv, const CompressArgs* ki, const CompressArgs* hca);
hipError_t launch_compress_fused(const CompressArgs* kv, const CompressArgs* ki, const CompressArgs* hca,
                                 hipStream_t s);

struct IndexerArgs {
  const void* qI;       // [B, nq, hI, cI]
  int q_dtype;
  const float* wI;      // [B, nq, hI]
  const void* keys;     // [B, S, row]
  const uint8_t* k_scales;
  int k_layout;
  int64_t B, nq;
  int hI, cI;
  int64_t S;
  int m;
  float* scores;        // [B, nq, S]
  int qfmt;             // 0: bf16 / f32 queries; 4 or 8: quantised to MXFP4 or MXFP8 (keys MXFP4)
  // candidate mode (cand != null; bf16 queries, MFMA path): no scores are
  // stored; a visible score >= lval[row] (a finite float or -inf) is kept as
  // its composite in cand[(row * splits + split) * cap + i] and the count of
  // each (row, split) goes to ccount[row * splits + split] (row = b nq + t,
  // split = the key range of one block, splits from indexer_grid)
  uint64_t* cand;
  uint32_t* ccount;
  const float* lval;
  int cap;
  // restricted mode (row_flags != null): a block computes (and stores scores)
  // only if one of its rows has a non-zero flag
  const int* row_flags;
  // key s of batch entry b is row b kbatch + koff + s kstride of keys (and
  // k_scales); kbatch 0 means S, kstride 0 means 1 (a strided sample of a key
  // array is scored in place)
  int64_t kbatch, koff;
  int kstride;
};
__host__ __device__ inline int64_t key_row(const IndexerArgs& a, int64_t b, int64_t s) {
  const int64_t kb = a.kbatch ? a.kbatch : a.S;
  return b * kb + a.koff + s * (a.kstride ? a.kstride : 1);
}

// Per-batch absolute positions travel to the kernels by value: a launch covers
// at most MAXB batch entries (launchers loop over larger batches).
constexpr int MAXB = 64;
struct PosTable {
  int64_t q_pos0[MAXB];
  int64_t win_pos0[MAXB];
};

// q_pos0: host array [B]
hipError_t launch_indexer(const IndexerArgs& a, const int64_t* q_pos0, hipStream_t s);

// ---- indexer planning (plan.cpp; host only)
constexpr int IDX_KT = 256;       // keys per LDS tile of the MFMA indexer
// the MFMA path applies (bf16 queries, 32 heads, cI 32/64/128, BF16 or MXFP4 keys)
bool indexer_mfma_ok(const IndexerArgs& a);
// grid of one MFMA-indexer launch over nb batch entries: query blocks of qb
// queries, each split into `splits` key ranges of tps tiles
struct IndexerGrid {
  int qb;
  int64_t qblocks;
  int splits, tps;
};
IndexerGrid indexer_grid(const IndexerArgs& a, int nb);

// ---- top-k planning (plan.cpp; host only)
constexpr int SK_KMAX = 1024;     // largest k of the streaming and histogram selects
constexpr int HS_BIN = 2048;      // histogram bins of the histogram select (11-bit digits)
constexpr int HS_COARSE = 64;     // every 32nd bin's suffix count, stored again after a part's bins
constexpr int HS_SUF = HS_BIN + HS_COARSE;   // words per part of the suffix counts
constexpr int HS_CAP = 8192;      // threshold-bin candidates of the histogram select
constexpr int TK_MAX_CAND = 16384;   // part winners a stage-2 merge holds in LDS

enum { TOPK_STREAM = 0, TOPK_STAGE = 1, TOPK_HIST = 2 };
struct TopkPlan {
  int kind;          // TOPK_*
  int part, nparts;  // scores per part, parts per row
  bool supported;
  size_t bytes;      // workspace the launch uses
  // histogram select: byte offsets of its workspace arrays
  size_t o_suf, o_meta, o_win, o_cand;
};
// plan for `rows` rows (of one launch: at most MAXB batch entries) of S scores
TopkPlan topk_make_plan(int64_t rows, int64_t S, int k);
hipError_t launch_topk(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                       const int64_t* q_pos0, int k, int32_t* idx, void* ws, const TopkPlan& plan,
                       hipStream_t s);
// row_flags (optional, [launch rows]): rows with a zero flag are skipped
hipError_t launch_topk_rows(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                            const int64_t* q_pos0, int k, int32_t* idx, void* ws, const TopkPlan& plan,
                            const int* row_flags, hipStream_t s);

// ---- index scores and top-k in one call (plan.cpp plans, topk.hip launches).
// Sampled-threshold path: every 32nd key (keys 32 j + 31) is scored first;
// a value at or below each row's ks-th best sample score is its threshold,
// the full pass keeps only scores at or above it as composites, and a per-row
// select takes the top k of those.  A row whose kept count is below
// min(k, visible) or whose lists overflowed is flagged, and its scores are
// recomputed in full and selected by the plain top-k, so the result is always
// the top-k of the full score row.
constexpr int IT_STRIDE = 32;     // one sample key per 32 keys
constexpr int IT_SELCAP = 3584;   // candidates one select block holds in LDS
struct IdxTopkPlan {
  bool fused;        // sampled-threshold path (else: full scores, then top-k)
  int ks;            // sample rank of the threshold
  int cap;           // candidate slots per (row, key split)
  IndexerGrid grid;  // of the full pass
  int64_t Ss;        // sample keys per batch entry
  TopkPlan tk_sample, tk_full;
  size_t o_sscore, o_sidx, o_stk, o_lkey, o_cand, o_cnt, o_flags, o_scores, o_ftk;
  size_t bytes;
};
// plan of one launch slice (a.B <= MAXB batch entries)
IdxTopkPlan idxtopk_make_plan(const IndexerArgs& a, int k);
// workspace of a whole call (the largest slice plan)
size_t idxtopk_workspace(const IndexerArgs& a, int k);
hipError_t launch_indexer_topk(const IndexerArgs& a, const int64_t* q_pos0, int k, int32_t* idx, void* ws,
                               hipStream_t s);

// the allocation-free top-k call's workspace: a static device array per GPU
constexpr size_t TOPK_SCRATCH_BYTES = (size_t)16 << 20;
// its device address on the current GPU (looked up once per device)
hipError_t topk_scratch_ptr(void** ptr);

struct AttnArgs {
  const void* q;        // [B, nq, nh, c]
  int q_dtype;
  int64_t B, nq;
  int nh, c;
  const void* kv_comp;  // [B, S, row]
  int kv_layout;
  int64_t S;
  const int32_t* idx;   // sparse: [B, nq, k]; dense: null
  int k;
  int ratio;            // dense: m'
  const void* kv_win;   // [B, W, row]
  int64_t W;
  int n_win;
  const float* sink;    // [nh] or null
  float scale;
  void* out;            // [B, nq, nh, c]
  void* ws;
  size_t ws_bytes;
  // output rotation in the store (rot_dims 0: none): the last rot_dims
  // channels of each output row, as pairs, rotated by -(query position),
  // exactly as the separate output-rotation call does to the stored row
  float rot_theta;
  int rot_dims;
};

// Q/KV RMSNorm + partial RoPE, and the output rotation (normrope.hip)
struct QPrepArgs {
  const void* in;       // [B, nq, nh, c]
  void* out;            // same shape and dtype (may alias in)
  int dtype;            // ACT_F32 | ACT_BF16
  int64_t B, nq;
  int nh, c;
  const float* gamma;   // [c] or null (1); unused for the output rotation
  float eps, theta;
  int R;                // rotated dims (the last R of each row)
  int out_rot;          // 1: no norm, rotate by -position, write the rotated dims only
};
struct KvPrepArgs {
  const void* in;       // [B, n, row] in ROW_F32 | ROW_BF16
  int in_layout;
  void* out;            // [B, n, row] in ROW_F32 | ROW_BF16 | ROW_FP8
  int out_layout;
  int64_t B, n;
  int c;
  const float* gamma;
  float eps, theta;
  int R;
  int64_t pos_stride;   // row i of batch entry b sits at pos0[b] + pos_stride * i
  int norm;             // 1: RMSNorm (times gamma) before the rotation; 0: rotation only
};
hipError_t launch_q_prep(const QPrepArgs& a, const int64_t* q_pos0, hipStream_t s);
hipError_t launch_kv_prep(const KvPrepArgs& a, const int64_t* pos0, hipStream_t s);

// streaming compressors and the window ring (stream.hip)
struct StreamArgs {
  const void* H;        // [B, n_new, d]
  int act;
  int64_t d;
  const void* W;        // [nmat * c, d]
  const float* bias;    // CSA [2, m, c]; HCA [m, c]
  int nmat, c, m, overlap;
  int64_t B, n_new;
  float* part;          // workspace: [KS, B * n_new, nmat * c] projection partials
  void* state;          // [B] x state_bytes
  int64_t state_bytes;
  void* cache;          // [B, S, row] or null
  uint8_t* cache_scales;
  int cache_layout;
  int64_t S;
  void* ring;           // [B, 2 ring_w, row] or null
  int64_t ring_w;
  int ring_layout;
  int norm;             // RMSNorm (gamma, eps) before the rotation
  const float* gamma;
  float eps, theta;
  int rope_dims;
};
// sizes and the split of d for the projection partials (plan.cpp; host only)
constexpr int STREAM_SP_COLS = 64;      // projection: output columns per block
constexpr int STREAM_META_BYTES = 256;  // header of a sequence's state
void stream_split(int64_t NC, int64_t d, int* ks, int64_t* kslice);
size_t stream_state_bytes(int overlap, int m, int c);
size_t stream_ws_bytes(int64_t rows, int overlap, int c, int64_t d);
hipError_t launch_stream_reset(void* state, int64_t B, int overlap, int m, int c, hipStream_t s);
hipError_t launch_stream(const StreamArgs& a, const int64_t* pos0, const int64_t* emit_from, hipStream_t s);

// bf16 GEMM C = A B^T, fp32 accumulation (gemm.hip)
struct GemmArgs {
  const void* A;        // [M, K] bf16, row stride lda elements
  int64_t lda, sA;      // sA: batch stride (elements)
  const void* B;        // [N, K] bf16
  int64_t ldb, sB;
  void* C;              // [M, N] bf16 or fp32
  int64_t ldc, sC;
  int c_f32;
  int64_t M, N, K, batch;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// ---- attention planning (plan.cpp; host only)
// Kernel-visible part of a plan: how queries form blocks and how key slots split.
struct AttnPlan {
  int64_t units_per_b;   // query groups per batch entry
  int qpw;               // queries per group
  int chunk;             // key slots per split (multiple of 32)
  int max_splits;        // grid.y
  int dense;
  float scale_log2;
};
enum { ATTN_GENERIC = 0, ATTN_MFMA = 1, ATTN_F8 = 2 };
constexpr int ATTN_SIDX_CAP = 2048;   // index-list slots a sparse MFMA block caches in LDS
constexpr int ATTN_MAX_SPLITS = 16;   // key splits of one attention unit (the merge holds them all in registers)
constexpr int ATTN_QPW_MAX = 8;       // most queries one MFMA block serves
struct AttnLaunchPlan {
  int path;              // ATTN_*
  int nrg;               // row groups of 32 rows per block (MFMA paths)
  AttnPlan pl;
  size_t ws_bytes;       // workspace bytes the launch writes (split partials)
};
// Key slots of the largest query group of a call: compressed entries of its
// last query (dense) or k (sparse), plus the window positions its queries span.
int64_t attn_group_slots(const AttnArgs& a, const int64_t* q_pos0, bool dense);
// The plan of a call whose groups have at most `slots` key slots.  ws_bytes is
// non-decreasing in `slots`, so a bound on the slots bounds the workspace.
AttnLaunchPlan attn_make_plan(const AttnArgs& a, bool dense, int64_t slots);
// Workspace bound for any call with these sizes whose queries see at most
// max_keys compressed entries plus window rows each (every path and layout).
size_t attn_workspace_bound(int64_t B, int64_t nq, int nh, int c, int64_t max_keys, bool dense);
hipError_t launch_attn(const AttnArgs& a, const int64_t* q_pos0, const int64_t* win_pos0,
                       const AttnLaunchPlan& plan, hipStream_t s);

}  // namespace dsv4
