// Host-side launchers of the libdsv4attn kernels (internal; the public C ABI
// is include/dsv4attn.h).  Every launcher assumes validated arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsv4 {

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
};

// Per-batch absolute positions travel to the kernels by value: a launch covers
// at most MAXB batch entries (launchers loop over larger batches).
constexpr int MAXB = 64;
struct PosTable {
  int64_t q_pos0[MAXB];
  int64_t win_pos0[MAXB];
};

// q_pos0: host array [B]
hipError_t launch_indexer(const IndexerArgs& a, const int64_t* q_pos0, hipStream_t s);

size_t topk_workspace_bytes(int64_t rows, int64_t S, int k);
bool topk_supported(int64_t rows, int64_t S, int k);
hipError_t launch_topk(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                       const int64_t* q_pos0, int k, int32_t* idx, void* ws, hipStream_t s);

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

size_t attn_workspace_bytes(int64_t B, int64_t nq, int nh, int c, int64_t max_keys, bool dense);
hipError_t launch_attn(const AttnArgs& a, const int64_t* q_pos0, const int64_t* win_pos0,
                       bool dense, hipStream_t s);

}  // namespace dsv4
