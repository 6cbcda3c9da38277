"""libdsv4attn: the DeepSeek-V4 CSA / HCA attention hot path for MI355X (gfx950).

The six calls (csa_compress, hca_compress, indexer_score, topk_select,
sparse_mqa_fwd, hca_dense_fwd), and the FP4-query variant of the indexer
(indexer_score_fp4q) and its FP8-query twin (indexer_score_fp8q), and the Q/KV RMSNorm + partial RoPE and output
rotation (q_norm_rope, kv_norm_rope, out_rope), and the query path and grouped
output projection on a bf16 MFMA GEMM (query_proj, output_proj, gemm_bf16_nt),
and the streaming decode-time compressors with the mirrored window ring
(stream_compress, stream_state_reset, swa_ring_pos0), are hand-written HIP
kernels behind the C ABI
of include/dsv4attn.h; this package is a thin ctypes binding over it.
"""
from ._lib import (BF16, EXPORTS, F32, ROW_BF16, ROW_F32, ROW_FP8_ROPE_BF16, ROW_MXFP4, Dsv4Error,
                   LIB_PATH, attn_plan, attn_workspace_size, compress_chunk, compress_chunk_nr_workspace_size, norm_rope, compressor, csa_compress, hca_compress, hca_dense_fwd,
                   indexer_score, indexer_score_fp4q, indexer_score_fp8q, indexer_topk, indexer_topk_workspace_size, kv_norm_rope, lib, out_rope, q_norm_rope,
                   gemm_bf16_nt, query_proj, query_proj_workspace_size, output_proj, output_proj_workspace_size, row_bytes, sparse_mqa_fwd, topk_select, topk_select_noalloc, topk_workspace_size,
                   stream_compress, stream_state_bytes, stream_state_reset, stream_workspace_size, swa_ring_pos0)

__all__ = ["BF16", "F32", "ROW_BF16", "ROW_F32", "ROW_FP8_ROPE_BF16", "ROW_MXFP4", "Dsv4Error", "EXPORTS",
           "LIB_PATH", "attn_plan", "attn_workspace_size", "compress_chunk", "compress_chunk_nr_workspace_size", "norm_rope", "compressor", "csa_compress", "hca_compress", "hca_dense_fwd",
           "indexer_score", "indexer_score_fp4q", "indexer_score_fp8q", "indexer_topk", "indexer_topk_workspace_size", "kv_norm_rope", "lib", "out_rope", "q_norm_rope",
           "gemm_bf16_nt", "query_proj", "query_proj_workspace_size", "output_proj", "output_proj_workspace_size", "row_bytes", "sparse_mqa_fwd", "topk_select", "topk_select_noalloc", "topk_workspace_size",
           "stream_compress", "stream_state_bytes", "stream_state_reset", "stream_workspace_size", "swa_ring_pos0"]
