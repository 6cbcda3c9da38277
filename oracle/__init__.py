"""float64 CPU oracle for the CSA / HCA hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from . import codecs, stream
from .dsv4 import (softmax_pool, csa_compress, csa_pool_weights, hca_compress,
                   visible_count, indexer_score, indexer_score_fp4q, indexer_score_fp8q, topk_select, core_attention,
                   window_rows, sparse_mqa, hca_dense, rmsnorm, rope_last, q_norm_rope,
                   kv_norm_rope, entry_positions, out_rope, query_proj, output_proj)

__all__ = ["codecs", "stream", "softmax_pool", "csa_compress", "csa_pool_weights", "hca_compress",
           "visible_count", "indexer_score", "indexer_score_fp4q", "indexer_score_fp8q", "topk_select", "core_attention",
           "window_rows", "sparse_mqa", "hca_dense", "rmsnorm", "rope_last", "q_norm_rope",
           "kv_norm_rope", "entry_positions", "out_rope", "query_proj", "output_proj"]
