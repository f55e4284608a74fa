"""KPool-indexed DeepSeek Sparse Attention forward for AMD MI355X (gfx950).

The compute lives in ``libkpool.so`` (hand-written HIP kernels behind the C ABI
of ``include/kpool.h``); this package is its Python binding.
"""
from ._lib import (KpoolError, dsa_forward, dsa_forward_shared, indexer_rotate_quant, indexer_score_topk,
                   indexer_score_topk_noalloc, indexer_score_topk_paged, indexer_topk_from_scores, kp_check_inputs,
                   kp_indexer_paged_workspace_bytes, kp_indexer_workspace_bytes, kp_mla_bwd_workspace_bytes,
                   kp_mla_fwd_workspace_bytes,
                   kp_row_width, kp_version, kpool_build, kpool_build_from, kpool_update_paged, lib, sparse_mla_bwd,
                   sparse_mla_fwd)

__all__ = ["KpoolError", "dsa_forward", "dsa_forward_shared", "indexer_rotate_quant", "indexer_score_topk",
           "indexer_score_topk_noalloc", "indexer_score_topk_paged", "indexer_topk_from_scores", "kp_check_inputs",
           "kp_indexer_paged_workspace_bytes", "kp_indexer_workspace_bytes", "kp_mla_bwd_workspace_bytes",
           "kp_mla_fwd_workspace_bytes",
           "kp_row_width", "kp_version", "kpool_build", "kpool_build_from", "kpool_update_paged", "lib",
           "sparse_mla_bwd", "sparse_mla_fwd"]
