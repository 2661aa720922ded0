"""DeepSeek-V3.2 sparse attention hot path on MI355X (gfx950).

Lightning-indexer scores -> per-query top-K -> absorbed sparse latent
attention, as hand-written HIP kernels in ``libdsa.so`` behind the C ABI of
``include/dsa.h``.  This package is the thin Python binding of that ABI.
"""
from ._binding import (DSA_BF16, DSA_F32, DSA_FP8_E4M3, ENTRY_FORWARD, ENTRY_SPARSE_MLA,
                       ENTRY_INDEXER_TOPK, ENTRY_TOPK, DsaError, DsaShape, dsa_absorb_output, dsa_absorb_prepare,
                       dsa_absorb_query, dsa_cache_fill, dsa_forward, dsa_forward_noalloc, dsa_forward_ragged,
                       dsa_indexer_query, dsa_indexer_scores, dsa_indexer_topk, dsa_indexer_scores_ragged,
                       dsa_output_projection, dsa_sparse_mla_fwd, dsa_timing_begin, dsa_timing_end, dsa_topk, lib,
                       make_shape, workspace_bytes)

__all__ = ["DSA_BF16", "DSA_F32", "DSA_FP8_E4M3", "ENTRY_FORWARD", "ENTRY_SPARSE_MLA",
           "ENTRY_INDEXER_TOPK", "ENTRY_TOPK", "DsaError", "DsaShape", "dsa_absorb_output", "dsa_absorb_prepare",
           "dsa_absorb_query", "dsa_cache_fill", "dsa_forward", "dsa_forward_noalloc", "dsa_forward_ragged",
           "dsa_indexer_query", "dsa_indexer_scores", "dsa_indexer_topk", "dsa_indexer_scores_ragged",
           "dsa_output_projection", "dsa_sparse_mla_fwd", "dsa_timing_begin", "dsa_timing_end", "dsa_topk", "lib",
           "make_shape", "workspace_bytes"]
