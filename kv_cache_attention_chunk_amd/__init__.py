"""MI355X-native chunk attention over a streaming video generator's KV cache.

The calls below bind the C ABI of libchunkattn.so (include/chunkattn.h):
dense / block-list / ragged / mixed-mode chunk attention emitting O and LSE,
one-pass PBSA (shared + per-query-block block lists), the LSE merge of a
local and a history branch, block means, coarse block scoring with top-K,
and PBSA block-list assembly.  Importing this package does not load the
library; the first call does, and fails if it is not built.
"""
from .api import (  # noqa: F401
    block_mean, block_mean_pair, block_score_topk, block_score_topk_batch,
    block_score_topk_lists, block_sparse_fwd, block_sparse_workspace, build_kv_index, cast_bf16_to_f16,
    chunk_attn_dual_fwd, chunk_attn_fwd, chunk_attn_mixed_fwd, chunk_attn_pbsa_fwd,
    chunk_attn_varlen_fwd, lse_merge, mla_chunk_attn, num_blocks, pack_plan, pack_ragged,
    persistent_update, workspace_bytes,
)

__all__ = [
    "chunk_attn_fwd", "chunk_attn_dual_fwd", "chunk_attn_pbsa_fwd", "chunk_attn_varlen_fwd",
    "chunk_attn_mixed_fwd", "lse_merge", "block_mean", "block_mean_pair", "block_score_topk",
    "block_score_topk_batch", "block_score_topk_lists", "build_kv_index", "block_sparse_fwd",
    "block_sparse_workspace",
    "num_blocks", "pack_plan", "pack_ragged", "persistent_update", "workspace_bytes",
    "mla_chunk_attn", "cast_bf16_to_f16",
]
