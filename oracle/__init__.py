"""CPU oracle (numpy, float64) for chunk attention over a KV cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library itself.  It shares no code
with the HIP path.
"""
from .chunk_attention import (  # noqa: F401
    NEG_INF, attention, block_mean, block_score_topk, block_spans, block_tokens,
    build_kv_index, chunk_attn_blocks, chunk_attn_dense, chunk_attn_varlen,
    chunk_mean_query, lse_merge, lse_merge_bshd, mla_chunk_attn, pack_ragged, persistent_update,
    sparse_selection,
)
