"""InfLLM v2 block-sparse attention for MI355X (gfx950): Python side of the C ABI.

The compute path lives in libinfllmv2.so (hand-written HIP kernels); this
package only marshals arguments (see capi.py) and offers small helpers that
allocate outputs with torch and call the C entry points in order.
"""
from .capi import (  # noqa: F401
    EXPORTS, InfLLMv2Error, infllmv2_cfg, make_cfg, lib, LIB_PATH,
    infllmv2_pool_kernels, infllmv2_score_blocks, infllmv2_topk_blocks,
    infllmv2_sparse_attn_prefill, infllmv2_decode_workspace_bytes,
    infllmv2_sparse_attn_decode, infllmv2_sparse_attn_decode_scores,
    infllmv2_sparse_attn_decode_scores_noalloc, infllmv2_dense_attn,
    infllmv2_prefill_backward_workspace_bytes, infllmv2_sparse_attn_prefill_backward,
    infllmv2_sliding_window_attn, infllmv2_append_kv, infllmv2_score_blocks_varlen,
    infllmv2_decode_varlen_workspace_bytes, infllmv2_sparse_attn_decode_varlen,
    infllmv2_score_lse_workspace_bytes, infllmv2_score_blocks_lse,
    infllmv2_strerror, infllmv2_last_error,
)
from . import ops  # noqa: F401
