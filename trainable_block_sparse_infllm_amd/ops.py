"""Call sequences over the C ABI: allocate outputs with torch, call the entry points in order.

Every step runs in the HIP library; these helpers only allocate and marshal.
bf16 tensors may be torch.bfloat16 or 16-bit integer tensors holding bf16 bits.
"""
from __future__ import annotations

import math

import torch

from . import capi


def _bf16_like(shape, ref):
    return torch.empty(shape, dtype=torch.bfloat16, device=ref.device)


def nblk(kv_cap: int, block: int = 64) -> int:
    return (kv_cap + block - 1) // block


class Workspace:
    """A reusable device buffer for the decode entry point (grown on demand)."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def kbar_shape(B: int, Hkv: int, kv_cap: int, D: int) -> tuple:
    """Kernel table [B][Hkv][ceil(nblk/32)][3][D/8][32][8]: tiles of 32 blocks, and inside
    a tile the 32 blocks' copies of each 16-byte piece adjacent."""
    return (B, Hkv, (nblk(kv_cap) + 31) // 32, 3, D // 8, 32, 8)


def pool_kernels(cfg, k, kv_cap, kv_len, first_block=0, kbar=None, stream=None):
    B, Hkv, _, D = k.shape
    if kbar is None:
        kbar = torch.zeros(kbar_shape(B, Hkv, kv_cap, D), dtype=torch.bfloat16, device=k.device)
    capi.infllmv2_pool_kernels(cfg, k, kv_cap, kv_len, first_block, kbar, stream)
    return kbar


def sparse_prefill(cfg, q, k, v, *, with_lse=True, stream=None):
    """Whole-sequence prefill: kernels -> fused score/top-K -> sparse attention."""
    B, Hq, T, D = q.shape
    kv_cap = k.shape[2]
    kbar = pool_kernels(cfg, k, kv_cap, T, stream=stream)
    idx = torch.empty((B, cfg.n_kv_heads, T, cfg.top_k), dtype=torch.int32, device=q.device)
    capi.infllmv2_topk_blocks(cfg, None, q, kbar, T, 0, 0, kv_cap, idx, stream)
    out = _bf16_like((B, Hq, T, D), q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if with_lse else None
    capi.infllmv2_sparse_attn_prefill(cfg, q, T, k, v, kv_cap, T, idx, out, lse, stream)
    return dict(kbar=kbar, idx=idx, out=out, lse=lse)


def sparse_prefill_backward(cfg, q, k, v, idx, out, lse, dout, *, kv_len=None, stream=None):
    """Gradients of the sparse prefill: returns dq [B][Hq][n_q][D], dk and dv
    [B][Hkv][kv_cap][D] (fp32; dk, dv rows past kv_len are zero here)."""
    B, Hq, n_q, D = q.shape
    kv_cap = k.shape[2]
    kv_len = n_q if kv_len is None else kv_len
    dq = torch.empty((B, Hq, n_q, D), dtype=torch.float32, device=q.device)
    dk = torch.zeros((B, cfg.n_kv_heads, kv_cap, D), dtype=torch.float32, device=q.device)
    dv = torch.zeros_like(dk)
    nbytes = capi.infllmv2_prefill_backward_workspace_bytes(cfg, n_q, kv_len)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    capi.infllmv2_sparse_attn_prefill_backward(cfg, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, dout,
                                               dq, dk, dv, ws, nbytes, stream)
    return dict(dq=dq, dk=dk, dv=dv)


def decode(cfg, q, k_cache, v_cache, kbar, kv_len, *, tree_mask=None, ws: Workspace | None = None,
           with_lse=True, stream=None):
    """n_q new tokens (tree nodes when tree_mask is given): scores -> top-K -> split attention."""
    B, Hq, n_q, D = q.shape
    kv_cap = k_cache.shape[2]
    is_tree = tree_mask is not None
    q_pos0 = kv_len - n_q        # a tree's nodes all score against the prefix P = kv_len - n_q
    scores = torch.empty((B, cfg.n_kv_heads, n_q, nblk(kv_cap)), dtype=torch.float32, device=q.device)
    capi.infllmv2_score_blocks(cfg, q, n_q, q_pos0, is_tree, kbar, kv_cap, scores, stream)
    idx = torch.empty((B, cfg.n_kv_heads, n_q, cfg.top_k), dtype=torch.int32, device=q.device)
    capi.infllmv2_topk_blocks(cfg, scores, None, None, n_q, q_pos0, is_tree, kv_cap, idx, stream)
    out = _bf16_like((B, Hq, n_q, D), q)
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device) if with_lse else None
    nbytes = capi.infllmv2_decode_workspace_bytes(cfg, n_q, kv_len)
    ws = ws or Workspace(q.device)
    buf = ws.get(nbytes)
    capi.infllmv2_sparse_attn_decode(cfg, q, n_q, k_cache, v_cache, kv_cap, kv_len, idx, tree_mask, out, lse,
                                     buf, buf.numel(), stream)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def decode_step(cfg, q, k_cache, v_cache, kbar, kv_len, *, ws: Workspace | None = None, with_lse=True,
                stream=None):
    """One single-token decode step: block scores, then selection and attention in one entry point."""
    B, Hq, n_q, D = q.shape
    if n_q != 1:
        raise ValueError("decode_step takes one new token per sequence")
    kv_cap = k_cache.shape[2]
    scores = torch.empty((B, cfg.n_kv_heads, 1, nblk(kv_cap)), dtype=torch.float32, device=q.device)
    capi.infllmv2_score_blocks(cfg, q, 1, kv_len - 1, 0, kbar, kv_cap, scores, stream)
    idx = torch.empty((B, cfg.n_kv_heads, 1, cfg.top_k), dtype=torch.int32, device=q.device)
    out = _bf16_like((B, Hq, 1, D), q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if with_lse else None
    nbytes = capi.infllmv2_decode_workspace_bytes(cfg, 1, kv_len)
    ws = ws or Workspace(q.device)
    buf = ws.get(nbytes)
    capi.infllmv2_sparse_attn_decode_scores(cfg, q, k_cache, v_cache, kv_cap, kv_len, scores, idx, out, lse,
                                            buf, buf.numel(), stream)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def dense(cfg, q, k, v, kv_len, *, causal=True, with_lse=True, stream=None):
    B, Hq, n_q, D = q.shape
    out = _bf16_like((B, Hq, n_q, D), q)
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device) if with_lse else None
    capi.infllmv2_dense_attn(cfg, q, n_q, k, v, k.shape[2], kv_len, causal, out, lse, stream)
    return dict(out=out, lse=lse)


def score_blocks_lse(cfg, q, kbar, q_pos0, kv_cap, *, is_tree=False, ws: Workspace | None = None, stream=None):
    """LSE-normalized block scores [B][Hkv][n_q][kv_cap/64] (the layout of the raw scores)."""
    B, Hq, n_q, D = q.shape
    scores = torch.empty((B, cfg.n_kv_heads, n_q, nblk(kv_cap)), dtype=torch.float32, device=q.device)
    nbytes = capi.infllmv2_score_lse_workspace_bytes(cfg, n_q, kv_cap)
    ws = ws or Workspace(q.device)
    buf = ws.get(nbytes)
    capi.infllmv2_score_blocks_lse(cfg, q, n_q, q_pos0, is_tree, kbar, kv_cap, scores, buf, buf.numel(), stream)
    return scores


def decode_step_lse(cfg, q, k_cache, v_cache, kbar, kv_len, *, ws: Workspace | None = None, with_lse=True,
                    stream=None):
    """A single-token decode step whose top-K uses the LSE-normalized scores."""
    B, Hq, n_q, D = q.shape
    if n_q != 1:
        raise ValueError("decode_step_lse takes one new token per sequence")
    kv_cap = k_cache.shape[2]
    ws = ws or Workspace(q.device)
    scores = score_blocks_lse(cfg, q, kbar, kv_len - 1, kv_cap, ws=ws, stream=stream)
    idx = torch.empty((B, cfg.n_kv_heads, 1, cfg.top_k), dtype=torch.int32, device=q.device)
    out = _bf16_like((B, Hq, 1, D), q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if with_lse else None
    nbytes = capi.infllmv2_decode_workspace_bytes(cfg, 1, kv_len)
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    capi.infllmv2_sparse_attn_decode_scores(cfg, q, k_cache, v_cache, kv_cap, kv_len, scores, idx, out, lse,
                                            buf, nbytes, stream)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def append_kv(cfg, k_new, v_new, k_cache, v_cache, kbar=None, *, kv_len=None, kv_lens=None, stream=None):
    """Write k_new, v_new [B][Hkv][n_new][D] at each sequence's length (kv_lens, a device int64
    tensor [B], or the scalar kv_len) and pool the blocks this completes into kbar."""
    if (kv_len is None) == (kv_lens is None):
        raise ValueError("give exactly one of kv_len and kv_lens")
    capi.infllmv2_append_kv(cfg, k_new, v_new, k_new.shape[2], k_cache, v_cache, k_cache.shape[2], kv_lens,
                            0 if kv_len is None else kv_len, kbar, stream)


def decode_step_varlen(cfg, q, k_cache, v_cache, kbar, kv_lens, kv_len_max, *, ws: Workspace | None = None,
                       with_lse=True, stream=None):
    """One decode step for a batch of variable lengths: sequence b's new token sits at
    kv_lens[b] - 1 (device int64 [B], at most kv_len_max)."""
    B, Hq, n_q, D = q.shape
    if n_q != 1:
        raise ValueError("decode_step_varlen takes one new token per sequence")
    kv_cap = k_cache.shape[2]
    scores = torch.empty((B, cfg.n_kv_heads, 1, nblk(kv_cap)), dtype=torch.float32, device=q.device)
    capi.infllmv2_score_blocks_varlen(cfg, q, kv_lens, kbar, kv_cap, scores, stream)
    idx = torch.empty((B, cfg.n_kv_heads, 1, cfg.top_k), dtype=torch.int32, device=q.device)
    out = _bf16_like((B, Hq, 1, D), q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if with_lse else None
    nbytes = capi.infllmv2_decode_varlen_workspace_bytes(cfg, kv_len_max)
    ws = ws or Workspace(q.device)
    buf = ws.get(nbytes)
    capi.infllmv2_sparse_attn_decode_varlen(cfg, q, k_cache, v_cache, kv_cap, kv_lens, kv_len_max, scores,
                                            idx, out, lse, buf, buf.numel(), stream)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


def sliding_window(cfg, q, k, v, kv_len, window, *, with_lse=True, stream=None):
    """Causal attention of each query over the last `window` positions up to its own."""
    B, Hq, n_q, D = q.shape
    out = _bf16_like((B, Hq, n_q, D), q)
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=q.device) if with_lse else None
    capi.infllmv2_sliding_window_attn(cfg, q, n_q, k, v, k.shape[2], kv_len, window, out, lse, stream)
    return dict(out=out, lse=lse)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
