"""Thin ctypes binding over libinfllmv2.so (C ABI in include/infllmv2.h).

One Python function per exported C function, with the same name and argument
order. Tensor arguments may be torch tensors (their data pointer is passed),
plain integers (raw device addresses) or None (NULL). Streams default to
torch's current stream. Nothing here computes: a missing library raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinfllmv2.so")

OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR = 0, -1, -2, -3, -4

EXPORTS = [
    "infllmv2_pool_kernels", "infllmv2_score_blocks", "infllmv2_topk_blocks",
    "infllmv2_sparse_attn_prefill", "infllmv2_decode_workspace_bytes",
    "infllmv2_sparse_attn_decode", "infllmv2_sparse_attn_decode_scores",
    "infllmv2_sparse_attn_decode_scores_noalloc", "infllmv2_dense_attn",
    "infllmv2_prefill_backward_workspace_bytes", "infllmv2_sparse_attn_prefill_backward",
    "infllmv2_sliding_window_attn", "infllmv2_append_kv", "infllmv2_score_blocks_varlen",
    "infllmv2_decode_varlen_workspace_bytes", "infllmv2_sparse_attn_decode_varlen",
    "infllmv2_score_lse_workspace_bytes", "infllmv2_score_blocks_lse",
    "infllmv2_strerror",
    "infllmv2_last_error",
]


class InfLLMv2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


class infllmv2_cfg(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_size", C.c_int32), ("kernel_size", C.c_int32),
                ("kernel_stride", C.c_int32), ("top_k", C.c_int32), ("dense_threshold", C.c_int32),
                ("softmax_scale", C.c_float)]


def make_cfg(batch, n_q_heads, n_kv_heads, head_dim, top_k=16, dense_threshold=0,
             softmax_scale=0.0, block_size=64, kernel_size=32, kernel_stride=16) -> infllmv2_cfg:
    return infllmv2_cfg(batch, n_q_heads, n_kv_heads, head_dim, block_size, kernel_size,
                        kernel_stride, top_k, dense_threshold, float(softmax_scale))


_lib = None


def lib():
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m trainable_block_sparse_infllm_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        cfg = C.POINTER(infllmv2_cfg)
        sig = {
            "infllmv2_pool_kernels": (i32, [cfg, P, i64, i64, i64, P, P]),
            "infllmv2_score_blocks": (i32, [cfg, P, i32, i64, i32, P, i64, P, P]),
            "infllmv2_topk_blocks": (i32, [cfg, P, P, P, i32, i64, i32, i64, P, P]),
            "infllmv2_sparse_attn_prefill": (i32, [cfg, P, i32, P, P, i64, i64, P, P, P, P]),
            "infllmv2_decode_workspace_bytes": (sz, [cfg, i32, i64]),
            "infllmv2_sparse_attn_decode": (i32, [cfg, P, i32, P, P, i64, i64, P, P, P, P, P, sz, P]),
            "infllmv2_sparse_attn_decode_scores": (i32, [cfg, P, P, P, i64, i64, P, P, P, P, P, sz, P]),
            "infllmv2_sparse_attn_decode_scores_noalloc": (i32, [cfg, P, P, P, i64, i64, P, P, P, P, P]),
            "infllmv2_dense_attn": (i32, [cfg, P, i32, P, P, i64, i64, i32, P, P, P]),
            "infllmv2_sliding_window_attn": (i32, [cfg, P, i32, P, P, i64, i64, i64, P, P, P]),
            "infllmv2_append_kv": (i32, [cfg, P, P, i32, P, P, i64, P, i64, P, P]),
            "infllmv2_score_lse_workspace_bytes": (C.c_size_t, [cfg, i32, i64]),
            "infllmv2_score_blocks_lse": (i32, [cfg, P, i32, i64, i32, P, i64, P, P, C.c_size_t, P]),
            "infllmv2_score_blocks_varlen": (i32, [cfg, P, P, P, i64, P, P]),
            "infllmv2_decode_varlen_workspace_bytes": (C.c_size_t, [cfg, i64]),
            "infllmv2_sparse_attn_decode_varlen": (i32, [cfg, P, P, P, i64, P, i64, P, P, P, P, P,
                                                         C.c_size_t, P]),
            "infllmv2_prefill_backward_workspace_bytes": (sz, [cfg, i32, i64]),
            "infllmv2_sparse_attn_prefill_backward": (i32, [cfg, P, i32, P, P, i64, i64, P, P, P, P,
                                                            P, P, P, P, sz, P]),
            "infllmv2_strerror": (C.c_char_p, [i32]),
            "infllmv2_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(x):
    """Device pointer of a tensor / raw int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != OK:
        raise InfLLMv2Error(rc, lib().infllmv2_last_error().decode())


def infllmv2_pool_kernels(cfg, k, kv_cap, kv_len, first_block, kbar, stream=None):
    _check(lib().infllmv2_pool_kernels(C.byref(cfg), _p(k), kv_cap, kv_len, first_block, _p(kbar), _s(stream)))


def infllmv2_score_blocks(cfg, q, n_q, q_pos0, is_tree, kbar, kv_cap, scores, stream=None):
    _check(lib().infllmv2_score_blocks(C.byref(cfg), _p(q), n_q, q_pos0, int(is_tree), _p(kbar), kv_cap,
                                       _p(scores), _s(stream)))


def infllmv2_topk_blocks(cfg, scores, q, kbar, n_q, q_pos0, is_tree, kv_cap, idx, stream=None):
    _check(lib().infllmv2_topk_blocks(C.byref(cfg), _p(scores), _p(q), _p(kbar), n_q, q_pos0, int(is_tree),
                                      kv_cap, _p(idx), _s(stream)))


def infllmv2_sparse_attn_prefill(cfg, q, n_q, k, v, kv_cap, kv_len, idx, out, lse=None, stream=None):
    _check(lib().infllmv2_sparse_attn_prefill(C.byref(cfg), _p(q), n_q, _p(k), _p(v), kv_cap, kv_len, _p(idx),
                                              _p(out), _p(lse), _s(stream)))


def infllmv2_decode_workspace_bytes(cfg, n_q, kv_len) -> int:
    return int(lib().infllmv2_decode_workspace_bytes(C.byref(cfg), n_q, kv_len))


def infllmv2_sparse_attn_decode(cfg, q, n_q, k_cache, v_cache, kv_cap, kv_len, idx, tree_mask, out, lse,
                                workspace, workspace_bytes, stream=None):
    _check(lib().infllmv2_sparse_attn_decode(C.byref(cfg), _p(q), n_q, _p(k_cache), _p(v_cache), kv_cap, kv_len,
                                             _p(idx), _p(tree_mask), _p(out), _p(lse), _p(workspace),
                                             workspace_bytes, _s(stream)))


def infllmv2_sparse_attn_decode_scores(cfg, q, k_cache, v_cache, kv_cap, kv_len, scores, idx_out, out, lse,
                                       workspace, workspace_bytes, stream=None):
    _check(lib().infllmv2_sparse_attn_decode_scores(C.byref(cfg), _p(q), _p(k_cache), _p(v_cache), kv_cap,
                                                    kv_len, _p(scores), _p(idx_out), _p(out), _p(lse),
                                                    _p(workspace), workspace_bytes, _s(stream)))


def infllmv2_sparse_attn_decode_scores_noalloc(cfg, q, k_cache, v_cache, kv_cap, kv_len, scores, idx_out, out,
                                               lse, stream=None):
    _check(lib().infllmv2_sparse_attn_decode_scores_noalloc(C.byref(cfg), _p(q), _p(k_cache), _p(v_cache),
                                                            kv_cap, kv_len, _p(scores), _p(idx_out), _p(out),
                                                            _p(lse), _s(stream)))


def infllmv2_dense_attn(cfg, q, n_q, k, v, kv_cap, kv_len, causal, out, lse=None, stream=None):
    _check(lib().infllmv2_dense_attn(C.byref(cfg), _p(q), n_q, _p(k), _p(v), kv_cap, kv_len, int(causal),
                                     _p(out), _p(lse), _s(stream)))


def infllmv2_sliding_window_attn(cfg, q, n_q, k, v, kv_cap, kv_len, window, out, lse=None, stream=None):
    _check(lib().infllmv2_sliding_window_attn(C.byref(cfg), _p(q), n_q, _p(k), _p(v), kv_cap, kv_len,
                                              int(window), _p(out), _p(lse), _s(stream)))


def infllmv2_prefill_backward_workspace_bytes(cfg, n_q, kv_len) -> int:
    return int(lib().infllmv2_prefill_backward_workspace_bytes(C.byref(cfg), n_q, kv_len))


def infllmv2_sparse_attn_prefill_backward(cfg, q, n_q, k, v, kv_cap, kv_len, idx, out, lse, dout, dq, dk,
                                          dv, workspace, workspace_bytes, stream=None):
    _check(lib().infllmv2_sparse_attn_prefill_backward(
        C.byref(cfg), _p(q), n_q, _p(k), _p(v), kv_cap, kv_len, _p(idx), _p(out), _p(lse), _p(dout),
        _p(dq), _p(dk), _p(dv), _p(workspace), workspace_bytes, _s(stream)))


def infllmv2_strerror(status: int) -> str:
    return lib().infllmv2_strerror(status).decode()


def infllmv2_last_error() -> str:
    return lib().infllmv2_last_error().decode()


def infllmv2_append_kv(cfg, k_new, v_new, n_new, k_cache, v_cache, kv_cap, kv_lens, kv_len, kbar,
                       stream=None):
    _check(lib().infllmv2_append_kv(C.byref(cfg), _p(k_new), _p(v_new), n_new, _p(k_cache), _p(v_cache),
                                    kv_cap, _p(kv_lens), kv_len, _p(kbar), _s(stream)))


def infllmv2_score_blocks_varlen(cfg, q, kv_lens, kbar, kv_cap, scores, stream=None):
    _check(lib().infllmv2_score_blocks_varlen(C.byref(cfg), _p(q), _p(kv_lens), _p(kbar), kv_cap,
                                              _p(scores), _s(stream)))


def infllmv2_decode_varlen_workspace_bytes(cfg, kv_len_max):
    return lib().infllmv2_decode_varlen_workspace_bytes(C.byref(cfg), kv_len_max)


def infllmv2_sparse_attn_decode_varlen(cfg, q, k_cache, v_cache, kv_cap, kv_lens, kv_len_max, scores,
                                       idx_out, out, lse, workspace, workspace_bytes, stream=None):
    _check(lib().infllmv2_sparse_attn_decode_varlen(C.byref(cfg), _p(q), _p(k_cache), _p(v_cache), kv_cap,
                                                    _p(kv_lens), kv_len_max, _p(scores), _p(idx_out),
                                                    _p(out), _p(lse), _p(workspace), workspace_bytes,
                                                    _s(stream)))


def infllmv2_score_lse_workspace_bytes(cfg, n_q, kv_cap):
    return lib().infllmv2_score_lse_workspace_bytes(C.byref(cfg), n_q, kv_cap)


def infllmv2_score_blocks_lse(cfg, q, n_q, q_pos0, is_tree, kbar, kv_cap, scores, workspace, workspace_bytes,
                              stream=None):
    _check(lib().infllmv2_score_blocks_lse(C.byref(cfg), _p(q), n_q, q_pos0, int(is_tree), _p(kbar), kv_cap,
                                           _p(scores), _p(workspace), workspace_bytes, _s(stream)))
