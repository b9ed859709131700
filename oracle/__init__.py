"""Python handle on the CPU oracle (oracle.c) for InfLLM v2 block-sparse attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The product library never imports it.

The C code is built with gcc (-O2, OpenMP, no FP contraction) into
oracle/liboracle.so. All arrays are numpy; bf16 tensors travel as their
uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

MODE_SPARSE, MODE_TREE, MODE_CAUSAL, MODE_FULL, MODE_WINDOW = 0, 1, 2, 3, 4


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                        "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def use_library(path: str) -> None:
    """Point this module at another build of oracle.c (used to plant mistakes in tests)."""
    global _lib, _LIB_PATH
    _lib = None
    _LIB_PATH = path


_LIB_PATH = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_PATH is None:
            build(force=False)
        L = C.CDLL(_LIB_PATH or _LIB)
        P = C.c_void_p
        i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
        L.orc_bf16_to_double.restype = dbl
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_bf16_from_double.restype = C.c_uint16
        L.orc_bf16_from_double.argtypes = [dbl]
        L.orc_num_threads.restype = i32
        L.orc_pool.restype = i32
        L.orc_pool.argtypes = [i32, i32, i32, i32, i32, i32, i64, i64, P, P]
        L.orc_scores.restype = i32
        L.orc_scores.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, i64, i32, P, P, P]
        L.orc_scores_lse.restype = i32
        L.orc_scores_lse.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, i64, dbl, i32, P, P, P]
        L.orc_select.restype = i32
        L.orc_select.argtypes = [i32, P, i64, P, i32, P]
        L.orc_keyset.restype = i64
        L.orc_keyset.argtypes = [i32, i32, i64, i64, P, i32, i32, C.c_uint64, i64, P]
        L.orc_attend.restype = i32
        L.orc_attend.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, P, i64, i64,
                                 P, i32, i32, i64, P, dbl, i32, P, P, P, P]
        L.orc_attend_backward.restype = i32
        L.orc_attend_backward.argtypes = [i32, i32, i32, i32, i32, i32, P, i32, P, P, P, i64, i64,
                                          P, i32, i32, i64, P, dbl, P, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def bf16_to_double(h: int) -> float:
    return float(lib().orc_bf16_to_double(int(h)))


def bf16_from_double(x: float) -> int:
    return int(lib().orc_bf16_from_double(float(x)))


# ---------------------------------------------------------------- stages
def pool(k: np.ndarray, kv_len: int, bs: int = 64, ks: int = 32, kst: int = 16) -> np.ndarray:
    """Semantic kernels: k [B,Hkv,kv_cap,D] -> kbar [B,Hkv,kv_cap/bs,kpb,D] (uint16)."""
    k = _c(k, np.uint16)
    B, Hkv, cap, D = k.shape
    kpb = (bs - ks) // kst + 1
    kbar = np.zeros((B, Hkv, cap // bs, kpb, D), dtype=np.uint16)
    rc = lib().orc_pool(B, Hkv, D, bs, ks, kst, cap, kv_len, _ptr(k), _ptr(kbar))
    if rc:
        raise ValueError("orc_pool rejected its arguments")
    return kbar


def positions(mode: str, n_q: int, q_pos0: int) -> np.ndarray:
    """Absolute position of each query row (tree: every node uses the prefix length)."""
    if mode == "tree":
        return np.full(n_q, q_pos0, dtype=np.int64)
    return q_pos0 + np.arange(n_q, dtype=np.int64)


def all_group_rows(B: int, Hkv: int, n_q: int) -> np.ndarray:
    b, g, i = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(n_q), indexing="ij")
    return np.stack([b.ravel(), g.ravel(), i.ravel()], 1).astype(np.int32)


def scores(q: np.ndarray, kbar: np.ndarray, pos: np.ndarray, rows: np.ndarray,
           n_kv_heads: int, bs: int = 64):
    """Block scores R [n_rows, nblk_cap] (fp64, -inf past the candidates) and candidate counts."""
    q = _c(q, np.uint16)
    kbar = _c(kbar, np.uint16)
    B, Hq, n_q, D = q.shape
    nblk_cap, kpb = kbar.shape[2], kbar.shape[3]
    rows = _c(rows, np.int32).reshape(-1, 3)
    pos = _c(pos, np.int64)
    R = np.empty((len(rows), nblk_cap), dtype=np.float64)
    Cn = np.empty(len(rows), dtype=np.int64)
    rc = lib().orc_scores(B, Hq, n_kv_heads, D, bs, kpb, _ptr(q), n_q, _ptr(pos), _ptr(kbar),
                          nblk_cap, len(rows), _ptr(rows), _ptr(R), _ptr(Cn))
    if rc:
        raise ValueError("orc_scores rejected its arguments")
    return R, Cn


def scores_lse(q: np.ndarray, kbar: np.ndarray, pos: np.ndarray, rows: np.ndarray,
               n_kv_heads: int, scale: float | None = None, bs: int = 64):
    """LSE-normalized block scores (orc_scores_lse): R [n_rows, nblk_cap] fp64, -inf past the
    candidates, and candidate counts. scale defaults to 1/sqrt(D)."""
    q = _c(q, np.uint16)
    kbar = _c(kbar, np.uint16)
    B, Hq, n_q, D = q.shape
    nblk_cap, kpb = kbar.shape[2], kbar.shape[3]
    rows = _c(rows, np.int32).reshape(-1, 3)
    pos = _c(pos, np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    R = np.empty((len(rows), nblk_cap), dtype=np.float64)
    Cn = np.empty(len(rows), dtype=np.int64)
    rc = lib().orc_scores_lse(B, Hq, n_kv_heads, D, bs, kpb, _ptr(q), n_q, _ptr(pos), _ptr(kbar),
                              nblk_cap, float(scale), len(rows), _ptr(rows), _ptr(R), _ptr(Cn))
    if rc:
        raise ValueError("orc_scores_lse rejected its arguments")
    return R, Cn


def select(R: np.ndarray, Cn: np.ndarray, K: int) -> np.ndarray:
    R = _c(R, np.float64)
    Cn = _c(Cn, np.int64)
    idx = np.empty((R.shape[0], K), dtype=np.int32)
    rc = lib().orc_select(R.shape[0], _ptr(R), R.shape[1], _ptr(Cn), K, _ptr(idx))
    if rc:
        raise ValueError("orc_select rejected its arguments")
    return idx


def keyset(mode: int, p: int, kv_len: int, sel, K: int, dense_threshold: int,
           mask: int = 0, bs: int = 64, window: int = 0) -> np.ndarray:
    keys = np.empty(kv_len + 64, dtype=np.int64)
    s = None if sel is None else _c(sel, np.int32)
    n = lib().orc_keyset(mode, bs, p, kv_len, _ptr(s), K, dense_threshold, int(mask), int(window),
                         _ptr(keys))
    if n < 0:
        raise ValueError("orc_keyset rejected its arguments")
    return keys[:n].copy()


def attend(mode: int, q, k, v, pos, kv_len: int, rows, n_kv_heads: int, *, idx=None, K: int = 0,
           dense_threshold: int = 0, tree_mask=None, scale: float | None = None, bs: int = 64,
           window: int = 0):
    """Attention rows (b, h, i): returns out [n, D] fp64, lse [n], attended-key counts [n]."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    B, Hq, n_q, D = q.shape
    cap = k.shape[2]
    rows = _c(rows, np.int32).reshape(-1, 3)
    pos = _c(pos, np.int64)
    if idx is not None:
        idx = _c(idx, np.int32)
        K = idx.shape[-1]
    if tree_mask is not None:
        tree_mask = _c(tree_mask, np.uint64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((len(rows), D), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    nk = np.empty(len(rows), dtype=np.int64)
    rc = lib().orc_attend(mode, B, Hq, n_kv_heads, D, bs, _ptr(q), n_q, _ptr(pos), _ptr(k), _ptr(v),
                          cap, kv_len, _ptr(idx), K, dense_threshold, int(window), _ptr(tree_mask),
                          float(scale),
                          len(rows), _ptr(rows), _ptr(out), _ptr(lse), _ptr(nk))
    if rc:
        raise ValueError("orc_attend rejected its arguments")
    return out, lse, nk


def attend_backward(mode: int, q, k, v, pos, kv_len: int, n_kv_heads: int, dout, *, idx=None,
                    K: int = 0, dense_threshold: int = 0, tree_mask=None, scale: float | None = None,
                    bs: int = 64, window: int = 0):
    """Gradients of sum(dout * o) over every row (b, h, i) of `q`, with the key sets of
    `attend`: returns dq [B][Hq][n_q][D], dk and dv [B][Hkv][kv_cap][D], all fp64."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    dout = _c(dout, np.uint16)
    B, Hq, n_q, D = q.shape
    cap = k.shape[2]
    pos = _c(pos, np.int64)
    if idx is not None:
        idx = _c(idx, np.int32)
        K = idx.shape[-1]
    if tree_mask is not None:
        tree_mask = _c(tree_mask, np.uint64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = np.empty((B, Hq, n_q, D), dtype=np.float64)
    dk = np.empty((B, n_kv_heads, cap, D), dtype=np.float64)
    dv = np.empty((B, n_kv_heads, cap, D), dtype=np.float64)
    rc = lib().orc_attend_backward(mode, B, Hq, n_kv_heads, D, bs, _ptr(q), n_q, _ptr(pos), _ptr(k),
                                   _ptr(v), cap, kv_len, _ptr(idx), K, dense_threshold, int(window),
                                   _ptr(tree_mask), float(scale), _ptr(dout), _ptr(dq), _ptr(dk),
                                   _ptr(dv))
    if rc:
        raise ValueError("orc_attend_backward rejected its arguments")
    return dq, dk, dv


# ------------------------------------------------------------ whole path
def sparse_forward(q, k, v, *, kv_len: int, q_pos0: int, n_kv_heads: int, top_k: int,
                   dense_threshold: int, tree_mask=None, group_rows=None, kbar=None,
                   bs: int = 64, ks: int = 32, kst: int = 16, scale=None, with_attention=True):
    """The InfLLM v2 path for the given query rows: kernels -> scores -> top-K -> attention.

    group_rows: (b, g, i) rows to compute (default: all). Attention is computed
    for every head of those groups. Returns a dict with kbar, R, C, idx (full
    array, -2 in rows not computed), out/lse/nkeys for the attention rows, and
    the rows themselves.
    """
    q = _c(q, np.uint16)
    B, Hq, n_q, D = q.shape
    G = Hq // n_kv_heads
    mode = "tree" if tree_mask is not None else "sparse"
    pos = positions(mode, n_q, q_pos0)
    if kbar is None:
        kbar = pool(k, kv_len, bs, ks, kst)
    if group_rows is None:
        group_rows = all_group_rows(B, n_kv_heads, n_q)
    group_rows = _c(group_rows, np.int32).reshape(-1, 3)
    R, Cn = scores(q, kbar, pos, group_rows, n_kv_heads, bs)
    sel = select(R, Cn, top_k)
    idx = np.full((B, n_kv_heads, n_q, top_k), -2, dtype=np.int32)
    idx[group_rows[:, 0], group_rows[:, 1], group_rows[:, 2]] = sel
    res = dict(kbar=kbar, R=R, C=Cn, idx=idx, sel=sel, group_rows=group_rows, pos=pos)
    if with_attention:
        hrows = np.array([(b, g * G + hh, i) for (b, g, i) in group_rows for hh in range(G)],
                         dtype=np.int32).reshape(-1, 3)
        out, lse, nk = attend(MODE_TREE if tree_mask is not None else MODE_SPARSE, q, k, v, pos,
                              kv_len, hrows, n_kv_heads, idx=idx, dense_threshold=dense_threshold,
                              tree_mask=tree_mask, scale=scale, bs=bs)
        res.update(out=out, lse=lse, nkeys=nk, head_rows=hrows)
    return res


def dense_forward(q, k, v, *, kv_len: int, n_kv_heads: int, causal: bool = True, rows=None,
                  scale=None, bs: int = 64):
    """Dense attention, bottom-right aligned: query i sits at position kv_len - n_q + i."""
    q = _c(q, np.uint16)
    B, Hq, n_q, D = q.shape
    pos = positions("prefill", n_q, kv_len - n_q)
    if rows is None:
        b, h, i = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(n_q), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int32)
    out, lse, nk = attend(MODE_CAUSAL if causal else MODE_FULL, q, k, v, pos, kv_len, rows,
                          n_kv_heads, scale=scale, bs=bs)
    return dict(out=out, lse=lse, nkeys=nk, rows=rows, pos=pos)


def window_forward(q, k, v, *, kv_len: int, n_kv_heads: int, window: int, rows=None, scale=None,
                   bs: int = 64):
    """Sliding-window causal attention (the draft model's): query i sits at position
    kv_len - n_q + i and attends keys max(0, p - window + 1) .. p."""
    q = _c(q, np.uint16)
    B, Hq, n_q, D = q.shape
    pos = positions("prefill", n_q, kv_len - n_q)
    if rows is None:
        b, h, i = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(n_q), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int32)
    out, lse, nk = attend(MODE_WINDOW, q, k, v, pos, kv_len, rows, n_kv_heads, scale=scale, bs=bs,
                          window=window)
    return dict(out=out, lse=lse, nkeys=nk, rows=rows, pos=pos)
