"""Helpers for GPU parity tests: move seeded inputs to the device, compare with the oracle."""
import sys

import numpy as np
import torch

import trainable_block_sparse_infllm_amd as lib

MAX_ABS, MEAN_ABS = 2e-2, 2e-3      # output tolerance (bf16 output vs fp64 oracle)
LSE_ABS = 2e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_u64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64).view(np.int64)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def kbar_rows(t: torch.Tensor) -> np.ndarray:
    """Device kernel table [B][Hkv][ntile][3][D/8][32][8] -> the oracle's [B][Hkv][nblk][3][D]
    (bf16 bits; nblk rounded up to whole tiles of 32 blocks)."""
    a = host_u16(t)
    B, Hkv, nt, kpb, P, tb, e = a.shape
    return np.ascontiguousarray(a.transpose(0, 1, 2, 5, 3, 4, 6).reshape(B, Hkv, nt * tb, kpb, P * e))


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def cfg_of(w, **over):
    kw = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
              top_k=w.top_k, dense_threshold=w.dense_threshold)
    kw.update(over)
    return lib.make_cfg(**kw)


def assert_close_rows(gpu_rows: np.ndarray, ref_rows: np.ndarray, what: str):
    err = np.abs(gpu_rows - ref_rows)
    mx, mean = float(err.max()), float(err.mean())
    note(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {gpu_rows.shape[0]} rows")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx} mean-abs {mean}"


def check_idx_rows(idx: np.ndarray, C: np.ndarray, K: int):
    """Properties every selection row must have: ascending, in range, right count, -1 tail."""
    for r in range(idx.shape[0]):
        c = int(C[r])
        n = min(c, K)
        row = idx[r]
        assert (row[n:] == -1).all(), (r, row)
        sel = row[:n]
        assert (sel >= 0).all() and (sel < c).all(), (r, row, c)
        assert (np.diff(sel) > 0).all(), (r, row)
