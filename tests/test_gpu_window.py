"""GPU parity of the sliding-window attention (the draft model's) against the oracle.

Row i sits at position p = kv_len - n_q + i and attends keys max(0, p - W + 1)
.. p. Cases cover windows inside one block, windows not a multiple of the
block size, a window of one key, windows wider than the prefix (dense
causal), chunked calls (n_q < kv_len), single-token decode steps, every
GQA group size, and head_dim 64 (served by the rows kernel). Tolerances as for the other attention outputs: bf16 out
max-abs <= 2e-2, mean-abs <= 2e-3; lse within LSE_ABS.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from trainable_block_sparse_infllm_amd import ops
from gpu_util import LSE_ABS, assert_close_rows, cfg_of, dev_bf16, host_f64, note

pytestmark = pytest.mark.gpu

P0 = synth.WORKLOADS["prefill_32k"]

# (Hq, Hkv, B, n_q, kv_len, window[, head_dim])
CASES = [
    (8, 2, 1, 1100, 1100, 300),      # prefill, window spans ~5 blocks, not a multiple of 64
    (8, 2, 2, 700, 700, 64),         # exactly one block wide
    (8, 2, 1, 500, 500, 65),         # one key past a block
    (4, 1, 1, 400, 400, 1),          # only the own key
    (8, 2, 1, 333, 333, 5000),       # wider than the prefix: dense causal
    (8, 2, 1, 97, 1500, 200),        # chunk of a longer prompt
    (8, 2, 2, 1, 5000, 1024),        # draft decode step
    (8, 2, 1, 3, 4097, 777),         # a few tokens at a block edge
    (2, 2, 1, 600, 600, 130),        # G = 1
    (16, 1, 1, 300, 300, 90),        # G = 16
    (16, 2, 1, 260, 900, 33),        # G = 8, chunk
    # head_dim 64 (the rows kernel's window mode)
    (2, 1, 1, 1100, 1100, 300, 64),  # G = 2, prefill
    (8, 2, 2, 97, 1500, 200, 64),    # chunk of a longer prompt
    (8, 2, 1, 1, 5000, 1024, 64),    # draft decode step
    (4, 1, 1, 400, 400, 1, 64),      # only the own key
    (8, 2, 1, 333, 333, 5000, 64),   # wider than the prefix: dense causal
]


@pytest.mark.parametrize("dims", CASES, ids=lambda c: "x".join(map(str, c)))
def test_sliding_window_matches_oracle(dims):
    Hq, Hkv, B, n_q, kv_len, W = dims[:6]
    D = dims[6] if len(dims) > 6 else 128
    w = P0.scaled(name="window", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, seq_len=kv_len,
                  n_plant=0, dense_threshold=0)
    note(f"window case B{B} Hq{Hq}/Hkv{Hkv} n_q{n_q} kv_len{kv_len} W{W} D{D}")
    d = synth.generate(w, seed=11)
    qn = np.ascontiguousarray(d["q"][:, :, kv_len - n_q:])
    ref = orc.window_forward(qn, d["k"], d["v"], kv_len=kv_len, n_kv_heads=Hkv, window=W)
    res = ops.sliding_window(cfg_of(w), dev_bf16(qn), dev_bf16(d["k"]), dev_bf16(d["v"]), kv_len, W)
    torch.cuda.synchronize()
    r = ref["rows"]
    assert set(ref["nkeys"].tolist()) <= set(range(1, W + 1))
    assert_close_rows(host_f64(res["out"])[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "window out")
    assert np.abs(host_f64(res["lse"])[r[:, 0], r[:, 1], r[:, 2]] - ref["lse"]).max() <= LSE_ABS


def test_sliding_window_wider_than_prefix_equals_dense_causal():
    w = P0.scaled(name="window_dense", n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=800, n_plant=0,
                  dense_threshold=0)
    d = synth.generate(w, seed=12)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    a = ops.sliding_window(cfg, q, k, v, 800, 800)
    b = ops.dense(cfg, q, k, v, 800, causal=True)
    torch.cuda.synchronize()
    # the same kernel walks the same blocks in the same order: identical bits
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])


def test_sliding_window_32k_full_size_sampled_rows():
    """The benchmark's window leg (the 32K prompt's shapes, W = 2048) in its launch
    configuration; the oracle computes sampled rows of every head: the first rows (window
    wider than the prefix), rows at block edges, the window's first full row and the last."""
    w = P0
    W = 2048
    T = w.seq_len
    d = synth.generate(w, seed=0, threads=16)
    res = ops.sliding_window(cfg_of(w), dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), T, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    toks = sorted(set([0, 1, 63, 64, W - 2, W - 1, W, W + 1, 4095, 4096, T - 1] + rng.integers(0, T, 12).tolist()))
    rows = np.array([(0, h, t) for h in range(w.n_q_heads) for t in toks], dtype=np.int32)
    note(f"window 32K full size: {len(rows)} sampled rows")
    ref = orc.window_forward(d["q"], d["k"], d["v"], kv_len=T, n_kv_heads=w.n_kv_heads, window=W, rows=rows)
    r = ref["rows"]
    assert set(ref["nkeys"].tolist()) <= set(range(1, W + 1))
    assert_close_rows(host_f64(res["out"])[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "window 32K out")
    assert np.abs(host_f64(res["lse"])[r[:, 0], r[:, 1], r[:, 2]] - ref["lse"]).max() <= LSE_ABS
