"""Degenerate shapes through every entry point: one token, one key, one block.

A one-token prefill attends only itself (out = its own value row, lse = scale q.k);
a decode step over a one-key cache likewise; tokens inside the first block have
no candidates (every selection slot -1). Bars as for the other attention outputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import synth
import trainable_block_sparse_infllm_amd as lib
from trainable_block_sparse_infllm_amd import ops
from gpu_util import LSE_ABS, assert_close_rows, cfg_of, dev_bf16, host_f64, note

pytestmark = pytest.mark.gpu

P0 = synth.WORKLOADS["prefill_32k"]
D0 = synth.WORKLOADS["decode_32k"]


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_within_the_first_blocks(T, D):
    w = P0.scaled(name="tiny_T", n_q_heads=8, n_kv_heads=2, head_dim=D, seq_len=T, top_k=4, dense_threshold=0,
                  n_plant=0)
    note(f"prefill T{T} D{D}")
    d = synth.generate(w, seed=2)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=T, q_pos0=0, n_kv_heads=2, top_k=4,
                             dense_threshold=0)
    res = ops.sparse_prefill(cfg_of(w), dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]))
    torch.cuda.synchronize()
    gidx = res["idx"].cpu().numpy()
    assert np.array_equal(gidx, ref["idx"])
    if T <= 128:
        assert (gidx[:, :, :64] == -1).all()               # the first block's tokens have no candidates
    hr = ref["head_rows"]
    assert_close_rows(host_f64(res["out"])[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], f"T{T} out")
    assert np.abs(host_f64(res["lse"])[hr[:, 0], hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS
    if T == 1:                                             # softmax over one key: the value row itself
        v0 = synth.bf16_to_f32(d["v"][0, :, 0]).astype(np.float64)
        got = host_f64(res["out"])[0, :, 0]
        assert np.allclose(got, np.repeat(v0, 4, axis=0), rtol=0, atol=2e-2 * np.abs(v0).max() + 1e-6)


@pytest.mark.parametrize("kv_len", [1, 64, 65])
def test_decode_over_the_first_block(kv_len):
    w = D0.scaled(name="tiny_dec", n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=kv_len, top_k=4,
                  dense_threshold=0, n_plant=0)
    d = synth.generate(w, seed=3)
    cfg = cfg_of(w)
    k, v = dev_bf16(d["k"]), dev_bf16(d["v"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], kv_len)
    res = ops.decode_step(cfg, dev_bf16(d["q"]), k, v, kbar, kv_len)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=kv_len, q_pos0=kv_len - 1, n_kv_heads=2, top_k=4,
                             dense_threshold=0)
    torch.cuda.synchronize()
    assert np.array_equal(res["idx"].cpu().numpy(), ref["idx"])
    hr = ref["head_rows"]
    assert_close_rows(host_f64(res["out"])[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], f"kv_len{kv_len} out")
    assert np.abs(host_f64(res["lse"])[hr[:, 0], hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS


def test_window_and_backward_on_one_token():
    w = P0.scaled(name="one_tok", n_q_heads=4, n_kv_heads=1, head_dim=128, seq_len=1, top_k=2, dense_threshold=0,
                  n_plant=0)
    d = synth.generate(w, seed=4)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    win = ops.sliding_window(cfg, q, k, v, 1, 16)
    fw = ops.sparse_prefill(cfg, q, k, v)
    dout = torch.ones_like(q)
    g = ops.sparse_prefill_backward(cfg, q, k, v, fw["idx"], fw["out"], fw["lse"], dout)
    torch.cuda.synchronize()
    assert torch.equal(win["out"], fw["out"])
    # one key: P = 1, dS = P (dP - dO.O) = 0 up to the bf16 output, so dq ~ 0 and dk ~ 0; dv = dO
    assert float(g["dq"].abs().max()) <= 1e-2 and float(g["dk"][:, :, :1].abs().max()) <= 1e-2
    assert torch.allclose(g["dv"][:, :, 0], torch.full_like(g["dv"][:, :, 0], 4.0))   # 4 heads share the key
