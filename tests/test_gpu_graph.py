"""A decode step captured in a HIP graph gives the eager result on every replay.

The graph holds the three decode launches (scores, top-K, split attention and
combine); replays are interleaved with unrelated eager work and
synchronisations, and each replay's output is compared with the eager one.
"""
import numpy as np
import pytest
import torch

import synth
import trainable_block_sparse_infllm_amd as lib
from trainable_block_sparse_infllm_amd import ops
from gpu_util import cfg_of, dev_bf16, dev_u64, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tree", [False, True])
def test_decode_graph_replays_match_eager(tree):
    w = synth.WORKLOADS["tree_128k" if tree else "decode_32k"].scaled(
        name="graph", n_q_heads=8, n_kv_heads=2, seq_len=8192)
    note(f"graph case tree={tree}")
    d = synth.generate(w, seed=1)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    mask = dev_u64(d["tree_mask"]) if tree else None
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], d["kv_len"])
    ws = ops.Workspace(q.device)
    eager = ops.decode(cfg, q, k, v, kbar, d["kv_len"], tree_mask=mask, ws=ws)
    torch.cuda.synchronize()
    ref_out, ref_idx = eager["out"].clone(), eager["idx"].clone()

    holder = {}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        holder["res"] = ops.decode(cfg, q, k, v, kbar, d["kv_len"], tree_mask=mask, ws=ws)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        holder["res"]["out"].zero_()
        holder["res"]["idx"].fill_(-7)
        junk.mul_(1.0001).add_(0.5)              # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(holder["res"]["idx"], ref_idx), f"replay {rep}: indices differ"
        assert torch.equal(holder["res"]["out"], ref_out), f"replay {rep}: outputs differ"
