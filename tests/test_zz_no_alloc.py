"""The allocation-free single-token decode entry point (scratch in a static device array)
against the workspace entry point it mirrors, through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to the workspace call on the same inputs
(the same kernels run over the same partials), and the selection against the oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
import trainable_block_sparse_infllm_amd as lib
from trainable_block_sparse_infllm_amd import ops
from oracle.gaps import open_gaps
from gpu_util import assert_close_rows, cfg_of, dev_bf16, host_f64, note

pytestmark = pytest.mark.gpu

CASES = [
    synth.WORKLOADS["decode_32k"].scaled(name="noalloc_big", batch=4, seq_len=65536, top_k=32, n_plant=32),
    synth.WORKLOADS["decode_32k"].scaled(name="noalloc_small", n_q_heads=8, n_kv_heads=2, head_dim=64,
                                         seq_len=5000, top_k=16, n_plant=8),
]


def _run(w, seed):
    note(f"no-alloc decode: {w.name} B{w.batch} Hq{w.n_q_heads}/Hkv{w.n_kv_heads} D{w.head_dim} "
         f"kv_len{w.kv_len} K{w.top_k}")
    d = synth.generate(w, seed=seed)
    kbar_o, _, _ = open_gaps(d, orc)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], q_pos0=d["kv_len"] - 1,
                             n_kv_heads=w.n_kv_heads, top_k=w.top_k, dense_threshold=w.dense_threshold,
                             kbar=kbar_o)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    cap, L = d["kv_cap"], d["kv_len"]
    kbar = ops.pool_kernels(cfg, k, cap, L)
    scores = torch.empty((w.batch, w.n_kv_heads, 1, ops.nblk(cap)), dtype=torch.float32, device="cuda")
    lib.infllmv2_score_blocks(cfg, q, 1, L - 1, 0, kbar, cap, scores)
    shape = (w.batch, w.n_q_heads, 1, w.head_dim)
    res = {}
    for which in ("workspace", "noalloc"):
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
        idx = torch.full((w.batch, w.n_kv_heads, 1, w.top_k), -7, dtype=torch.int32, device="cuda")
        if which == "workspace":
            nb = lib.infllmv2_decode_workspace_bytes(cfg, 1, L)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            lib.infllmv2_sparse_attn_decode_scores(cfg, q, k, v, cap, L, scores, idx, out, lse, ws, nb)
        else:
            lib.infllmv2_sparse_attn_decode_scores_noalloc(cfg, q, k, v, cap, L, scores, idx, out, lse)
        torch.cuda.synchronize()
        res[which] = (idx, out, lse)
    (i0, o0, l0), (i1, o1, l1) = res["workspace"], res["noalloc"]
    assert torch.equal(i1, i0), "selected blocks differ from the workspace entry point"
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), "outputs differ from the workspace entry point"
    assert torch.equal(l1, l0), "lse differs from the workspace entry point"
    assert np.array_equal(i1.cpu().numpy(), ref["idx"]), "selection differs from the oracle"
    hr = ref["head_rows"]
    assert_close_rows(host_f64(o1)[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], f"{w.name} no-alloc out")


def test_noalloc_decode_two_calls_second_smaller():
    _run(CASES[0], seed=31)
    _run(CASES[1], seed=32)
