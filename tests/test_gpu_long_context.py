"""GPU parity past the per-tile union kernel's range: head_dim 128 calls whose
context exceeds 8192 blocks (kv_len > 524288) run the rows kernel, for sparse
(mode 0), dense causal and sliding-window attention, all through the C ABI.
Also the fused score + top-K for one and two query heads per group with more
candidates than 1024 and 2048 (score rows of 8 and 16 KB per token in LDS)."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
import trainable_block_sparse_infllm_amd as lib
from oracle.gaps import open_gaps
from gpu_util import LSE_ABS, assert_close_rows, cfg_of, dev_bf16, dev_i32, host_f64, note

pytestmark = pytest.mark.gpu

LONG = 530_000          # 8282 blocks: more than the union kernel's 8192
N_Q = 48                # a chunk of query rows at the end of the context (ragged against 16/32-token tiles)


@pytest.fixture(scope="module")
def long_chunk():
    """One KV head with 4 query heads, head_dim 128, a 530000-token cache and the
    last 48 positions as queries (fresh seeded rows along the group's shared direction)."""
    w = synth.WORKLOADS["decode_32k"].scaled(name="long_chunk", n_q_heads=4, n_kv_heads=1, seq_len=LONG,
                                             top_k=16, n_plant=16, dense_threshold=1024)
    note(f"long-context chunk: B1 Hq4/Hkv1 D128 kv_len {LONG} n_q {N_Q}")
    d = synth.generate(w, seed=5)
    q = np.empty((1, 4, N_Q, 128), dtype=np.uint16)
    for i in range(N_Q):
        q[0, :, i] = synth.redraw_q_token(w, 5, 0, 0, LONG - N_Q + i, 10_000)
    d.update(q=q, n_q=N_Q, q_pos0=LONG - N_Q)
    kbar_o, redrawn, _ = open_gaps(d, orc)
    note(f"  gaps opened ({redrawn} token redraws)")
    dev = dict(q=dev_bf16(d["q"]), k=dev_bf16(d["k"]), v=dev_bf16(d["v"]))
    return w, d, kbar_o, dev


def test_long_context_sparse_rows_kernel(long_chunk):
    w, d, kbar_o, dev = long_chunk
    L = d["kv_len"]
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=L, q_pos0=L - N_Q, n_kv_heads=1, top_k=w.top_k,
                             dense_threshold=w.dense_threshold, kbar=kbar_o)
    out = torch.empty((1, 4, N_Q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 4, N_Q), dtype=torch.float32, device="cuda")
    lib.infllmv2_sparse_attn_prefill(cfg_of(w), dev["q"], N_Q, dev["k"], dev["v"], d["kv_cap"], L,
                                     dev_i32(ref["idx"]), out, lse)
    torch.cuda.synchronize()
    hr = ref["head_rows"]
    assert_close_rows(host_f64(out)[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], "sparse, 8282 blocks")
    assert np.abs(host_f64(lse)[hr[:, 0], hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS


def test_long_context_dense_causal_rows_kernel(long_chunk):
    w, d, _, dev = long_chunk
    L = d["kv_len"]
    ref = orc.dense_forward(d["q"], d["k"], d["v"], kv_len=L, n_kv_heads=1, causal=True)
    out = torch.empty((1, 4, N_Q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 4, N_Q), dtype=torch.float32, device="cuda")
    lib.infllmv2_dense_attn(cfg_of(w), dev["q"], N_Q, dev["k"], dev["v"], d["kv_cap"], L, 1, out, lse)
    torch.cuda.synchronize()
    r = ref["rows"]
    assert_close_rows(host_f64(out)[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "dense causal, 8282 blocks")
    assert np.abs(host_f64(lse)[r[:, 0], r[:, 1], r[:, 2]] - ref["lse"]).max() <= LSE_ABS


@pytest.mark.parametrize("window", [2048, 100])
def test_long_context_window_rows_kernel(long_chunk, window):
    w, d, _, dev = long_chunk
    L = d["kv_len"]
    ref = orc.window_forward(d["q"], d["k"], d["v"], kv_len=L, n_kv_heads=1, window=window)
    out = torch.empty((1, 4, N_Q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 4, N_Q), dtype=torch.float32, device="cuda")
    lib.infllmv2_sliding_window_attn(cfg_of(w), dev["q"], N_Q, dev["k"], dev["v"], d["kv_cap"], L, window,
                                     out, lse)
    torch.cuda.synchronize()
    r = ref["rows"]
    assert_close_rows(host_f64(out)[r[:, 0], r[:, 1], r[:, 2]], ref["out"], f"window {window}, 8282 blocks")
    assert np.abs(host_f64(lse)[r[:, 0], r[:, 1], r[:, 2]] - ref["lse"]).max() <= LSE_ABS


@pytest.mark.parametrize("L,n_q,hq,hkv,K", [(70_000, 40, 2, 2, 16),     # G1, 1093 candidates
                                            (140_000, 24, 2, 2, 8),     # G1, 2187: 9 tokens per workgroup
                                            (140_000, 24, 4, 2, 16),    # G2, 2187 candidates
                                            (262_000, 12, 2, 1, 16)])   # G2, 4093 candidates
def test_fused_topk_many_candidates_small_groups(L, n_q, hq, hkv, K):
    """Fused scoring + selection when a token's score row is 8 or 16 KB, for one and two
    query heads per group (the workgroup holds fewer tokens' rows in LDS)."""
    w = synth.WORKLOADS["prefill_32k"].scaled(name="fused_small_g", n_q_heads=hq, n_kv_heads=hkv, seq_len=L,
                                              top_k=K, n_plant=4, dense_threshold=0)
    note(f"fused top-K, small groups: L{L} n_q{n_q} Hq{hq}/Hkv{hkv} K{K}")
    d = synth.generate(w, seed=21)
    P = L - n_q
    qn = np.ascontiguousarray(d["q"][:, :, P:])
    kbar_o = orc.pool(d["k"], L)
    dd = dict(d, q=qn, n_q=n_q, q_pos0=P)
    pos = P + np.arange(n_q, dtype=np.int64)
    open_gaps(dd, orc, kbar=kbar_o, pos=pos)
    qn = dd["q"]
    R, Cn = orc.scores(qn, kbar_o, pos, orc.all_group_rows(w.batch, hkv, n_q), hkv)
    ref = orc.select(R, Cn, K)
    cfg = cfg_of(w)
    k = dev_bf16(d["k"])
    from trainable_block_sparse_infllm_amd import ops
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], L)
    idx = torch.empty((w.batch, hkv, n_q, K), dtype=torch.int32, device="cuda")
    lib.infllmv2_topk_blocks(cfg, None, dev_bf16(qn), kbar, n_q, P, 0, d["kv_cap"], idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().reshape(-1, K), ref)
