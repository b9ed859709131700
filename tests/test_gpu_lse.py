"""GPU parity of the LSE-normalized block scores and the selection made from them.

Scores: every finite entry within 1e-4 relative (fp32 exp2 and dot products
against the fp64 oracle; the values lie in (0, G]) and the -inf pattern (the
candidate sets) identical. Selection: bit-exact block indices, with query
tokens redrawn by the oracle until the K-th and (K+1)-th LSE scores differ by
more than 1e-3 relative (tests/gaps.py). A decode step that selects from these
scores matches the oracle's attention over the same blocks.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from trainable_block_sparse_infllm_amd import ops
from oracle.gaps import open_gaps
from gpu_util import LSE_ABS, assert_close_rows, cfg_of, dev_bf16, dev_i32, host_f64, note

pytestmark = pytest.mark.gpu

D0 = synth.WORKLOADS["decode_32k"]
T0 = synth.WORKLOADS["tree_128k"]


def _compare_scores(gs, R, Cn):
    fin = np.isfinite(R)
    assert np.array_equal(np.isfinite(gs), fin), "candidate sets differ"
    err = np.abs(gs[fin] - R[fin]) / np.abs(R[fin])
    note(f"  lse scores: max rel err {err.max():.2e} over {fin.sum()} entries")
    assert err.max() <= 1e-4


CASES = {
    # (B, Hq, Hkv, D, kv_len, n_q, K)
    "decode_g4": (2, 8, 2, 128, 9000, 1, 8),
    "decode_g1": (1, 4, 4, 128, 5000, 1, 16),
    "decode_g16_d64": (1, 16, 1, 64, 3000, 1, 4),
    "rows_g8": (1, 16, 2, 128, 4200, 20, 8),
    "rows_g2_d64": (2, 4, 2, 64, 2100, 33, 3),
}


@pytest.mark.parametrize("case", list(CASES))
def test_lse_scores_and_selection_match_oracle(case):
    B, Hq, Hkv, D, kv_len, n_q, K = CASES[case]
    w = D0.scaled(name=f"lse_{case}", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, seq_len=kv_len,
                  top_k=K, dense_threshold=0, n_plant=4)
    note(f"lse case {case}: B{B} Hq{Hq}/Hkv{Hkv} D{D} kv_len{kv_len} n_q{n_q} K{K}")
    d = synth.generate(w, seed=3)
    q = np.ascontiguousarray(np.repeat(d["q"], n_q, axis=2)) if n_q > 1 else d["q"]
    P = kv_len - n_q
    pos = P + np.arange(n_q)
    dd = dict(d, q=q, n_q=n_q, q_pos0=P)
    kbar_o, _, _ = open_gaps(dd, orc, pos=pos, score_fn=orc.scores_lse, relative=True)
    q = dd["q"]
    rows = orc.all_group_rows(B, Hkv, n_q)
    R, Cn = orc.scores_lse(q, kbar_o, pos, rows, Hkv)
    cfg = cfg_of(w)
    kbar = ops.pool_kernels(cfg, dev_bf16(d["k"]), d["kv_cap"], kv_len)
    scores = ops.score_blocks_lse(cfg, dev_bf16(q), kbar, P, d["kv_cap"])
    idx = torch.empty((B, Hkv, n_q, K), dtype=torch.int32, device="cuda")
    from trainable_block_sparse_infllm_amd import capi
    capi.infllmv2_topk_blocks(cfg, scores, None, None, n_q, P, 0, d["kv_cap"], idx)
    torch.cuda.synchronize()
    gs = scores.cpu().numpy().reshape(len(rows), -1)[:, :R.shape[1]]
    _compare_scores(gs, R, Cn)
    assert np.array_equal(idx.cpu().numpy().reshape(len(rows), K), orc.select(R, Cn, K)), \
        "block indices differ"


def test_lse_tree_rows_share_the_prefix_candidates():
    B, Hq, Hkv, n_tree = 1, 8, 2, 7
    w = T0.scaled(name="lse_tree", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, seq_len=3000, top_k=6, n_plant=3,
                  n_tree=n_tree, tree_depth=3, dense_threshold=0)
    d = synth.generate(w, seed=4)
    P = d["kv_len"] - d["n_q"]
    pos = np.full(d["n_q"], P, dtype=np.int64)
    kbar_o, _, _ = open_gaps(d, orc, pos=pos, score_fn=orc.scores_lse, relative=True)
    rows = orc.all_group_rows(B, Hkv, d["n_q"])
    R, Cn = orc.scores_lse(d["q"], kbar_o, pos, rows, Hkv)
    cfg = cfg_of(w)
    kbar = ops.pool_kernels(cfg, dev_bf16(d["k"]), d["kv_cap"], d["kv_len"])
    scores = ops.score_blocks_lse(cfg, dev_bf16(d["q"]), kbar, P, d["kv_cap"], is_tree=True)
    torch.cuda.synchronize()
    gs = scores.cpu().numpy().reshape(len(rows), -1)[:, :R.shape[1]]
    _compare_scores(gs, R, Cn)


def test_lse_decode_step_end_to_end():
    w = D0.scaled(name="lse_step", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=7000, top_k=8, n_plant=4,
                  dense_threshold=1024)
    d = synth.generate(w, seed=5)
    L = d["kv_len"]
    pos = np.array([L - 1])
    kbar_o, _, _ = open_gaps(d, orc, pos=pos, score_fn=orc.scores_lse, relative=True)
    rows = orc.all_group_rows(w.batch, w.n_kv_heads, 1)
    R, Cn = orc.scores_lse(d["q"], kbar_o, pos, rows, w.n_kv_heads)
    sel = orc.select(R, Cn, w.top_k)
    idx_o = sel.reshape(w.batch, w.n_kv_heads, 1, w.top_k)
    G = w.group
    hrows = np.array([(b, g * G + hh, 0) for (b, g, _) in rows for hh in range(G)], np.int32)
    out_o, lse_o, _ = orc.attend(orc.MODE_SPARSE, d["q"], d["k"], d["v"], pos, L, hrows, w.n_kv_heads,
                                 idx=idx_o, dense_threshold=w.dense_threshold)
    cfg = cfg_of(w)
    k, v = dev_bf16(d["k"]), dev_bf16(d["v"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], L)
    res = ops.decode_step_lse(cfg, dev_bf16(d["q"]), k, v, kbar, L)
    torch.cuda.synchronize()
    assert np.array_equal(res["idx"].cpu().numpy(), idx_o)
    go = host_f64(res["out"])[hrows[:, 0], hrows[:, 1], hrows[:, 2]]
    assert_close_rows(go, out_o, "lse decode out")
    gl = host_f64(res["lse"])[hrows[:, 0], hrows[:, 1], hrows[:, 2]]
    assert np.abs(gl - lse_o).max() <= LSE_ABS


def test_lse_decode_128k_batch8_full_size():
    """The benchmark's LSE-selection leg (128K, batch 8, K = 32) in its launch configuration:
    selection exact and outputs within tolerance for every (sequence, head)."""
    w = synth.WORKLOADS["decode_128k_b8"]
    d = synth.generate(w, seed=6, threads=16)
    L = d["kv_len"]
    pos = np.array([L - 1])
    kbar_o, _, _ = open_gaps(d, orc, pos=pos, score_fn=orc.scores_lse, relative=True)
    rows = orc.all_group_rows(w.batch, w.n_kv_heads, 1)
    R, Cn = orc.scores_lse(d["q"], kbar_o, pos, rows, w.n_kv_heads)
    idx_o = orc.select(R, Cn, w.top_k).reshape(w.batch, w.n_kv_heads, 1, w.top_k)
    G = w.group
    hrows = np.array([(b, g * G + hh, 0) for (b, g, _) in rows for hh in range(G)], np.int32)
    note(f"lse 128K full size: {len(hrows)} rows")
    out_o, lse_o, _ = orc.attend(orc.MODE_SPARSE, d["q"], d["k"], d["v"], pos, L, hrows, w.n_kv_heads,
                                 idx=idx_o, dense_threshold=w.dense_threshold)
    cfg = cfg_of(w)
    k, v = dev_bf16(d["k"]), dev_bf16(d["v"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], L)
    res = ops.decode_step_lse(cfg, dev_bf16(d["q"]), k, v, kbar, L)
    torch.cuda.synchronize()
    assert np.array_equal(res["idx"].cpu().numpy(), idx_o)
    go = host_f64(res["out"])[hrows[:, 0], hrows[:, 1], hrows[:, 2]]
    assert_close_rows(go, out_o, "lse decode 128K out")
    gl = host_f64(res["lse"])[hrows[:, 0], hrows[:, 1], hrows[:, 2]]
    assert np.abs(gl - lse_o).max() <= LSE_ABS
