"""GPU parity of the sparse prefill backward (dq, dk, dv) against the oracle.

The key sets come from the GPU forward's own selection (idx), so the check is
the backward alone; the forward's out and lse feed it as in training.
Tolerance (fp32 outputs from bf16 operands): P and dS enter the MFMA products
rounded to bf16 (relative 2^-9 per term) and Delta = dO . O uses the bf16
forward output. dq sums dS_t k_t over a row's keys with sum_t dS_t = 0, so the
rounding noise is large next to the result: replaying exactly these two
roundings in fp64 gives a mean error of about 3-4e-3 of mean|dq| and a max of
about 7e-3 of max|dq| (tests/test_oracle_backward.py checks that replay
against the bounds used here): max-abs <= 2e-2 * max|ref|, mean-abs <= 1e-2 *
mean|ref|. dk and dv sum over queries, where no such cancellation occurs, and
keep mean-abs <= 2e-3 * mean|ref|.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
import trainable_block_sparse_infllm_amd as lib
from trainable_block_sparse_infllm_amd import ops
from gpu_util import cfg_of, dev_bf16, note

pytestmark = pytest.mark.gpu

W0 = synth.WORKLOADS["tiny_prefill_2k"]

CASES = {
    "g4_mixed": W0.scaled(name="bwd_g4", n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=1100, top_k=4,
                          dense_threshold=300, n_plant=2),
    "g1": W0.scaled(name="bwd_g1", n_q_heads=2, n_kv_heads=2, head_dim=128, seq_len=700, top_k=3,
                    dense_threshold=0, n_plant=2),
    "g2_b2": W0.scaled(name="bwd_g2", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, seq_len=900, top_k=5,
                       dense_threshold=200, n_plant=2),
    "g8": W0.scaled(name="bwd_g8", n_q_heads=16, n_kv_heads=2, head_dim=128, seq_len=640, top_k=2,
                    dense_threshold=0, n_plant=1),
    "g16_dense": W0.scaled(name="bwd_g16", n_q_heads=16, n_kv_heads=1, head_dim=128, seq_len=500, top_k=2,
                           dense_threshold=600, n_plant=1),
    # the 32K workload's shape rules at 3K tokens and batch 2: K = 16, a 1024-token dense
    # prefix, many segments per block, split blocks and full chunk rings
    # head_dim 64: the library pads q, k, v, out, dO to 128 zero columns and runs the same kernels
    "d64_g4": W0.scaled(name="bwd_d64_g4", n_q_heads=8, n_kv_heads=2, head_dim=64, seq_len=1000, top_k=4,
                        dense_threshold=300, n_plant=2),
    "d64_g2_b2": W0.scaled(name="bwd_d64_g2", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=777,
                           top_k=3, dense_threshold=0, n_plant=2),
    "t3072_k16_b2": W0.scaled(name="bwd_t3k", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=3072,
                              top_k=16, dense_threshold=1024, n_plant=8),
}


def _close(name, got, ref, mean_tol):
    err = np.abs(got - ref)
    scale_max, scale_mean = np.abs(ref).max(), np.abs(ref).mean()
    note(f"  {name}: max-abs {err.max():.3e} (ref max {scale_max:.3e}), mean-abs {err.mean():.3e} "
         f"(ref mean {scale_mean:.3e})")
    bad = []
    if err.max() > 2e-2 * scale_max + 1e-6:
        bad.append(f"{name} max-abs")
    if err.mean() > mean_tol * scale_mean + 1e-7:
        bad.append(f"{name} mean-abs")
    return bad


def run_backward(w, seed=0):
    note(f"backward case {w.name}: B{w.batch} Hq{w.n_q_heads}/Hkv{w.n_kv_heads} T{w.seq_len} K{w.top_k} "
         f"thr{w.dense_threshold}")
    d = synth.generate(w, seed=seed)
    T = w.seq_len
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    fw = ops.sparse_prefill(cfg, q, k, v)
    rng = np.random.default_rng(seed + 7)
    dout_h = synth.to_bf16_bits(rng.standard_normal(d["q"].shape).astype(np.float32)).reshape(d["q"].shape)
    dout = dev_bf16(dout_h)
    g = ops.sparse_prefill_backward(cfg, q, k, v, fw["idx"], fw["out"], fw["lse"], dout, kv_len=T)
    torch.cuda.synchronize()
    idx = fw["idx"].cpu().numpy()
    pos = orc.positions("prefill", T, 0)
    dq, dk, dv = orc.attend_backward(orc.MODE_SPARSE, d["q"], d["k"], d["v"], pos, T, w.n_kv_heads, dout_h,
                                     idx=idx, dense_threshold=w.dense_threshold)
    bad = _close("dq", g["dq"].cpu().numpy(), dq, 1e-2)
    bad += _close("dk", g["dk"].cpu().numpy()[:, :, :T], dk[:, :, :T], 2e-3)
    bad += _close("dv", g["dv"].cpu().numpy()[:, :, :T], dv[:, :, :T], 2e-3)
    assert not bad, bad
    return g


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_backward_matches_oracle(case):
    run_backward(CASES[case])


def _rows_per_block(idx, T, K, G, dense_threshold):
    """Query rows (token x head of the group) attending each key block, from the selection."""
    nblk = (T - 1) // 64 + 1
    cnt = np.zeros((idx.shape[0], idx.shape[1], nblk), np.int64)
    for b in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            for t in range(T):
                own = t // 64
                if dense_threshold > 0 and t + 1 < dense_threshold:
                    cnt[b, g, :own + 1] += 1
                    continue
                sel = [j for j in idx[b, g, t] if 0 <= j < own]
                cnt[b, g, sel] += 1
                cnt[b, g, own] += 1
    return cnt * G


HEAVY = {
    # K = 16 covers every candidate for the first 1088 tokens, so block 0 is
    # attended by more than 1024 tokens = 4096 rows of a 4-head group
    "g4": W0.scaled(name="bwd_heavy_g4", n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=1600, top_k=16,
                    dense_threshold=0, n_plant=8),
    # 16 heads per group: 256 tokens already fill one segment
    "g16": W0.scaled(name="bwd_heavy_g16", n_q_heads=16, n_kv_heads=1, head_dim=128, seq_len=1300, top_k=8,
                     dense_threshold=0, n_plant=4),
}


@pytest.mark.parametrize("case", list(HEAVY))
def test_prefill_backward_heavy_keys_split_atomically(case):
    # blocks attended by more than one segment's 4096 query rows have their
    # dk, dv summed over several workgroups with fp32 atomics
    w = HEAVY[case]
    g = run_backward(w)
    cfg = cfg_of(w)
    d = synth.generate(w, seed=0)
    fw = ops.sparse_prefill(cfg, dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]))
    rows = _rows_per_block(fw["idx"].cpu().numpy(), w.seq_len, w.top_k, w.group, w.dense_threshold)
    assert rows.max() > 4096, f"no block needs a split (max rows {rows.max()})"


@pytest.mark.parametrize("n_q,kv_len,thr,D", [(500, 1200, 0, 128), (333, 900, 700, 128), (64, 2000, 0, 128),
                                               (300, 1100, 0, 64)])
def test_prefill_backward_chunk_after_prefix(n_q, kv_len, thr, D):
    """A chunk of n_q queries at positions kv_len - n_q .. kv_len - 1 over a longer cache:
    prefix keys get dk, dv from the rows that attend them; rows past kv_len stay untouched."""
    w = W0.scaled(name="bwd_chunk", n_q_heads=8, n_kv_heads=2, head_dim=D, seq_len=kv_len, top_k=4,
                  dense_threshold=thr, n_plant=2)
    note(f"backward chunk n_q{n_q} kv_len{kv_len} thr{thr} D{D}")
    d = synth.generate(w, seed=9)
    cfg = cfg_of(w)
    cap = d["kv_cap"]
    P = kv_len - n_q
    qh = np.ascontiguousarray(d["q"][:, :, P:])
    q, k, v = dev_bf16(qh), dev_bf16(d["k"]), dev_bf16(d["v"])
    kbar = ops.pool_kernels(cfg, k, cap, kv_len)
    idx = torch.empty((1, w.n_kv_heads, n_q, w.top_k), dtype=torch.int32, device="cuda")
    lib.infllmv2_topk_blocks(cfg, None, q, kbar, n_q, P, 0, cap, idx, None)
    out = torch.empty_like(q)
    lse = torch.empty((1, w.n_q_heads, n_q), dtype=torch.float32, device="cuda")
    lib.infllmv2_sparse_attn_prefill(cfg, q, n_q, k, v, cap, kv_len, idx, out, lse, None)
    rng = np.random.default_rng(11)
    dout_h = synth.to_bf16_bits(rng.standard_normal(qh.shape).astype(np.float32)).reshape(qh.shape)
    g = ops.sparse_prefill_backward(cfg, q, k, v, idx, out, lse, dev_bf16(dout_h), kv_len=kv_len)
    torch.cuda.synchronize()
    pos = orc.positions("prefill", n_q, P)
    dq, dk, dv = orc.attend_backward(orc.MODE_SPARSE, qh, d["k"], d["v"], pos, kv_len, w.n_kv_heads, dout_h,
                                     idx=idx.cpu().numpy(), dense_threshold=thr)
    bad = _close("dq", g["dq"].cpu().numpy(), dq, 1e-2)
    bad += _close("dk", g["dk"].cpu().numpy()[:, :, :kv_len], dk[:, :, :kv_len], 2e-3)
    bad += _close("dv", g["dv"].cpu().numpy()[:, :, :kv_len], dv[:, :, :kv_len], 2e-3)
    assert not bad, bad
    assert (g["dk"][:, :, kv_len:] == 0).all() and (g["dv"][:, :, kv_len:] == 0).all()


def test_prefill_backward_32k_full_size_sampled():
    """The benchmark's backward workload (32K tokens, 32/8 heads, K = 16, dense below 1024) in
    its launch configuration. dq is checked on sampled rows: a row's gradient depends only on its
    own key set, so the oracle computes it from those rows alone. dk and dv are checked on
    sampled key blocks of two groups: the oracle runs every row that attends the block (from the
    GPU forward's selection), which makes its dk, dv of that block exact."""
    w = synth.WORKLOADS["prefill_32k"]
    T, G, K, thr = w.seq_len, w.group, w.top_k, w.dense_threshold
    d = synth.generate(w, seed=0, threads=16)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    fw = ops.sparse_prefill(cfg, q, k, v)
    rng = np.random.default_rng(21)
    dout_h = synth.to_bf16_bits(rng.standard_normal(d["q"].shape).astype(np.float32)).reshape(d["q"].shape)
    g_res = ops.sparse_prefill_backward(cfg, q, k, v, fw["idx"], fw["out"], fw["lse"], dev_bf16(dout_h),
                                        kv_len=T)
    torch.cuda.synchronize()
    idx = fw["idx"].cpu().numpy()
    dq_gpu = g_res["dq"].cpu().numpy()

    # dq: sampled tokens (block edges, the dense threshold, the last token), every head
    toks = np.array(sorted(set([0, 63, 64, 1022, 1023, 1024, 4095, 4096, 20000, T - 1]
                               + rng.integers(0, T, 22).tolist())), dtype=np.int64)
    note(f"backward 32K: dq on {len(toks)} tokens x {w.n_q_heads} heads")
    dq_ref, _, _ = orc.attend_backward(orc.MODE_SPARSE, np.ascontiguousarray(d["q"][:, :, toks]), d["k"], d["v"],
                                       toks, T, w.n_kv_heads, np.ascontiguousarray(dout_h[:, :, toks]),
                                       idx=np.ascontiguousarray(idx[:, :, toks]), dense_threshold=thr)
    bad = _close("dq (sampled rows)", dq_gpu[:, :, toks], dq_ref, 1e-2)

    # dk, dv: per group, the last block (attended by its own tokens only), the sparse-region
    # block attended by the most tokens up to 1500 (selected by many rows), and the last block
    # of the dense prefix (attended by every dense row past it and by selecting rows) when it
    # has at most 3000 attending tokens
    own = np.arange(T) // 64
    for g in (0, 5):
        att = np.zeros((T, T // 64), dtype=bool)
        att[np.arange(T), own] = True
        dense = np.arange(T) + 1 < thr
        att[dense] = np.arange(T // 64)[None, :] <= own[dense, None]
        sel = idx[0, g]
        ok = (sel >= 0) & (sel < own[:, None])
        tt, kk = np.nonzero(ok)
        att[tt, sel[tt, kk]] = True
        counts = att.sum(axis=0)
        sparse_blocks = np.arange(thr // 64 + 1, T // 64 - 1)
        modest = sparse_blocks[counts[sparse_blocks] <= 1500]
        picks = [T // 64 - 1, int(modest[np.argmax(counts[modest])])]
        if counts[thr // 64 - 1] <= 3000:
            picks.append(thr // 64 - 1)
        for j in picks:
            rows_t = np.nonzero(att[:, j])[0].astype(np.int64)
            note(f"backward 32K: group {g} block {j}: {len(rows_t)} attending tokens")
            hs = slice(g * G, (g + 1) * G)
            _, dk_ref, dv_ref = orc.attend_backward(
                orc.MODE_SPARSE, np.ascontiguousarray(d["q"][:, hs][:, :, rows_t]),
                np.ascontiguousarray(d["k"][:, g:g + 1]), np.ascontiguousarray(d["v"][:, g:g + 1]), rows_t, T, 1,
                np.ascontiguousarray(dout_h[:, hs][:, :, rows_t]),
                idx=np.ascontiguousarray(idx[:, g:g + 1][:, :, rows_t]), dense_threshold=thr)
            keys = slice(j * 64, (j + 1) * 64)
            bad += _close(f"dk g{g} b{j}", g_res["dk"][0, g, keys].cpu().numpy(), dk_ref[0, 0, keys], 2e-3)
            bad += _close(f"dv g{g} b{j}", g_res["dv"][0, g, keys].cpu().numpy(), dv_ref[0, 0, keys], 2e-3)
    assert not bad, bad
