"""GPU parity of the decode loop's cache maintenance and of variable-length batches.

Appending writes the new tokens' K and V rows exactly (bit for bit) and pools
exactly the blocks the append completes (k̄ bit-exact against the oracle's
pooling of the updated cache, every other entry untouched). A loop of
append -> score -> select -> attend steps, with equal or per-sequence lengths,
matches the oracle at every step: block indices bit-exact, outputs within
max-abs 2e-2 / mean-abs 2e-3, lse within 2e-3. Selection boundaries are opened
by redrawing queries with the oracle (tests/gaps.py).
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from trainable_block_sparse_infllm_amd import ops
from oracle.gaps import open_gaps
from gpu_util import LSE_ABS, assert_close_rows, cfg_of, dev_bf16, host_f64, kbar_rows, note

pytestmark = pytest.mark.gpu

D0 = synth.WORKLOADS["decode_32k"]
SENTINEL = 0x4480                        # bf16 1024.0: marks cache rows no append should touch


def _workload(B, L, **kw):
    base = dict(name="loop", batch=B, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=L, top_k=8,
                dense_threshold=1024, n_plant=4)
    base.update(kw)
    return D0.scaled(**base)


def _kbar_host(kbar):
    """GPU k̄ -> [B][Hkv][nblk][3][D] bf16 bits."""
    return kbar_rows(kbar)


@pytest.mark.parametrize("D", [128, 64], ids=["d128", "d64"])
@pytest.mark.parametrize("varlen", [False, True], ids=["same_len", "varlen"])
@pytest.mark.parametrize("n_new", [1, 5, 64, 150])
def test_append_writes_rows_and_pools_completed_blocks(varlen, n_new, D):
    B, L = 3, 1400
    w = _workload(B, L, head_dim=D)
    d = synth.generate(w, seed=5)
    cap = d["kv_cap"]
    lens0 = [130, 63, 1000] if varlen else [700] * B
    note(f"append case D{D} n_new{n_new} lens{lens0}")
    kf, vf = d["k"], d["v"]                                   # the full sequences
    kc = np.full_like(kf, SENTINEL)
    vc = np.full_like(vf, SENTINEL)
    kn = np.empty((B, w.n_kv_heads, n_new, w.head_dim), np.uint16)
    vn = np.empty_like(kn)
    for b, l0 in enumerate(lens0):
        kc[b, :, :l0] = kf[b, :, :l0]
        vc[b, :, :l0] = vf[b, :, :l0]
        kn[b] = kf[b, :, l0:l0 + n_new]
        vn[b] = vf[b, :, l0:l0 + n_new]
    cfg = cfg_of(w)
    k_cache, v_cache = dev_bf16(kc), dev_bf16(vc)
    kbar = torch.zeros(ops.kbar_shape(B, w.n_kv_heads, cap, w.head_dim), dtype=torch.bfloat16, device="cuda")
    if varlen:
        lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
        ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_lens=lens)
    else:
        ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_len=lens0[0])
    torch.cuda.synchronize()
    kg = k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    kb = _kbar_host(kbar)
    for b, l0 in enumerate(lens0):
        l1 = l0 + n_new
        assert np.array_equal(kg[b, :, :l1], kf[b, :, :l1]) and np.array_equal(vg[b, :, :l1], vf[b, :, :l1])
        assert (kg[b, :, l1:] == SENTINEL).all() and (vg[b, :, l1:] == SENTINEL).all()
        ref = orc.pool(kf[b:b + 1], l1)[0]                   # [Hkv][nblk][3][D]
        done = range(l0 // 64, l1 // 64)                      # blocks this append completes
        for j in range(kb.shape[2]):
            if j in done:
                assert np.array_equal(kb[b, :, j], ref[:, j]), (b, j)
            else:
                assert (kb[b, :, j] == 0).all(), (b, j)


def test_append_past_capacity_is_cut():
    """Per-sequence appends that reach past the cache capacity: rows at or past kv_cap are not
    written, and only blocks that end within the capacity are pooled (the last one completed
    by rows of the append)."""
    B, L, n_new = 3, 1400, 40
    w = _workload(B, L, head_dim=128)
    d = synth.generate(w, seed=6)
    cap = d["kv_cap"]                                        # 1408: 22 blocks
    lens0 = [1380, 1350, 1407]
    note(f"append past capacity: cap {cap} n_new {n_new} lens {lens0}")
    rng = np.random.default_rng(6)
    kc, vc = d["k"].copy(), d["v"].copy()
    for b, l0 in enumerate(lens0):
        kc[b, :, l0:] = SENTINEL
        vc[b, :, l0:] = SENTINEL
    kn = synth.to_bf16_bits(rng.standard_normal((B, w.n_kv_heads, n_new, w.head_dim)).astype(np.float32))
    vn = synth.to_bf16_bits(rng.standard_normal((B, w.n_kv_heads, n_new, w.head_dim)).astype(np.float32))
    cfg = cfg_of(w)
    k_cache, v_cache = dev_bf16(kc), dev_bf16(vc)
    kbar = torch.zeros(ops.kbar_shape(B, w.n_kv_heads, cap, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
    ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_lens=lens)
    torch.cuda.synchronize()
    kg = k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    kb = _kbar_host(kbar)
    for b, l0 in enumerate(lens0):
        l1 = min(l0 + n_new, cap)
        want_k, want_v = kc[b].copy(), vc[b].copy()
        want_k[:, l0:l1] = kn[b, :, :l1 - l0]
        want_v[:, l0:l1] = vn[b, :, :l1 - l0]
        assert np.array_equal(kg[b], want_k) and np.array_equal(vg[b], want_v), b
        ref = orc.pool(want_k[None], l1)[0]
        done = range(l0 // 64, l1 // 64)
        for j in range(kb.shape[2]):
            if j in done:
                assert np.array_equal(kb[b, :, j], ref[:, j]), (b, j)
            else:
                assert (kb[b, :, j] == 0).all(), (b, j)


def _oracle_step(w, q, kf, vf, b, L):
    """The oracle's decode of sequence b's token at position L - 1 over its first L keys."""
    kbar_o = orc.pool(kf[b:b + 1], L)
    return orc.sparse_forward(q[b:b + 1], kf[b:b + 1], vf[b:b + 1], kv_len=L, q_pos0=L - 1,
                              n_kv_heads=w.n_kv_heads, top_k=w.top_k, dense_threshold=w.dense_threshold,
                              kbar=kbar_o)


def _open_step_gaps(w, q, kf, lens, seed):
    G = w.group
    for b, L in enumerate(lens):
        d = dict(workload=w, seed=seed, q=q, k=kf, kv_len=L, n_q=1, q_pos0=L - 1)
        rows = [(b, g, 0) for g in range(w.n_kv_heads)]
        open_gaps(d, orc, group_rows=rows, kbar=orc.pool(kf, L), pos=np.array([L - 1]))
    return q


@pytest.mark.parametrize("D", [128, 64], ids=["d128", "d64"])
@pytest.mark.parametrize("varlen", [False, True], ids=["same_len", "varlen"])
def test_decode_loop_append_then_attend(varlen, D):
    """Three steps of append(1 token) -> scores -> select -> attend. The lengths cross
    block boundaries (a block completed by one step's append is a candidate in the
    next) and one sequence stays below the dense threshold."""
    B, steps = 4, 3
    w = _workload(B, 3300, head_dim=D)
    d = synth.generate(w, seed=6)
    kf, vf, cap = d["k"], d["v"], d["kv_cap"]
    lens0 = [127, 3000, 900, 64 * 40 - 1] if varlen else [2047] * B
    cfg = cfg_of(w)
    # caches hold each sequence's first lens0[b] tokens; k̄ pooled per sequence
    kc = np.full_like(kf, SENTINEL)
    vc = np.full_like(vf, SENTINEL)
    for b, l0 in enumerate(lens0):
        kc[b, :, :l0] = kf[b, :, :l0]
        vc[b, :, :l0] = vf[b, :, :l0]
    k_cache, v_cache = dev_bf16(kc), dev_bf16(vc)
    kbar = torch.zeros(ops.kbar_shape(B, w.n_kv_heads, cap, w.head_dim), dtype=torch.bfloat16, device="cuda")
    for b, l0 in enumerate(lens0):
        one = cfg_of(w, batch=1)
        ops.pool_kernels(one, k_cache[b:b + 1], cap, l0, kbar=kbar[b:b + 1])
    lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
    cur = list(lens0)
    for s in range(steps):
        note(f"loop step {s}: lens {cur} -> +1")
        kn = np.stack([kf[b, :, cur[b]:cur[b] + 1] for b in range(B)])
        vn = np.stack([vf[b, :, cur[b]:cur[b] + 1] for b in range(B)])
        if varlen:
            ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_lens=lens)
            lens += 1
        else:
            ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_len=cur[0])
        cur = [c + 1 for c in cur]
        q = synth.generate(w, seed=100 + s)["q"]
        q = _open_step_gaps(w, q, kf, cur, 100 + s)
        if varlen:
            res = ops.decode_step_varlen(cfg, dev_bf16(q), k_cache, v_cache, kbar, lens, max(cur))
        else:
            res = ops.decode_step(cfg, dev_bf16(q), k_cache, v_cache, kbar, cur[0])
        torch.cuda.synchronize()
        gidx = res["idx"].cpu().numpy()
        gout, glse = host_f64(res["out"]), host_f64(res["lse"])
        for b in range(B):
            ref = _oracle_step(w, q, kf, vf, b, cur[b])
            assert np.array_equal(gidx[b:b + 1], ref["idx"]), f"step {s} seq {b}: block indices differ"
            hr = ref["head_rows"]
            assert_close_rows(gout[b][hr[:, 1], hr[:, 2]], ref["out"], f"step {s} seq {b} out")
            assert np.abs(glse[b][hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS


def test_varlen_scores_match_oracle_and_mask_past_candidates():
    B = 4
    w = _workload(B, 5000, top_k=16)
    d = synth.generate(w, seed=7)
    kf, cap = d["k"], d["kv_cap"]
    lens0 = [5000, 64, 1025, 4097]
    cfg = cfg_of(w)
    k = dev_bf16(kf)
    kbar = ops.pool_kernels(cfg, k, cap, 5000)
    lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
    q = d["q"]
    scores = torch.full((B, w.n_kv_heads, 1, cap // 64), 7.0, dtype=torch.float32, device="cuda")
    from trainable_block_sparse_infllm_amd import capi
    capi.infllmv2_score_blocks_varlen(cfg, dev_bf16(q), lens, kbar, cap, scores)
    torch.cuda.synchronize()
    gs = scores.cpu().numpy()
    for b, L in enumerate(lens0):
        kbar_o = orc.pool(kf[b:b + 1], L)
        pos = np.array([L - 1])
        R, Cn = orc.scores(q[b:b + 1], kbar_o, pos, orc.all_group_rows(1, w.n_kv_heads, 1), w.n_kv_heads)
        C = (L - 1) // 64
        for g in range(w.n_kv_heads):
            row = gs[b, g, 0]
            assert np.all(np.isneginf(row[C:])), (b, g)
            assert np.allclose(row[:C], R[g, :C], rtol=1e-5, atol=1e-3), (b, g)


def test_varlen_decode_128k_batch8_full_size():
    """The measured decode_128k_b8 shapes with per-sequence lengths 131072 - 4096 b: an append
    of one token per sequence, then varlen scores, selection and attention, checked against the
    oracle for every sequence."""
    w = synth.WORKLOADS["decode_128k_b8"]
    d = synth.generate(w, seed=0, threads=16)
    kf, vf, cap = d["k"], d["v"], d["kv_cap"]
    B = w.batch
    lens0 = [131071 - 4096 * b for b in range(B)]
    cur = [L + 1 for L in lens0]
    note(f"varlen full size: lengths {cur}")
    cfg = cfg_of(w)
    k_cache, v_cache = dev_bf16(kf), dev_bf16(vf)
    kbar = ops.pool_kernels(cfg, k_cache, cap, min(lens0))
    for b, l0 in enumerate(lens0):                       # each sequence's complete blocks
        ops.pool_kernels(cfg_of(w, batch=1), k_cache[b:b + 1], cap, l0, kbar=kbar[b:b + 1])
    kn = np.stack([kf[b, :, lens0[b]:lens0[b] + 1] for b in range(B)])
    vn = np.stack([vf[b, :, lens0[b]:lens0[b] + 1] for b in range(B)])
    lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
    ops.append_kv(cfg, dev_bf16(kn), dev_bf16(vn), k_cache, v_cache, kbar, kv_lens=lens)
    lens += 1
    q = _open_step_gaps(w, d["q"].copy(), kf, cur, 0)
    res = ops.decode_step_varlen(cfg, dev_bf16(q), k_cache, v_cache, kbar, lens, max(cur))
    torch.cuda.synchronize()
    gidx = res["idx"].cpu().numpy()
    gout, glse = host_f64(res["out"]), host_f64(res["lse"])
    for b in range(B):
        ref = _oracle_step(w, q, kf, vf, b, cur[b])
        assert np.array_equal(gidx[b:b + 1], ref["idx"]), f"seq {b}: block indices differ"
        hr = ref["head_rows"]
        assert_close_rows(gout[b][hr[:, 1], hr[:, 2]], ref["out"], f"seq {b} out")
        assert np.abs(glse[b][hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS
