"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Bars: kernels (k̄) and block indices bit-exact; block scores within fp32
accumulation error; attention outputs within max-abs 2e-2 and mean-abs 2e-3 of
the fp64 oracle (bf16 in, fp32 accumulate, bf16 out); lse within 2e-3.
Inputs are seeded (synth) with top-K boundaries opened to > 1e-3 by the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
import trainable_block_sparse_infllm_amd as lib
from trainable_block_sparse_infllm_amd import ops
from oracle.gaps import open_gaps
from gpu_util import (LSE_ABS, assert_close_rows, cfg_of, check_idx_rows, dev_bf16, dev_i32, dev_u64, kbar_rows,
                      host_f64, host_u16, note)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
P0 = W["prefill_32k"]
D0 = W["decode_32k"]
T0 = W["tree_128k"]

PREFILL_CASES = {
    "g4_d128_ragged_thr": P0.scaled(name="p_g4", n_q_heads=8, n_kv_heads=2, seq_len=1000, top_k=4,
                                    dense_threshold=300, n_plant=3),
    "g2_d64_b2": P0.scaled(name="p_g2", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=777,
                           top_k=3, dense_threshold=0, n_plant=2),
    "g1_d64": P0.scaled(name="p_g1", n_q_heads=2, n_kv_heads=2, head_dim=64, seq_len=600, top_k=2,
                        dense_threshold=100, n_plant=2),
    "g8_d128": P0.scaled(name="p_g8", n_q_heads=16, n_kv_heads=2, seq_len=520, top_k=3, dense_threshold=0,
                         n_plant=2),
    "g16_d64": P0.scaled(name="p_g16", n_q_heads=16, n_kv_heads=1, head_dim=64, seq_len=300, top_k=2,
                         dense_threshold=0, n_plant=1),
    "g1_d128": P0.scaled(name="p_g1_128", n_q_heads=2, n_kv_heads=2, seq_len=700, top_k=3,
                         dense_threshold=200, n_plant=2),
    "g2_d128_b2": P0.scaled(name="p_g2_128", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=900, top_k=5,
                            dense_threshold=0, n_plant=3),
    "g16_d128": P0.scaled(name="p_g16_128", n_q_heads=16, n_kv_heads=1, seq_len=300, top_k=2,
                          dense_threshold=0, n_plant=1),
    "short_no_candidates": P0.scaled(name="p_short", n_q_heads=8, n_kv_heads=2, seq_len=50, top_k=4,
                                     dense_threshold=0, n_plant=0),
    "tiny_prefill_2k": W["tiny_prefill_2k"],
    "prefill_4k_full_heads": P0.scaled(name="p_4k", seq_len=4096),
    # head_dim 64 with enough (b, g) tiles for the rows kernel's full sub-tile count (the small
    # cases above take its one-sub-tile form)
    "d64_full_tiles": P0.scaled(name="p_d64_big", batch=2, n_q_heads=16, n_kv_heads=8, head_dim=64,
                                seq_len=4096, top_k=8, dense_threshold=1024, n_plant=4),
}

DECODE_CASES = {
    "b2_g4_d128": D0.scaled(name="d_small", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=5000, top_k=8,
                            n_plant=8),
    "dense_below_threshold": D0.scaled(name="d_dense", n_q_heads=8, n_kv_heads=2, seq_len=700, top_k=4,
                                       n_plant=2),
    "no_candidates": D0.scaled(name="d_tiny", n_q_heads=8, n_kv_heads=2, seq_len=30, top_k=4, n_plant=0,
                               dense_threshold=0),
    "g2_d64_k_exceeds": D0.scaled(name="d_g2", n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=1500,
                                  top_k=40, n_plant=3, dense_threshold=0),
    "decode_32k": D0,
    # the largest K the in-kernel selection takes, over 2047 candidates
    "k64_128k": D0.scaled(name="d_k64", seq_len=131072, top_k=64, n_plant=32),
}

TREE_CASES = {
    "p1000_n7_d64": T0.scaled(name="t_small", n_q_heads=8, n_kv_heads=2, head_dim=64, seq_len=1000, top_k=4,
                              n_plant=4, n_tree=7, tree_depth=3, dense_threshold=0),
    "p4096_n16_d128": T0.scaled(name="t_mid", seq_len=4096, top_k=8, n_plant=8),
    "dense_prefix": T0.scaled(name="t_dense", n_q_heads=8, n_kv_heads=2, seq_len=500, top_k=2, n_plant=2,
                              n_tree=5, tree_depth=3),
    "single_node": T0.scaled(name="t_one", n_q_heads=8, n_kv_heads=2, seq_len=2000, top_k=4, n_plant=4,
                             n_tree=1, tree_depth=1, dense_threshold=0),
    # 160 (node, head) rows: the scoring kernel's two-tile wavefronts and a partial last row tile
    "p2048_n40_d128": T0.scaled(name="t_n40", seq_len=2048, top_k=8, n_plant=8, n_tree=40, tree_depth=6),
    # GQA 8: 128 rows per group, 625 candidates (selection by eight wavefronts per row)
    "g8_p40000": T0.scaled(name="t_g8", n_q_heads=16, n_kv_heads=2, seq_len=40000, top_k=16, n_plant=8),
    # GQA 16: 256 rows per group (two-tile scoring wavefronts, head sums across lane pairs)
    "g16_p3000": T0.scaled(name="t_g16", n_q_heads=16, n_kv_heads=1, seq_len=3000, top_k=8, n_plant=4),
}


def _kbar_check(d, kbar_gpu, kbar_o):
    nfull = d["kv_len"] // 64
    g = kbar_rows(kbar_gpu)
    assert np.array_equal(g[:, :, :nfull], kbar_o[:, :, :nfull]), "k̄ differs from the oracle"


# ---------------------------------------------------------------------------- prefill
def run_prefill(w, seed=0, group_rows=None):
    note(f"prefill case {w.name}: B{w.batch} Hq{w.n_q_heads}/Hkv{w.n_kv_heads} D{w.head_dim} "
         f"T{w.seq_len} K{w.top_k} thr{w.dense_threshold} seed{seed}")
    d = synth.generate(w, seed=seed)
    kbar_o, redrawn, _ = open_gaps(d, orc, group_rows=group_rows)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], q_pos0=0, n_kv_heads=w.n_kv_heads,
                             top_k=w.top_k, dense_threshold=w.dense_threshold, group_rows=group_rows,
                             kbar=kbar_o)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    res = ops.sparse_prefill(cfg, q, k, v)
    torch.cuda.synchronize()
    _kbar_check(d, res["kbar"], kbar_o)
    gidx = res["idx"].cpu().numpy()
    gr = ref["group_rows"]
    assert np.array_equal(gidx[gr[:, 0], gr[:, 1], gr[:, 2]], ref["sel"]), "block indices differ"
    hr = ref["head_rows"]
    gout = host_f64(res["out"])[hr[:, 0], hr[:, 1], hr[:, 2]]
    assert_close_rows(gout, ref["out"], f"{w.name} out")
    glse = host_f64(res["lse"])[hr[:, 0], hr[:, 1], hr[:, 2]]
    assert np.abs(glse - ref["lse"]).max() <= LSE_ABS
    return d, ref, res


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_end_to_end(case):
    run_prefill(PREFILL_CASES[case])


def test_prefill_attention_with_oracle_indices():
    w = PREFILL_CASES["g4_d128_ragged_thr"]
    d = synth.generate(w, seed=3)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], q_pos0=0, n_kv_heads=w.n_kv_heads,
                             top_k=w.top_k, dense_threshold=w.dense_threshold)
    cfg = cfg_of(w)
    out = torch.empty((w.batch, w.n_q_heads, w.seq_len, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lib.infllmv2_sparse_attn_prefill(cfg, dev_bf16(d["q"]), w.seq_len, dev_bf16(d["k"]), dev_bf16(d["v"]),
                                     d["kv_cap"], d["kv_len"], dev_i32(ref["idx"]), out, None)
    torch.cuda.synchronize()
    hr = ref["head_rows"]
    assert_close_rows(host_f64(out)[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], "prefill attention")


@pytest.mark.parametrize("n_q,kv_len,thr", [(300, 1500, 1300), (64, 2000, 0), (37, 1111, 0)])
def test_prefill_attention_chunk_with_oracle_indices(n_q, kv_len, thr):
    """A chunk of n_q queries at the end of a longer context (positions
    kv_len - n_q .. kv_len - 1), block indices from the oracle."""
    w = PREFILL_CASES["g4_d128_ragged_thr"].scaled(name="p_chunk", seq_len=kv_len, dense_threshold=thr)
    note(f"prefill chunk n_q{n_q} kv_len{kv_len} thr{thr}")
    d = synth.generate(w, seed=4)
    qn = np.ascontiguousarray(d["q"][:, :, kv_len - n_q:])
    ref = orc.sparse_forward(qn, d["k"], d["v"], kv_len=kv_len, q_pos0=kv_len - n_q, n_kv_heads=w.n_kv_heads,
                             top_k=w.top_k, dense_threshold=thr)
    cfg = cfg_of(w)
    out = torch.empty((w.batch, w.n_q_heads, n_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads, n_q), dtype=torch.float32, device="cuda")
    lib.infllmv2_sparse_attn_prefill(cfg, dev_bf16(qn), n_q, dev_bf16(d["k"]), dev_bf16(d["v"]),
                                     d["kv_cap"], kv_len, dev_i32(ref["idx"]), out, lse)
    torch.cuda.synchronize()
    hr = ref["head_rows"]
    assert_close_rows(host_f64(out)[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], "prefill chunk")
    assert np.abs(host_f64(lse)[hr[:, 0], hr[:, 1], hr[:, 2]] - ref["lse"]).max() <= LSE_ABS


# Whole 32-token tiles of the 32K prefill compared row by row (every token of the tile, all
# query heads of every KV group): the attention kernel's tile for GQA 4 is 32 tokens and the
# fused top-K kernel's 16, so each listed tile covers whole workgroups of both. Depths spread
# over the sequence; tile 31 (tokens 992-1023) holds the dense-threshold boundary (row 1022
# dense, 1023 sparse), tiles 32 and 33 the first fully sparse rows, tile 1023 the last token.
PREFILL_32K_TILES = [0, 1, 31, 32, 33, 64, 127, 200, 255, 256, 400, 511, 512, 700, 900, 1023]


def test_prefill_32k_full_size_whole_tiles():
    """The full prefill workload in the benchmark's launch configuration; the
    oracle checks every row of 16 whole 32-token tiles per KV group (block
    edges, the dense threshold boundary, the last token), and every selection
    row of the call is checked for validity."""
    w = P0
    toks = [32 * tile + t for tile in PREFILL_32K_TILES for t in range(32)]
    rows = np.array([(0, g, t) for g in range(w.n_kv_heads) for t in toks], dtype=np.int32)
    d, ref, res = run_prefill(w, seed=0, group_rows=rows)
    gidx = res["idx"].cpu().numpy().reshape(-1, w.top_k)
    C = np.tile(np.arange(w.seq_len) // 64, w.batch * w.n_kv_heads)
    check_idx_rows(gidx, C, w.top_k)


# (table length, first row's candidate count, K, value stored past each row's candidates):
# one wavefront per row (C <= 256), and one workgroup per row (C > 512; K above 64 takes its
# exact fallback; C % 4 == 0 and != 0 both occur among the 5 rows; values past C that would
# win if read)
TOPK_SCORE_CASES = [(300, 250, 16, -np.inf), (2100, 2040, 16, 1e30), (2100, 2040, 64, -np.inf),
                    (2100, 2040, 100, 1e30), (700, 600, 32, 1e30)]


@pytest.mark.parametrize("nblk,c0,K,tail", TOPK_SCORE_CASES)
def test_topk_from_fp32_scores_is_exact_with_ties(nblk, c0, K, tail):
    """Selection from a score tensor equals the oracle's rule on the same fp32
    scores, ties included (scores quantized so that many are equal)."""
    rng = np.random.default_rng(5)
    B, Hkv, n_q = 2, 3, 5
    note(f"top-K from scores: nblk {nblk} C {c0}..{c0 + n_q - 1} K {K} tail {tail}")
    R = np.round(rng.standard_normal((B * Hkv * n_q, nblk)) * 4) / 4
    q_pos0 = 64 * c0
    C = np.tile((q_pos0 + np.arange(n_q)) // 64, B * Hkv)
    for r in range(R.shape[0]):
        R[r, C[r]:] = -np.inf
    ref = orc.select(R.astype(np.float32).astype(np.float64), C, K)
    for r in range(R.shape[0]):
        R[r, C[r]:] = tail
    cfg = lib.make_cfg(B, Hkv * 4, Hkv, 128, top_k=K)
    idx = torch.empty((B, Hkv, n_q, K), dtype=torch.int32, device="cuda")
    scores = torch.from_numpy(R.astype(np.float32)).cuda()
    lib.infllmv2_topk_blocks(cfg, scores, None, None, n_q, q_pos0, 0, nblk * 64, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().reshape(-1, K), ref)


def _fused_topk_chunk(w, L, n_q, tree, seed, periodic=0):
    """Scores + top-K of n_q query rows at the end of an L-token context (tree: all
    rows at position L - n_q) through the fused entry point, and the oracle's."""
    d = synth.generate(w, seed=seed)
    if periodic:
        for j in range(periodic, L // 64):
            d["k"][:, :, 64 * j:64 * j + 64] = d["k"][:, :, 64 * (j % periodic):64 * (j % periodic) + 64]
    P = L - n_q
    qn = np.ascontiguousarray(d["q"][:, :, P:])
    pos = np.full(n_q, P, dtype=np.int64) if tree else P + np.arange(n_q, dtype=np.int64)
    kbar_o = orc.pool(d["k"], L)
    rows = orc.all_group_rows(w.batch, w.n_kv_heads, n_q)
    if not periodic:
        dd = dict(d, q=qn, n_q=n_q, q_pos0=P)
        open_gaps(dd, orc, kbar=kbar_o, pos=pos)
        qn = dd["q"]
    R, Cn = orc.scores(qn, kbar_o, pos, rows, w.n_kv_heads)
    ref = orc.select(R, Cn, w.top_k)
    cfg = cfg_of(w)
    k = dev_bf16(d["k"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], L)
    idx = torch.empty((w.batch, w.n_kv_heads, n_q, w.top_k), dtype=torch.int32, device="cuda")
    lib.infllmv2_topk_blocks(cfg, None, dev_bf16(qn), kbar, n_q, P, int(tree), d["kv_cap"], idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy().reshape(-1, w.top_k), ref, R, Cn


@pytest.mark.parametrize("L,n_q,tree,hq,hkv,K", [(20000, 64, False, 8, 2, 16), (20000, 16, True, 8, 2, 16),
                                                 (40000, 64, False, 4, 1, 16), (9000, 40, False, 16, 2, 8),
                                                 (9000, 40, False, 16, 1, 5), (6000, 70, False, 2, 2, 12)])
def test_fused_topk_chunk_matches_oracle(L, n_q, tree, hq, hkv, K):
    """Fused scoring + selection for a chunk of queries late in a long context:
    at most 512 candidates and K <= 16 take the per-token-group kernel, 40000
    tokens (624 candidates) the general one."""
    w = P0.scaled(name="fused_chunk", n_q_heads=hq, n_kv_heads=hkv, seq_len=L, top_k=K, n_plant=4,
                  dense_threshold=0)
    note(f"fused top-K L{L} n_q{n_q} tree{tree} Hq{hq}/Hkv{hkv} K{K}")
    gidx, ref, _, _ = _fused_topk_chunk(w, L, n_q, tree, seed=13)
    assert np.array_equal(gidx, ref)


def test_fused_topk_exact_ties_take_lower_index():
    """Blocks repeating with period 5 tie exactly (identical kernels): the K
    selected are the lowest indices of the best class."""
    L, n_q = 8192, 64
    w = P0.scaled(name="fused_ties", n_q_heads=8, n_kv_heads=2, seq_len=L, top_k=16, n_plant=0,
                  dense_threshold=0)
    gidx, ref, R, Cn = _fused_topk_chunk(w, L, n_q, False, seed=17, periodic=5)
    for r in range(len(Cn)):
        top = np.unique(R[r, :Cn[r]])[::-1]
        assert top[0] - top[1] > 1e-3, "classes too close for an exact comparison"
    assert np.array_equal(gidx, ref)
    assert (np.diff(gidx, axis=1) % 5 == 0).all(), "selection should be one tie class"


# ---------------------------------------------------------------------------- decode / tree
def run_decode(w, seed=0, tree=True):
    mask = None
    note(f"decode case {w.name} ({w.mode}{'' if tree else ', rows without tree'}): B{w.batch} "
         f"Hq{w.n_q_heads}/Hkv{w.n_kv_heads} D{w.head_dim} kv_len{w.kv_len} n_q{w.n_q} K{w.top_k} seed{seed}")
    d = synth.generate(w, seed=seed)
    P = d["kv_len"] - d["n_q"]
    if w.mode == "tree" and tree:
        mask = d["tree_mask"]
        pos = np.full(d["n_q"], P, dtype=np.int64)
    else:
        pos = P + np.arange(d["n_q"], dtype=np.int64)
    kbar_o, _, _ = open_gaps(d, orc, pos=pos)
    ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], q_pos0=P, n_kv_heads=w.n_kv_heads,
                             top_k=w.top_k, dense_threshold=w.dense_threshold, tree_mask=mask, kbar=kbar_o)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], d["kv_len"])
    res = ops.decode(cfg, q, k, v, kbar, d["kv_len"], tree_mask=None if mask is None else dev_u64(mask))
    torch.cuda.synchronize()
    _kbar_check(d, kbar, kbar_o)
    gs = res["scores"].cpu().numpy().reshape(-1, ref["R"].shape[1])
    Ro = ref["R"]
    fin = np.isfinite(Ro)
    assert np.array_equal(np.isfinite(gs), fin), "candidate sets differ"
    assert (np.abs(gs[fin] - Ro[fin]) <= 1e-3 + 1e-5 * np.abs(Ro[fin])).all(), "block scores differ"
    gidx = res["idx"].cpu().numpy()
    assert np.array_equal(gidx, ref["idx"]), "block indices differ"
    hr = ref["head_rows"]
    gout = host_f64(res["out"])[hr[:, 0], hr[:, 1], hr[:, 2]]
    assert_close_rows(gout, ref["out"], f"{w.name} out")
    glse = host_f64(res["lse"])[hr[:, 0], hr[:, 1], hr[:, 2]]
    assert np.abs(glse - ref["lse"]).max() <= LSE_ABS
    return d, ref, res


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_end_to_end(case):
    run_decode(DECODE_CASES[case])


@pytest.mark.parametrize("case", list(TREE_CASES))
def test_tree_end_to_end(case):
    run_decode(TREE_CASES[case])


def test_tree_union_beyond_the_typical_size():
    """A tree whose nodes mostly pick different blocks (nothing planted): the
    union of a group exceeds the typical size the attention grid is sized for
    (about 2(K+1) blocks plus the rows' own), so its workgroups walk further
    splits in turn."""
    w = T0.scaled(name="t_wide", seq_len=16384, top_k=8, n_plant=0, dense_threshold=0)
    d, ref, _ = run_decode(w, seed=3)
    n_q, kv_len = d["n_q"], d["kv_len"]
    P = kv_len - n_q
    local = (kv_len - 1) // 64 - P // 64 + 1
    union = max(len({int(j) for j in ref["idx"][b, g].ravel() if j >= 0}) + local
                for b in range(w.batch) for g in range(w.n_kv_heads))
    sb = 4                                  # union entries per split for two 16-row sub-tiles
    typical = sb * -(-(2 * (w.top_k + 1) + -(-n_q // 64) + 1) // sb)
    assert union > typical, (union, typical)


def _decode_scores_matches_split_path(w, seed=0):
    """The fused entry (selection inside the attention kernel) reproduces the
    separate top-K + attention entry points bit for bit."""
    d, ref, res = run_decode(w, seed=seed)
    cfg = cfg_of(w)
    k, v = dev_bf16(d["k"]), dev_bf16(d["v"])
    q = dev_bf16(d["q"])
    out = torch.empty_like(res["out"])
    lse = torch.empty_like(res["lse"])
    idx = torch.full_like(res["idx"], -7)
    nbytes = lib.infllmv2_decode_workspace_bytes(cfg, 1, d["kv_len"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lib.infllmv2_sparse_attn_decode_scores(cfg, q, k, v, d["kv_cap"], d["kv_len"], res["scores"], idx, out, lse,
                                           ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(idx, res["idx"]), "selected blocks differ"
    assert torch.equal(out.view(torch.int16), res["out"].view(torch.int16)), "outputs differ"
    assert torch.equal(lse, res["lse"]), "lse differs"


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_from_scores_equals_split_path(case):
    _decode_scores_matches_split_path(DECODE_CASES[case])


def test_decode_from_scores_128k_batch8_full_size():
    _decode_scores_matches_split_path(W["decode_128k_b8"])


@pytest.mark.parametrize("B,Hkv,kv_len,kv_cap", [(8, 8, 131072, 131072),      # eight-wavefront selection
                                                # over 512 candidates with three-entry splits: the
                                                # workgroup gets five helper wavefronts for it
                                                (2, 4, 65636, 65636),
                                                (1, 8, 64 * 1026 + 5, 64 * 1027),  # rows not 16-byte aligned
                                                (2, 4, 30000, 30000),          # one-wavefront selection
                                                (1, 2, 16000, 16000)])
def test_decode_selection_from_scores_exact(B, Hkv, kv_len, kv_cap):
    """Selection inside the decode kernel equals the oracle's rule on hand-made
    fp32 scores: quantized values (many exact ties), -0 and +0 mixed (equal as
    fp32), one row of all-equal scores (the exact fallback), and garbage past
    the candidates (ignored)."""
    rng = np.random.default_rng(11)
    K, D, G = 32, 128, 4
    nblk = ops.nblk(kv_cap)
    C = (kv_len - 1) // 64
    R = (np.round(rng.standard_normal((B * Hkv, nblk)) * 4) / 4).astype(np.float32)
    zeros = R == 0
    R[zeros] = np.where(rng.random(np.count_nonzero(zeros)) < 0.5, np.float32(-0.0), np.float32(0.0))
    R[0, :] = 0.5
    ref = orc.select(np.where(np.arange(nblk) < C, R, -np.inf).astype(np.float64), np.full(B * Hkv, C), K)
    R[:, C:] = 1e30
    cfg = lib.make_cfg(B, Hkv * G, Hkv, D, top_k=K)
    note(f"decode selection: B{B} Hkv{Hkv} kv_len {kv_len} nblk {nblk}")
    q = torch.randn((B, Hkv * G, 1, D), device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, kv_cap, D), device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, kv_cap, D), device="cuda").to(torch.bfloat16)
    scores = torch.from_numpy(R).cuda()
    idx = torch.full((B, Hkv, 1, K), -7, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    nbytes = lib.infllmv2_decode_workspace_bytes(cfg, 1, kv_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lib.infllmv2_sparse_attn_decode_scores(cfg, q, k, v, kv_cap, kv_len, scores, idx, out, None, ws, nbytes)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().reshape(-1, K), ref)


def test_multi_token_decode_without_tree():
    run_decode(TREE_CASES["p1000_n7_d64"].scaled(name="mt_rows", seq_len=1020), tree=False)


def test_decode_128k_batch8_full_size():
    d, ref, res = run_decode(W["decode_128k_b8"])
    # planted blocks are the relevant ones: each (b, g) selects exactly its planted set
    assert np.array_equal(np.sort(ref["idx"][:, :, 0], axis=-1), np.sort(d["planted"], axis=-1))


def test_tree_128k_full_size():
    run_decode(W["tree_128k"])


# ---------------------------------------------------------------------------- dense
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dims", [(8, 2, 128, 700, 700), (4, 1, 64, 333, 1000), (16, 2, 64, 65, 4000),
                                  (8, 2, 128, 150, 1100), (4, 4, 128, 97, 513), (16, 1, 128, 40, 300)])
def test_dense_attention(causal, dims):
    Hq, Hkv, D, n_q, kv_len = dims
    w = P0.scaled(name="dense", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, seq_len=kv_len, n_plant=0)
    note(f"dense case Hq{Hq}/Hkv{Hkv} D{D} n_q{n_q} kv_len{kv_len} causal{causal}")
    d = synth.generate(w, seed=7)
    qn = np.ascontiguousarray(d["q"][:, :, kv_len - n_q:])
    ref = orc.dense_forward(qn, d["k"], d["v"], kv_len=kv_len, n_kv_heads=Hkv, causal=causal)
    res = ops.dense(cfg_of(w), dev_bf16(qn), dev_bf16(d["k"]), dev_bf16(d["v"]), kv_len, causal=causal)
    torch.cuda.synchronize()
    r = ref["rows"]
    assert_close_rows(host_f64(res["out"])[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "dense out")
    assert np.abs(host_f64(res["lse"])[r[:, 0], r[:, 1], r[:, 2]] - ref["lse"]).max() <= LSE_ABS


def test_sparse_with_covering_k_equals_dense():
    """K at least the candidate count: the sparse path is dense causal attention."""
    w = P0.scaled(name="cover", n_q_heads=8, n_kv_heads=2, seq_len=900, top_k=16, dense_threshold=0)
    d = synth.generate(w, seed=9)
    cfg = cfg_of(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    sp = ops.sparse_prefill(cfg, q, k, v)
    de = ops.dense(cfg, q, k, v, d["kv_len"], causal=True)
    ref = orc.dense_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], n_kv_heads=2)
    torch.cuda.synchronize()
    r = ref["rows"]
    assert_close_rows(host_f64(sp["out"])[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "sparse (covering K)")
    assert_close_rows(host_f64(de["out"])[r[:, 0], r[:, 1], r[:, 2]], ref["out"], "dense")


def test_pool_incremental_blocks_match():
    w = D0.scaled(name="pool_inc", n_q_heads=8, n_kv_heads=2, seq_len=3000)
    d = synth.generate(w, seed=2)
    kbar_o = orc.pool(d["k"], 3000)
    cfg = cfg_of(w)
    k = dev_bf16(d["k"])
    kbar = ops.pool_kernels(cfg, k, d["kv_cap"], 1000)             # blocks 0..14
    lib.infllmv2_pool_kernels(cfg, k, d["kv_cap"], 3000, 15, kbar)   # extend to 46 blocks
    torch.cuda.synchronize()
    assert np.array_equal(kbar_rows(kbar)[:, :, :46], kbar_o[:, :, :46])


def test_decode_workspace_reused_across_shapes():
    """Consecutive decode calls share one workspace (arrival counters must come back to zero)."""
    ws = ops.Workspace(torch.device("cuda"))
    for i, (B, Hkv, L) in enumerate([(1, 2, 3000), (2, 4, 5000), (1, 2, 3000), (3, 4, 4100)]):
        w = D0.scaled(name=f"ws{i}", batch=B, n_q_heads=4 * Hkv, n_kv_heads=Hkv, seq_len=L, top_k=8, n_plant=8)
        note(f"workspace reuse call {i}: B{B} Hkv{Hkv} kv_len{L}")
        d = synth.generate(w, seed=20 + i)
        kbar_o, _, _ = open_gaps(d, orc)
        ref = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=L, q_pos0=L - 1, n_kv_heads=Hkv, top_k=8,
                                 dense_threshold=w.dense_threshold, kbar=kbar_o)
        cfg = cfg_of(w)
        k = dev_bf16(d["k"])
        kbar = ops.pool_kernels(cfg, k, d["kv_cap"], L)
        res = ops.decode(cfg, dev_bf16(d["q"]), k, dev_bf16(d["v"]), kbar, L, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(res["idx"].cpu().numpy(), ref["idx"])
        hr = ref["head_rows"]
        assert_close_rows(host_f64(res["out"])[hr[:, 0], hr[:, 1], hr[:, 2]], ref["out"], f"call {i}")
