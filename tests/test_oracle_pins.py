"""Pins for the CPU oracle: values fixed by the pages and by mathematics, not by the oracle.

Each check here would fail under a plausible slip in oracle.c (a dropped term,
a wrong sign or index, a transposed operand); tests/test_oracle_mutants.py
plants such slips and confirms it.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import brute

W0 = synth.WORKLOADS["tiny_prefill_2k"]


def tiny(name, **kw):
    base = dict(name=name, n_q_heads=4, n_kv_heads=2, head_dim=8, seq_len=320, top_k=2,
                dense_threshold=0, n_plant=1)
    base.update(kw)
    return W0.scaled(**base)


def bfbits(x) -> int:
    return int(synth.to_bf16_bits(np.float32(x))[0])


def rows_of(x):
    return [list(map(int, r)) for r in x]


# ---------------------------------------------------------------- bf16 rounding
GOLD_BF16 = [  # IEEE-754 binary16-brain format facts (8 significant bits, fp32 exponent range)
    (1.0, 0x3F80), (-2.5, 0xC020), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82),
    (1 + 2 ** -8 + 2 ** -30, 0x3F81), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
    (3 * 2.0 ** -134, 0x0002), (2.0 ** -126, 0x0080), ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80), (-0.0, 0x8000), (65280.0, 0x477F), (65408.0, 0x4780),
]


@pytest.mark.parametrize("x,bits", GOLD_BF16)
def test_bf16_round_known_values(orc, x, bits):
    assert orc.bf16_from_double(x) == bits
    if x != 0 or bits == 0:                      # a Fraction has no negative zero
        assert brute.bf16_round(Fraction(x)) == bits


def test_bf16_round_matches_torch_on_fp32(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([orc.bf16_from_double(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_matches_exact_rational_on_doubles(orc):
    rng = np.random.default_rng(2)
    for v in rng.standard_normal(2000) * 10.0:
        assert orc.bf16_from_double(float(v)) == brute.bf16_round(Fraction(float(v)))


# ---------------------------------------------------------------- kernels (pooling)
def test_pool_constant_window_gives_constant(orc):
    k = np.zeros((1, 1, 128, 4), dtype=np.uint16)
    vals = [0x3FC0, 0xBF80, 0x4049, 0x3E00]            # 1.5, -1, 3.140625, 0.125
    for e, h in enumerate(vals):
        k[0, 0, :, e] = h
    kbar = orc.pool(k, 128)
    assert kbar.shape == (1, 1, 2, 3, 4)
    assert (kbar == np.array(vals, dtype=np.uint16)).all()


def test_pool_ramp_closed_form(orc):
    # K[t, e] = (t + 2e) / 64, exact in bf16 for t + 2e < 256. Window starting at
    # s has mean (s + 15.5 + 2e) / 64, exact in bf16 while s + 15.5 + 2e < 128.
    T, D = 128, 4
    k = np.zeros((1, 1, T, D), dtype=np.uint16)
    for t in range(T):
        for e in range(D):
            k[0, 0, t, e] = bfbits((t + 2 * e) / 64.0)
    kbar = orc.pool(k, T)
    for j in range(2):
        for m in range(3):
            s = 64 * j + 16 * m
            for e in range(D):
                assert synth.bf16_to_f32(kbar[0, 0, j, m, e]) == (s + 15.5 + 2 * e) / 64.0


def test_pool_only_complete_blocks(orc):
    k = np.full((1, 1, 192, 2), 0x3F80, dtype=np.uint16)
    kbar = orc.pool(k, 150)                              # blocks 0, 1 complete; block 2 not
    assert (kbar[0, 0, :2] == 0x3F80).all()
    assert (kbar[0, 0, 2] == 0).all()


def test_pool_matches_exact_brute(orc):
    w = tiny("pin_pool")
    d = synth.generate(w, seed=3)
    kbar = orc.pool(d["k"], d["kv_len"])
    for g in range(w.n_kv_heads):
        ref = brute.kernels(rows_of(d["k"][0, g, :d["kv_len"]]))
        for j, blk in ref.items():
            assert np.array_equal(kbar[0, g, j], np.array(blk, dtype=np.uint16))


# ---------------------------------------------------------------- block scores
def _one_hot_kbar(B, Hkv, nblk, D, vals):
    kbar = np.zeros((B, Hkv, nblk, 3, D), dtype=np.uint16)
    for (j, m), x in vals.items():
        kbar[0, 0, j, m, 0] = bfbits(x)
    return kbar


def test_scores_closed_form_max_then_sum(orc):
    # Two heads in one group, q_h = a_h * e0; kernel m of block j = b_jm * e0.
    # R(j) = sum_h max_m a_h * b_jm.
    a = [2.0, -1.0]
    b = {(0, 0): 1.0, (0, 1): 3.0, (0, 2): -2.0, (1, 0): 0.5, (1, 1): 0.25, (1, 2): -4.0}
    q = np.zeros((1, 2, 1, 4), dtype=np.uint16)
    for h in range(2):
        q[0, h, 0, 0] = bfbits(a[h])
    kbar = _one_hot_kbar(1, 1, 3, 4, b)
    R, Cn = orc.scores(q, kbar, np.array([150]), np.array([[0, 0, 0]]), n_kv_heads=1)
    assert Cn[0] == 2
    exp = [sum(max(a[h] * b[(j, m)] for m in range(3)) for h in range(2)) for j in range(2)]
    assert R[0, 0] == exp[0] and R[0, 1] == exp[1]      # 6 + 2 = 8; 1 + 4 = 5
    assert R[0, 2] == -math.inf


def test_scores_match_literal_brute(orc):
    w = tiny("pin_scores", seq_len=448)
    d = synth.generate(w, seed=4)
    kbar = orc.pool(d["k"], d["kv_len"])
    pos = np.arange(w.n_q)
    rows = np.array([(0, g, i) for g in range(w.n_kv_heads) for i in (0, 63, 64, 200, 447)])
    R, Cn = orc.scores(d["q"], kbar, pos, rows, w.n_kv_heads)
    G = w.group
    for r, (b, g, i) in enumerate(rows):
        assert Cn[r] == i // 64
        for j in range(Cn[r]):
            ref = brute.block_score(rows_of(d["q"][b, g * G:(g + 1) * G, i]), rows_of(kbar[b, g, j]))
            assert abs(R[r, j] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_scores_invariances(orc):
    w = tiny("pin_inv", seq_len=448)
    d = synth.generate(w, seed=5)
    kbar = orc.pool(d["k"], d["kv_len"])
    rows = np.array([(0, 1, 447)])
    R, _ = orc.scores(d["q"], kbar, np.arange(w.n_q), rows, w.n_kv_heads)
    q2 = d["q"].copy()
    q2[0, [2, 3]] = d["q"][0, [3, 2]]                     # swap the heads of group 1
    R2, _ = orc.scores(q2, kbar, np.arange(w.n_q), rows, w.n_kv_heads)
    assert np.allclose(R, R2, rtol=0, atol=1e-12)
    q3 = synth.to_bf16_bits(2.0 * synth.bf16_to_f32(d["q"]))   # exact doubling
    R3, _ = orc.scores(q3, kbar, np.arange(w.n_q), rows, w.n_kv_heads)
    fin = np.isfinite(R)
    assert np.array_equal(R3[fin], 2.0 * R[fin])


# ---------------------------------------------------------------- selection
def test_select_exhaustive_with_ties(orc):
    rng = np.random.default_rng(6)
    for trial in range(150):
        C = int(rng.integers(1, 11))
        K = int(rng.integers(1, 6))
        R = rng.integers(-3, 4, size=12).astype(np.float64)        # many exact ties
        R[C:] = -np.inf
        got = orc.select(R[None, :], np.array([C]), K)[0]
        assert list(got) == brute.select(list(R), C, K), (trial, R, C, K)


def test_select_matches_lexsort(orc):
    rng = np.random.default_rng(7)
    R = rng.standard_normal((50, 600))
    R[:, ::7] = R[:, 3:4]                                          # shared values -> ties
    Cn = rng.integers(0, 600, size=50)
    for r in range(50):
        R[r, Cn[r]:] = -np.inf
    idx = orc.select(R, Cn, 16)
    for r in range(50):
        c = Cn[r]
        if c <= 16:
            exp = list(range(c)) + [-1] * (16 - c)
        else:
            order = np.lexsort((np.arange(c), -R[r, :c].astype(np.float32)))
            exp = sorted(order[:16].tolist())
        assert list(idx[r]) == exp


def test_select_decides_in_fp32(orc):
    # Scores that differ only below fp32 resolution tie, and the lower index wins.
    R = np.array([[1.0 + 1e-12, 1.0, 0.5]])
    assert list(orc.select(R, np.array([3]), 1)[0]) == [0]
    R = np.array([[1.0, 1.0 + 1e-12, 0.5]])
    assert list(orc.select(R, np.array([3]), 1)[0]) == [0]


# ---------------------------------------------------------------- attended keys / attention
def test_keyset_rules(orc):
    sel = np.array([0, 2, -1], dtype=np.int32)
    ks = orc.keyset(orc.MODE_SPARSE, 200, 4096, sel, 3, 0)
    assert ks.tolist() == list(range(0, 64)) + list(range(128, 192)) + list(range(192, 201))
    ks = orc.keyset(orc.MODE_SPARSE, 200, 4096, sel, 3, 202)       # n_ctx 201 < 202: dense
    assert ks.tolist() == list(range(201))
    ks = orc.keyset(orc.MODE_SPARSE, 200, 4096, sel, 3, 201)       # n_ctx 201: sparse
    assert ks.tolist()[-1] == 200 and len(ks) == 64 * 2 + 9
    ks = orc.keyset(orc.MODE_TREE, 256, 4096, np.array([1], np.int32), 1, 0, mask=0b1011)
    assert ks.tolist() == list(range(64, 128)) + [256, 257, 259]
    ks = orc.keyset(orc.MODE_TREE, 300, 4096, np.array([1], np.int32), 1, 0, mask=0b1)
    assert ks.tolist() == list(range(64, 128)) + list(range(256, 300)) + [300]


def _sdpa_fp64(q, k, v, G, causal_pos):
    qf = torch.from_numpy(synth.bf16_to_f32(q).astype(np.float64))
    kf = torch.from_numpy(synth.bf16_to_f32(k).astype(np.float64)).repeat_interleave(G, dim=1)
    vf = torch.from_numpy(synth.bf16_to_f32(v).astype(np.float64)).repeat_interleave(G, dim=1)
    T = kf.shape[2]
    allowed = torch.arange(T)[None, :] <= torch.from_numpy(causal_pos)[:, None]
    return torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, attn_mask=allowed).numpy()


def test_dense_matches_torch_sdpa_fp64(orc):
    w = tiny("pin_dense", seq_len=300)
    d = synth.generate(w, seed=8)
    # bottom-right aligned: the last 40 of 300 keys' positions carry queries
    q = d["q"][:, :, -40:]
    res = orc.dense_forward(q, d["k"], d["v"], kv_len=300, n_kv_heads=w.n_kv_heads)
    ref = _sdpa_fp64(q, d["k"][:, :, :300], d["v"][:, :, :300], w.group, np.arange(260, 300))
    assert np.allclose(res["out"].reshape(ref.shape), ref, rtol=0, atol=1e-12)


def test_topk_covering_all_blocks_equals_dense_causal(orc):
    w = tiny("pin_cover", seq_len=640, top_k=16)          # at most 9 candidates < K
    d = synth.generate(w, seed=9)
    sp = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=640, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=16, dense_threshold=0)
    de = orc.dense_forward(d["q"], d["k"], d["v"], kv_len=640, n_kv_heads=w.n_kv_heads,
                           rows=sp["head_rows"])
    assert np.array_equal(sp["nkeys"], de["nkeys"])
    assert np.allclose(sp["out"], de["out"], rtol=0, atol=1e-12)
    ref = _sdpa_fp64(d["q"], d["k"], d["v"], w.group, np.arange(640))
    hr = sp["head_rows"]
    assert np.allclose(sp["out"], ref[hr[:, 0], hr[:, 1], hr[:, 2]], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- the pages' figures
def test_attended_fraction_matches_the_pages_bound(orc):
    """tests/golden/page_claims.json: at the pages' context lengths (32K pretraining window,
    128K evaluation) a long-context row attends fewer than 5% of the keys before it, under the
    top-K settings of the measured workloads (K = 16 at 32K, K = 32 at 128K)."""
    import json, os
    claims = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_claims.json")))
    bound = claims["attended_fraction_below"]["value"]
    for L, K in [(claims["pretrain_context"]["value"], 16), (claims["eval_context"]["value"], 32)]:
        p = L - 1
        sel = np.arange(K, dtype=np.int32) * ((p // 64) // K)          # any K distinct candidates
        keys = orc.keyset(orc.MODE_SPARSE, p, L, sel, K, 1024)
        assert len(keys) == K * 64 + p % 64 + 1
        assert len(keys) / (p + 1) < bound, (L, K, len(keys))


# ---------------------------------------------------------------- LSE-normalized scores
def _onehot_case(G):
    """One group of G heads, D = 8, a row at position 130 (candidates: blocks 0 and 1).
    Block 0's kernels: e0, 0, 0; block 1's: 0, 0, 0. Head 0's query is e0, the others 0."""
    D, nblk = 8, 3
    kbar = np.zeros((1, 1, nblk, 3, D), np.uint16)
    kbar[0, 0, 0, 0, 0] = bfbits(1.0)
    q = np.zeros((1, G, 1, D), np.uint16)
    q[0, 0, 0, 0] = bfbits(1.0)
    return q, kbar, np.array([130]), np.array([[0, 0, 0]], np.int32)


def test_lse_scores_hand_example(orc):
    # scale ln 2: head 0's kernel scores are ln2, 0, 0 | 0, 0, 0, so exp gives 2,1,1 | 1,1,1
    # (sum 7): blocks get 2/7 and 1/7; every zero query sees six equal kernels: 1/6 each
    q, kbar, pos, rows = _onehot_case(1)
    R, C = orc.scores_lse(q, kbar, pos, rows, 1, scale=math.log(2.0))
    assert C.tolist() == [2] and np.isneginf(R[0, 2])
    assert np.allclose(R[0, :2], [2 / 7, 1 / 7], rtol=1e-14, atol=0)
    q, kbar, pos, rows = _onehot_case(2)
    R, _ = orc.scores_lse(q, kbar, pos, rows, 1, scale=math.log(2.0))
    assert np.allclose(R[0, :2], [2 / 7 + 1 / 6, 1 / 7 + 1 / 6], rtol=1e-14, atol=0)


def test_lse_scores_zero_query_closed_form(orc):
    w = tiny("pin_lse0", seq_len=640)
    d = synth.generate(w, seed=31)
    kbar = orc.pool(d["k"], 640)
    q = np.zeros_like(d["q"])
    pos = np.arange(640)
    rows = orc.all_group_rows(1, w.n_kv_heads, 640)
    R, C = orc.scores_lse(q, kbar, pos, rows, w.n_kv_heads)
    for r in range(0, len(rows), 37):                 # all 3C kernels tie: each block gets G / (3C)
        c = int(C[r])
        if c:
            assert np.allclose(R[r, :c], w.group / (3 * c), rtol=1e-13, atol=0)
        assert np.isneginf(R[r, c:]).all()


def _selection_gap_ok(R, C, K):
    """Rows whose K-th and (K+1)-th raw scores differ clearly (no fp32 near-ties)."""
    ok = []
    for r, c in enumerate(C):
        if c <= K:
            ok.append(True)
            continue
        srt = np.sort(R[r, :c])[::-1]
        ok.append(srt[K - 1] - srt[K] > 1e-6 * max(1.0, abs(srt[K])))
    return np.array(ok)


def test_lse_selection_equals_raw_with_one_head_per_group(orc):
    _lse_selection_equals_raw(orc, identical_heads=False)


def test_lse_selection_equals_raw_with_identical_heads(orc):
    _lse_selection_equals_raw(orc, identical_heads=True)


def _lse_selection_equals_raw(orc, identical_heads):
    """One head per group (or identical heads): R_lse = G exp(max_m s - LSE) is an increasing
    function of the raw score, so both select the same blocks."""
    if identical_heads:
        w = tiny("pin_lse_same", n_q_heads=4, n_kv_heads=1, seq_len=900, top_k=3)
    else:
        w = tiny("pin_lse_g1", n_q_heads=2, n_kv_heads=2, seq_len=900, top_k=3)
    d = synth.generate(w, seed=32)
    q = d["q"].copy()
    if identical_heads:
        q[:, 1:] = q[:, :1]
    kbar = orc.pool(d["k"], 900)
    pos = np.arange(900)
    rows = orc.all_group_rows(1, w.n_kv_heads, 900)
    Rr, C = orc.scores(q, kbar, pos, rows, w.n_kv_heads)
    Rl, C2 = orc.scores_lse(q, kbar, pos, rows, w.n_kv_heads)
    assert np.array_equal(C, C2)
    ok = _selection_gap_ok(Rr, C, w.top_k)
    assert ok.mean() > 0.9
    assert np.array_equal(orc.select(Rr, C, w.top_k)[ok], orc.select(Rl, C, w.top_k)[ok])


# ---------------------------------------------------------------- sliding window (draft model)
def test_window_keyset_rules(orc):
    assert orc.keyset(orc.MODE_WINDOW, 5, 100, None, 0, 0, window=3).tolist() == [3, 4, 5]
    assert orc.keyset(orc.MODE_WINDOW, 1, 100, None, 0, 0, window=5).tolist() == [0, 1]
    assert orc.keyset(orc.MODE_WINDOW, 70, 100, None, 0, 0, window=1).tolist() == [70]
    assert orc.keyset(orc.MODE_WINDOW, 99, 100, None, 0, 0, window=64).tolist() == list(range(36, 100))
    with pytest.raises(ValueError):
        orc.keyset(orc.MODE_WINDOW, 5, 100, None, 0, 0, window=0)


def test_window_matches_torch_sdpa_band_mask_fp64(orc):
    w = tiny("pin_window", seq_len=300)
    d = synth.generate(w, seed=21)
    W = 37
    q = d["q"][:, :, -90:]                                 # positions 210..299
    res = orc.window_forward(q, d["k"], d["v"], kv_len=300, n_kv_heads=w.n_kv_heads, window=W)
    G = w.group
    qf = torch.from_numpy(synth.bf16_to_f32(q).astype(np.float64))
    kf = torch.from_numpy(synth.bf16_to_f32(d["k"][:, :, :300]).astype(np.float64)).repeat_interleave(G, 1)
    vf = torch.from_numpy(synth.bf16_to_f32(d["v"][:, :, :300]).astype(np.float64)).repeat_interleave(G, 1)
    key = torch.arange(300)[None, :]
    pos = torch.arange(210, 300)[:, None]
    band = (key <= pos) & (key > pos - W)
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, attn_mask=band).numpy()
    assert np.allclose(res["out"].reshape(ref.shape), ref, rtol=0, atol=1e-12)
    assert set(res["nkeys"].tolist()) == {W}


def test_window_of_one_returns_own_value(orc):
    w = tiny("pin_window1", seq_len=200)
    d = synth.generate(w, seed=22)
    res = orc.window_forward(d["q"], d["k"], d["v"], kv_len=200, n_kv_heads=w.n_kv_heads, window=1)
    G = w.group
    for (b, h, i), o, l in zip(res["rows"], res["out"], res["lse"]):
        vv = synth.bf16_to_f32(d["v"][b, h // G, i]).astype(np.float64)
        assert np.array_equal(o, vv)                        # softmax over one key is exactly 1
        qk = float(np.dot(synth.bf16_to_f32(d["q"][b, h, i]).astype(np.float64),
                          synth.bf16_to_f32(d["k"][b, h // G, i]).astype(np.float64)))
        assert math.isclose(l, qk / math.sqrt(w.head_dim), rel_tol=0, abs_tol=1e-12)


def test_window_covering_the_prefix_equals_dense_causal(orc):
    w = tiny("pin_window_all", seq_len=260)
    d = synth.generate(w, seed=23)
    wi = orc.window_forward(d["q"], d["k"], d["v"], kv_len=260, n_kv_heads=w.n_kv_heads, window=260)
    de = orc.dense_forward(d["q"], d["k"], d["v"], kv_len=260, n_kv_heads=w.n_kv_heads)
    assert np.array_equal(wi["nkeys"], de["nkeys"])
    assert np.allclose(wi["out"], de["out"], rtol=0, atol=0)


def test_threshold_above_every_row_equals_dense(orc):
    w = tiny("pin_thr", seq_len=400)
    d = synth.generate(w, seed=10)
    sp = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=400, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=401)
    de = orc.dense_forward(d["q"], d["k"], d["v"], kv_len=400, n_kv_heads=w.n_kv_heads,
                           rows=sp["head_rows"])
    assert np.allclose(sp["out"], de["out"], rtol=0, atol=1e-12)


def test_threshold_boundary_rows(orc):
    w = tiny("pin_thr2", seq_len=400)
    d = synth.generate(w, seed=11)
    thr = 300
    sp = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=400, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=thr)
    nk = dict(((b, h, i), n) for (b, h, i), n in zip(map(tuple, sp["head_rows"]), sp["nkeys"]))
    assert nk[(0, 0, thr - 2)] == thr - 1                       # n_ctx = thr-1 < thr: dense
    assert nk[(0, 0, thr - 1)] == 2 * 64 + (thr - 1) % 64 + 1   # n_ctx = thr: sparse


def test_constant_v_and_zero_q(orc):
    w = tiny("pin_const", seq_len=320)
    d = synth.generate(w, seed=12)
    v = np.zeros_like(d["v"])
    v[..., :] = synth.to_bf16_bits(np.linspace(-1, 1, w.head_dim, dtype=np.float32))
    sp = orc.sparse_forward(d["q"], d["k"], v, kv_len=320, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0)
    assert np.allclose(sp["out"], synth.bf16_to_f32(v[0, 0, 0])[None, :], rtol=0, atol=1e-12)
    # Q = 0: uniform weights -> plain mean of the attended V rows, and lse = log(n)
    q0 = np.zeros_like(d["q"])
    sp0 = orc.sparse_forward(q0, d["k"], d["v"], kv_len=320, q_pos0=0, n_kv_heads=w.n_kv_heads,
                             top_k=2, dense_threshold=0, kbar=sp["kbar"])
    vf = synth.bf16_to_f32(d["v"]).astype(np.float64)
    G = w.group
    for r, (b, h, i) in enumerate(sp0["head_rows"][::37]):
        r = r * 37
        keys = orc.keyset(orc.MODE_SPARSE, int(i), 320, sp0["idx"][b, h // G, i], 2, 0)
        assert np.allclose(sp0["out"][r], vf[b, h // G, keys].mean(0), rtol=0, atol=1e-12)
        assert abs(sp0["lse"][r] - math.log(len(keys))) < 1e-12


def test_one_hot_v_recovers_support_and_gqa_sharing(orc):
    # T <= D: V[t] = e_t, so out[e] is the softmax weight of key e: its support
    # is the attended key set, the same for every head of a group.
    w = tiny("pin_onehot", seq_len=256, head_dim=256, top_k=1)
    d = synth.generate(w, seed=13)
    v = np.zeros_like(d["v"])
    for t in range(256):
        v[:, :, t, t] = 0x3F80
    sp = orc.sparse_forward(d["q"], d["k"], v, kv_len=256, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=1, dense_threshold=0)
    G = w.group
    supp = {}
    for r, (b, h, i) in enumerate(sp["head_rows"]):
        s = tuple(np.nonzero(sp["out"][r] > 0)[0].tolist())
        ref = brute.attended_keys(int(i), sp["idx"][b, h // G, i].tolist(), 0)
        assert list(s) == ref
        supp.setdefault((b, h // G, i), set()).add(s)
    assert all(len(x) == 1 for x in supp.values())


def test_end_to_end_matches_brute(orc):
    w = tiny("pin_e2e", seq_len=384, dense_threshold=150, top_k=2)
    d = synth.generate(w, seed=14)
    sp = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=384, q_pos0=0, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=150)
    G, D = w.group, w.head_dim
    kb = {g: brute.kernels(rows_of(d["k"][0, g, :384])) for g in range(w.n_kv_heads)}
    for r, (b, h, i) in enumerate(sp["head_rows"]):
        if i % 23 and i not in (148, 149, 383):
            continue
        g = h // G
        C = i // 64
        R = [brute.block_score(rows_of(d["q"][0, g * G:(g + 1) * G, i]), kb[g][j]) for j in range(C)]
        sel = brute.select(R, C, 2)
        assert sp["idx"][b, g, i].tolist() == sel
        keys = brute.attended_keys(int(i), sel, 150)
        out, lse = brute.attention(d["q"][b, h, i].tolist(), rows_of(d["k"][b, g]),
                                   rows_of(d["v"][b, g]), keys, 1 / math.sqrt(D))
        assert np.allclose(sp["out"][r], out, rtol=0, atol=1e-12)
        assert abs(sp["lse"][r] - lse) < 1e-12


# ---------------------------------------------------------------- tree verification
def _tree_case(orc, mask, n_tree, seed, P=256, tree_name="pin_tree"):
    w = tiny(tree_name, seq_len=P).scaled(mode="tree", n_tree=n_tree, tree_depth=2)
    d = synth.generate(w, seed=seed)
    return w, d


def test_single_node_tree_equals_decode(orc):
    w, d = _tree_case(orc, None, 1, 15, P=300)
    P = 300
    mask = np.array([[1]], dtype=np.uint64)
    tr = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=P + 1, q_pos0=P, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0, tree_mask=mask)
    de = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=P + 1, q_pos0=P, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0)
    assert np.array_equal(tr["idx"], de["idx"])
    assert np.array_equal(tr["nkeys"], de["nkeys"])
    assert np.allclose(tr["out"], de["out"], rtol=0, atol=1e-12)


def test_chain_tree_equals_prefill_continuation(orc):
    n = 8
    w, d = _tree_case(orc, None, n, 16, P=256)
    P = 256
    mask = np.array([[(1 << (i + 1)) - 1 for i in range(n)]], dtype=np.uint64)
    tr = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=P + n, q_pos0=P, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0, tree_mask=mask)
    pf = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=P + n, q_pos0=P, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0)         # rows at positions P + i
    assert np.array_equal(tr["idx"], pf["idx"])
    assert np.allclose(tr["out"], pf["out"], rtol=0, atol=1e-12)


def test_star_tree_sees_root_and_self(orc):
    n = 5
    w, d = _tree_case(orc, None, n, 17, P=256)
    mask = np.array([[1] + [1 | (1 << i) for i in range(1, n)]], dtype=np.uint64)
    tr = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=256 + n, q_pos0=256,
                            n_kv_heads=w.n_kv_heads, top_k=2, dense_threshold=0, tree_mask=mask)
    G = w.group
    for r, (b, h, i) in enumerate(tr["head_rows"]):
        ks = orc.keyset(orc.MODE_TREE, 256, 256 + n, tr["idx"][b, h // G, i], 2, 0, mask=int(mask[0, i]))
        assert ks[-(1 if i == 0 else 2):].tolist() == ([256] if i == 0 else [256, 256 + i])
        assert tr["nkeys"][r] == 2 * 64 + (1 if i == 0 else 2)


def test_tree_brute(orc):
    n = 6
    w, d = _tree_case(orc, None, n, 18, P=330)
    P = 330
    parent = [-1, 0, 0, 1, 3, 2]
    mask = synth.tree_masks(np.array(parent))[None, :]
    tr = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=P + n, q_pos0=P, n_kv_heads=w.n_kv_heads,
                            top_k=2, dense_threshold=0, tree_mask=mask)
    G, D = w.group, w.head_dim
    kb = {g: brute.kernels(rows_of(d["k"][0, g, :P + n])) for g in range(w.n_kv_heads)}
    for r, (b, h, i) in enumerate(tr["head_rows"]):
        g = h // G
        C = P // 64
        R = [brute.block_score(rows_of(d["q"][0, g * G:(g + 1) * G, i]), kb[g][j]) for j in range(C)]
        sel = brute.select(R, C, 2)
        assert tr["idx"][b, g, i].tolist() == sel
        keys = brute.attended_keys(None, sel, 0, tree_P=P, tree_mask=int(mask[0, i]))
        out, lse = brute.attention(d["q"][b, h, i].tolist(), rows_of(d["k"][b, g]),
                                   rows_of(d["v"][b, g]), keys, 1 / math.sqrt(D))
        assert np.allclose(tr["out"][r], out, rtol=0, atol=1e-12)
        assert abs(tr["lse"][r] - lse) < 1e-12
