"""The seeded input generator: determinism, distribution, planting, trees, gap opening."""
import numpy as np
import torch

import synth
from oracle.gaps import open_gaps, boundary_gaps

SMALL_DECODE = synth.WORKLOADS["decode_32k"].scaled(name="t_dec", n_q_heads=8, n_kv_heads=2, seq_len=4096,
                                                     top_k=8, n_plant=8)


def test_same_seed_same_bytes_and_seed_matters():
    a = synth.generate(SMALL_DECODE, seed=1)
    b = synth.generate(SMALL_DECODE, seed=1)
    c = synth.generate(SMALL_DECODE, seed=2)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), ref)


def test_values_are_standard_normal_and_tail_is_zero():
    w = SMALL_DECODE.scaled(name="t_dist", seq_len=4000)
    d = synth.generate(w, seed=3)
    for key in ("q", "v"):
        x = synth.bf16_to_f32(d[key][..., :4000, :] if key == "v" else d[key]).astype(np.float64)
        assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    assert d["kv_cap"] == 4032 and (d["k"][:, :, 4000:] == 0).all()


def test_planted_blocks_are_selected_in_decode():
    import oracle as orc
    d = synth.generate(SMALL_DECODE, seed=4)
    res = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=d["kv_len"], q_pos0=d["q_pos0"],
                             n_kv_heads=2, top_k=8, dense_threshold=1024, with_attention=False)
    for g in range(2):
        assert sorted(res["idx"][0, g, 0].tolist()) == sorted(d["planted"][0, g].tolist())


def test_tree_shape():
    w = synth.WORKLOADS["tree_128k"]
    for seed in range(5):
        parent, _ = synth.tree_parents(w, seed, 0)
        depth = [1] * len(parent)
        for i in range(1, len(parent)):
            assert 0 <= parent[i] < i
            depth[i] = depth[parent[i]] + 1
        assert max(depth) == 4 and len(parent) == 16
        mask = synth.tree_masks(parent)
        for i in range(16):
            anc = {i}
            j = i
            while parent[j] >= 0:
                j = parent[j]
                anc.add(j)
            assert {b for b in range(64) if (int(mask[i]) >> b) & 1} == anc


def test_open_gaps_redraws_only_failing_tokens():
    import oracle as orc
    w = synth.WORKLOADS["prefill_32k"].scaled(name="t_gap", n_q_heads=8, n_kv_heads=2, seq_len=2048,
                                              n_plant=4, top_k=4, head_dim=64)
    d = synth.generate(w, seed=5)
    q0 = d["q"].copy()
    kbar, redrawn, min_gap = open_gaps(d, orc, min_gap=0.05)
    changed = np.nonzero((d["q"] != q0).any(axis=-1).any(axis=1)[0])[0]
    assert redrawn >= len(changed) > 0
    R, Cn = orc.scores(d["q"], kbar, np.arange(2048), orc.all_group_rows(1, 2, 2048), 2)
    assert boundary_gaps(R, Cn, 4).min() > 0.05
