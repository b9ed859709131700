"""Pins for the oracle's attention backward (the gradients the trainable path
needs): fixed by an independent differentiation and by mathematics.

- torch autograd in fp64 over an explicit boolean mask built from the oracle's
  key sets (a different implementation of the same definition: softmax
  attention restricted to the attended keys);
- sum rule: each row's dL/ds sums to zero over its keys, so the dk of all
  rows sum to zero;
- q = 0: uniform weights, so dk = 0 and dv of a key = sum over the rows that
  attend it of dO / n_row;
- a row attending one key only has dq = 0 and dk = 0 (its softmax is constant).
"""
import math

import numpy as np
import pytest
import torch

import synth

W0 = synth.WORKLOADS["tiny_prefill_2k"]


def tiny(name, **kw):
    base = dict(name=name, n_q_heads=4, n_kv_heads=2, head_dim=16, seq_len=260, top_k=2,
                dense_threshold=100, n_plant=1)
    base.update(kw)
    return W0.scaled(**base)


def _case(orc, w, seed):
    d = synth.generate(w, seed=seed)
    T = w.seq_len
    res = orc.sparse_forward(d["q"], d["k"], d["v"], kv_len=T, q_pos0=0, n_kv_heads=w.n_kv_heads,
                             top_k=w.top_k, dense_threshold=w.dense_threshold, with_attention=False)
    rng = np.random.default_rng(seed + 100)
    dout = synth.to_bf16_bits(rng.standard_normal(d["q"].shape).astype(np.float32)).reshape(d["q"].shape)
    return d, res["idx"], dout


def _mask(orc, mode, B, Hkv, n_q, kv_len, pos, idx, K, thr, tree_mask=None):
    m = np.zeros((B, Hkv, n_q, kv_len), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(n_q):
                sel = None if idx is None else idx[b, g, i]
                tm = 0 if tree_mask is None else int(tree_mask[b, i])
                keys = orc.keyset(mode, int(pos[i]), kv_len, sel, K, thr, tm)
                m[b, g, i, keys] = True
    return m


def _torch_grads(q, k, v, dout, mask, G, scale):
    f = lambda a: torch.from_numpy(synth.bf16_to_f32(a).astype(np.float64))
    qt, kt, vt, gt = f(q).requires_grad_(), f(k).requires_grad_(), f(v).requires_grad_(), f(dout)
    kk = kt.repeat_interleave(G, dim=1)
    vv = vt.repeat_interleave(G, dim=1)
    mm = torch.from_numpy(mask).repeat_interleave(G, dim=1)
    n = mm.shape[-1]
    s = scale * qt @ kk[:, :, :n].transpose(-1, -2)
    s = s.masked_fill(~mm, -math.inf)
    o = torch.softmax(s, dim=-1) @ vv[:, :, :n]
    (o * gt).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("seed,thr", [(0, 100), (1, 0), (2, 300)])
def test_backward_matches_torch_autograd_sparse(orc, seed, thr):
    w = tiny("bwd_sparse", dense_threshold=thr)
    d, idx, dout = _case(orc, w, seed)
    T, G = w.seq_len, w.n_q_heads // w.n_kv_heads
    pos = orc.positions("prefill", T, 0)
    dq, dk, dv = orc.attend_backward(orc.MODE_SPARSE, d["q"], d["k"], d["v"], pos, T, w.n_kv_heads,
                                     dout, idx=idx, dense_threshold=thr)
    mask = _mask(orc, orc.MODE_SPARSE, w.batch, w.n_kv_heads, T, T, pos, idx, w.top_k, thr)
    tq, tk, tv = _torch_grads(d["q"], d["k"], d["v"], dout, mask, G, 1 / math.sqrt(w.head_dim))
    for a, b in ((dq, tq), (dk[:, :, :T], tk[:, :, :T]), (dv[:, :, :T], tv[:, :, :T])):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-10)


def test_backward_matches_torch_autograd_dense_and_tree(orc):
    w = tiny("bwd_dense", seq_len=150)
    d, idx, dout = _case(orc, w, 3)
    T, G = w.seq_len, w.n_q_heads // w.n_kv_heads
    pos = orc.positions("prefill", T, 0)
    dq, dk, dv = orc.attend_backward(orc.MODE_CAUSAL, d["q"], d["k"], d["v"], pos, T, w.n_kv_heads, dout)
    mask = _mask(orc, orc.MODE_CAUSAL, w.batch, w.n_kv_heads, T, T, pos, None, 0, 0)
    tq, tk, tv = _torch_grads(d["q"], d["k"], d["v"], dout, mask, G, 1 / math.sqrt(w.head_dim))
    assert np.allclose(dq, tq, rtol=1e-10, atol=1e-10)
    assert np.allclose(dk[:, :, :T], tk[:, :, :T], rtol=1e-10, atol=1e-10)
    assert np.allclose(dv[:, :, :T], tv[:, :, :T], rtol=1e-10, atol=1e-10)
    # a draft tree of 4 nodes after a 140-token prefix: nodes see the prefix and their ancestors
    n, P = 4, 140
    qn = np.ascontiguousarray(d["q"][:, :, :n])
    gn = np.ascontiguousarray(dout[:, :, :n])
    tm = np.array([[0b1, 0b11, 0b101, 0b1011]] * w.batch, dtype=np.uint64)
    posn = orc.positions("tree", n, P)
    dq, dk, dv = orc.attend_backward(orc.MODE_TREE, qn, d["k"], d["v"], posn, P + n, w.n_kv_heads, gn,
                                     idx=np.zeros((w.batch, w.n_kv_heads, n, 1), np.int32) - 1,
                                     dense_threshold=10 ** 6, tree_mask=tm)
    mask = _mask(orc, orc.MODE_TREE, w.batch, w.n_kv_heads, n, P + n, posn,
                 np.zeros((w.batch, w.n_kv_heads, n, 1), np.int32) - 1, 1, 10 ** 6, tm)
    tq, tk, tv = _torch_grads(qn, d["k"], d["v"], gn, mask, G, 1 / math.sqrt(w.head_dim))
    assert np.allclose(dq, tq, rtol=1e-10, atol=1e-10)
    assert np.allclose(dk[:, :, :P + n], tk[:, :, :P + n], rtol=1e-10, atol=1e-10)
    assert np.allclose(dv[:, :, :P + n], tv[:, :, :P + n], rtol=1e-10, atol=1e-10)


def test_backward_sum_rule_and_zero_query(orc):
    w = tiny("bwd_rules")
    d, idx, dout = _case(orc, w, 4)
    T = w.seq_len
    pos = orc.positions("prefill", T, 0)
    dq, dk, dv = orc.attend_backward(orc.MODE_SPARSE, d["q"], d["k"], d["v"], pos, T, w.n_kv_heads,
                                     dout, idx=idx, dense_threshold=w.dense_threshold)
    # sum over keys of dk: each row's dS sums to zero over its keys
    assert np.abs(dk.sum(axis=2)).max() <= 1e-9 * max(1.0, np.abs(dk).max())
    # q = 0: every row weighs its n keys 1/n
    q0 = np.zeros_like(d["q"])
    dq, dk, dv = orc.attend_backward(orc.MODE_SPARSE, q0, d["k"], d["v"], pos, T, w.n_kv_heads,
                                     dout, idx=idx, dense_threshold=w.dense_threshold)
    assert np.abs(dk).max() == 0.0
    G = w.n_q_heads // w.n_kv_heads
    g_f = synth.bf16_to_f32(dout).astype(np.float64)
    exp_dv = np.zeros_like(dv)
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            for i in range(T):
                keys = orc.keyset(orc.MODE_SPARSE, i, T, idx[b, h // G, i], w.top_k, w.dense_threshold)
                exp_dv[b, h // G, keys] += g_f[b, h, i] / len(keys)
    assert np.allclose(dv, exp_dv, rtol=1e-12, atol=1e-12)
    # the first row attends key 0 only: no gradient reaches q or k through it
    dq1, dk1, dv1 = orc.attend_backward(orc.MODE_CAUSAL, d["q"][:, :, :1], d["k"], d["v"],
                                        orc.positions("prefill", 1, 0), 1, w.n_kv_heads, dout[:, :, :1])
    assert np.abs(dq1).max() == 0.0 and np.abs(dk1).max() == 0.0


def test_backward_tolerance_covers_bf16_arithmetic(orc):
    """The GPU backward rounds dS to bf16 before its products and forms
    Delta = dO . O from the bf16 forward output. Replaying exactly those two
    roundings in fp64 on sampled rows must stay well inside the GPU test's
    bounds for dq (mean-abs <= 1e-2 mean|dq|, max-abs <= 2e-2 max|dq|)."""
    w = tiny("bwd_tol", n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=1100, top_k=4,
             dense_threshold=300, n_plant=2)
    d, idx, dout = _case(orc, w, 0)
    T, G = w.seq_len, 4
    f = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    bf = lambda x: synth.bf16_to_f32(synth.to_bf16_bits(x.astype(np.float32)).reshape(x.shape)).astype(np.float64)
    q, k, v, g = f(d["q"]), f(d["k"]), f(d["v"]), f(dout)
    sc = 1 / math.sqrt(128)
    ex, ap = [], []
    for h in range(8):
        for i in range(0, T, 11):
            keys = orc.keyset(orc.MODE_SPARSE, i, T, idx[0, h // G, i], w.top_k, w.dense_threshold)
            kk, vv = k[0, h // G, keys], v[0, h // G, keys]
            s = sc * kk @ q[0, h, i]
            p = np.exp(s - s.max())
            p /= p.sum()
            dp = vv @ g[0, h, i]
            ex.append(sc * (p * (dp - p @ dp)) @ kk)
            ap.append(sc * bf(p * (dp - bf(p @ vv) @ g[0, h, i])) @ kk)
    ex, ap = np.array(ex), np.array(ap)
    err = np.abs(ap - ex)
    assert err.mean() <= 0.6e-2 * np.abs(ex).mean()
    assert err.max() <= 1e-2 * np.abs(ex).max()
