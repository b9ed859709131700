"""Seeded synthetic inputs for InfLLM v2 block-sparse attention.

Both the CPU oracle and the HIP library are fed from here; this module
holds none of the method's arithmetic (no pooling, scoring, selection or
attention). It only draws numbers and lays them out.

Recipe (every element of Q, K and V is an N(0,1) draw rounded to bf16):
  * streams: each slice comes from its own counter-based Philox stream,
    keyed by (seed, workload id, tag, indices...), so any slice can be
    re-drawn without touching the others;
  * Q[b,h,i,:] = bf16((z[b,h,i,:] + c[b,g,:]) / sqrt(2)), z and c ~ N(0,I),
    c shared by all heads h of KV group g = h // G and by all tokens.
    Each element stays N(0,1); the shared part gives the group's queries a
    common direction, so blocks planted along it are relevant to every
    query of the group (the pages' selection has something to find);
  * K, V[b,g,t,:] ~ N(0,I) for t < kv_len, zero in the capacity tail;
  * planting: for n_plant distinct candidate blocks j per (b, g), chosen
    uniformly, every key row of block j becomes bf16(K + 3 * m_g), where
    m_g is the mean of group g's bf16 query rows (all heads, all tokens);
  * tree: node 0 is the root (depth 1); node i picks its parent uniformly
    among earlier nodes of depth < depth_max; the draw repeats (next
    attempt) until some node reaches depth_max. mask[i] = mask[parent] |
    (1 << i): bit j set means node i may attend tree slot j.
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import Workload

TAG_Q, TAG_K, TAG_V, TAG_PLANT, TAG_TREE, TAG_QFIX, TAG_SHARED = 1, 2, 3, 4, 5, 6, 7

_INV_SQRT2 = np.float32(1.0 / np.sqrt(2.0))


def workload_id(w: Workload) -> int:
    return zlib.crc32(w.name.encode()) & 0x7FFFFFFF


def stream(seed: int, wid: int, tag: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, wid, tag, *idx])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def shared_dir(w: Workload, seed: int, b: int, g: int) -> np.ndarray:
    return _normal(stream(seed, workload_id(w), TAG_SHARED, b, g), (w.head_dim,))


def _q_rows(z: np.ndarray, c: np.ndarray) -> np.ndarray:
    return to_bf16_bits((z + c) * _INV_SQRT2)


def redraw_q_token(w: Workload, seed: int, b: int, g: int, i: int, attempt: int) -> np.ndarray:
    """Fresh query rows [G, D] for token i of group g (used to open score gaps)."""
    z = _normal(stream(seed, workload_id(w), TAG_QFIX, b, g, i, attempt), (w.group, w.head_dim))
    return _q_rows(z, shared_dir(w, seed, b, g)[None, :])


def tree_parents(w: Workload, seed: int, b: int) -> tuple[np.ndarray, int]:
    n, dmax = w.n_tree, w.tree_depth
    for attempt in range(1000):
        rng = stream(seed, workload_id(w), TAG_TREE, b, attempt)
        parent = np.full(n, -1, dtype=np.int32)
        depth = np.ones(n, dtype=np.int32)
        for i in range(1, n):
            elig = [j for j in range(i) if depth[j] < dmax]
            p = elig[int(rng.integers(len(elig)))]
            parent[i] = p
            depth[i] = depth[p] + 1
        if depth.max() == dmax or n == 1:
            return parent, attempt
    raise RuntimeError("tree draw did not reach the requested depth")


def tree_masks(parent: np.ndarray) -> np.ndarray:
    mask = np.zeros(len(parent), dtype=np.uint64)
    for i, p in enumerate(parent):
        mask[i] = (mask[p] if p >= 0 else np.uint64(0)) | np.uint64(1 << i)
    return mask


def generate(w: Workload, seed: int = 0, threads: int = 8) -> dict:
    """Draw one input set for workload w. Arrays hold bf16 bit patterns (uint16)."""
    assert w.n_q_heads % w.n_kv_heads == 0
    wid = workload_id(w)
    B, Hq, Hkv, D, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    nq, kv_len, kv_cap = w.n_q, w.kv_len, w.kv_cap

    q = np.empty((B, Hq, nq, D), dtype=np.uint16)
    k = np.zeros((B, Hkv, kv_cap, D), dtype=np.uint16)
    v = np.zeros((B, Hkv, kv_cap, D), dtype=np.uint16)
    c = np.stack([np.stack([shared_dir(w, seed, b, g) for g in range(Hkv)]) for b in range(B)])

    def fill_q(bh):
        b, h = bh
        z = _normal(stream(seed, wid, TAG_Q, b, h), (nq, D))
        q[b, h] = _q_rows(z, c[b, h // G][None, :])

    def fill_kv(job):
        arr, tag, b, g = job
        arr[b, g, :kv_len] = to_bf16_bits(_normal(stream(seed, wid, tag, b, g), (kv_len, D)))

    jobs_kv = [(k, TAG_K, b, g) for b in range(B) for g in range(Hkv)] + \
              [(v, TAG_V, b, g) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill_q, [(b, h) for b in range(B) for h in range(Hq)]))
        list(ex.map(fill_kv, jobs_kv))

    n_cand = w.n_cand_max
    n_plant = min(w.n_plant, n_cand)
    planted = np.zeros((B, Hkv, n_plant), dtype=np.int32)
    qmean = np.zeros((B, Hkv, D), dtype=np.float32)
    bs = w.block_size

    def plant(bg):
        b, g = bg
        rows = bf16_to_f32(q[b, g * G:(g + 1) * G]).reshape(-1, D)
        m = rows.astype(np.float64).mean(axis=0).astype(np.float32)
        qmean[b, g] = m
        js = np.sort(stream(seed, wid, TAG_PLANT, b, g).choice(n_cand, n_plant, replace=False))
        planted[b, g] = js
        shift = np.float32(3.0) * m
        for j in js:
            blk = k[b, g, j * bs:(j + 1) * bs]
            k[b, g, j * bs:(j + 1) * bs] = to_bf16_bits(bf16_to_f32(blk) + shift[None, :])

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(plant, [(b, g) for b in range(B) for g in range(Hkv)]))

    out = dict(workload=w, seed=seed, q=q, k=k, v=v, planted=planted, qmean=qmean,
               kv_len=kv_len, kv_cap=kv_cap, q_pos0=w.q_pos0, n_q=nq)
    if w.mode == "tree":
        parents, masks, attempts = [], [], []
        for b in range(B):
            p, a = tree_parents(w, seed, b)
            parents.append(p)
            masks.append(tree_masks(p))
            attempts.append(a)
        out["parent"] = np.stack(parents)
        out["tree_mask"] = np.stack(masks)
        out["tree_attempts"] = attempts
    return out
