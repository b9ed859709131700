"""Brute-force restatement of InfLLM v2 block-sparse attention, pure Python, tiny inputs only.

TEST INFRASTRUCTURE ONLY. Written separately from oracle.c (no shared code,
no numpy in the arithmetic) so that the two can pin each other:
  * kernels: exact mean with fractions.Fraction, then an exact
    round-half-to-even onto the bf16 grid;
  * scores: the literal definition, max over a block's kernels per head then
    sum over the group's heads, with correctly rounded sums (math.fsum);
  * selection: exhaustive search over every K-subset of candidates for the
    largest exact score sum (scores taken as fp32), smallest ascending
    index tuple on equal sums;
  * attention: the attended key set written out from its description, then
    softmax with math.exp.

Sources: MiniCPM4 technical-report summary (QbitAI repost), section "Model
architecture: InfLLM v2" items 1 and 2 (kernels, max relevance, GQA-shared
blocks) and the dense rule for short contexts; same summary, section on
fusing speculative sampling with long-context algorithms (tree mask).
"""
from __future__ import annotations

import itertools
import math
import struct
from fractions import Fraction


def bf16_value(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (h & 0xFFFF) << 16))[0]


def bf16_round(x: Fraction) -> int:
    """Exact round-half-to-even of a rational onto bf16; returns the bit pattern."""
    if x == 0:
        return 0
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * quantum
    if val >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        f = float(val)                      # exact: val is on the bf16 grid
        bits = struct.unpack("<I", struct.pack("<f", f))[0] >> 16
    return bits | (0x8000 if neg else 0)


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def kernels(k_rows, bs=64, ks=32, kst=16):
    """k_rows: list over tokens of lists of bf16 bits (one head). Returns {j: [[bits]*D]*kpb}."""
    D = len(k_rows[0])
    kpb = (bs - ks) // kst + 1
    out = {}
    for j in range(len(k_rows) // bs):
        blk = []
        for m in range(kpb):
            start = j * bs + m * kst
            blk.append([bf16_round(sum(Fraction(bf16_value(k_rows[t][e])) for t in range(start, start + ks))
                                   / ks) for e in range(D)])
        out[j] = blk
    return out


def block_score(q_heads, kbar_block):
    """q_heads: G lists of bf16 bits; kbar_block: kpb lists of bf16 bits."""
    total = []
    for qh in q_heads:
        best = max(math.fsum(bf16_value(a) * bf16_value(b) for a, b in zip(qh, kv)) for kv in kbar_block)
        total.append(best)
    return math.fsum(total)


def select(R, C, K):
    """Exhaustive top-K: largest exact sum of fp32 scores, then smallest ascending tuple."""
    if C <= K:
        return list(range(C)) + [-1] * (K - C)
    best, best_key = None, None
    for comb in itertools.combinations(range(C), K):       # ascending tuples, lexicographic order
        s = sum(Fraction(f32(R[j])) for j in comb)
        if best is None or s > best_key:
            best, best_key = comb, s
    return list(best)


def attended_keys(p, sel, dense_threshold, bs=64, tree_P=None, tree_mask=0):
    """Key positions a query row attends (see oracle.c section 4 for the rule's source)."""
    if tree_P is None:
        if dense_threshold > 0 and p + 1 < dense_threshold:
            return list(range(p + 1))
        keys = set()
        for j in sel:
            if j >= 0:
                keys.update(range(j * bs, j * bs + bs))
        keys.update(range((p // bs) * bs, p + 1))
        return sorted(keys)
    P = tree_P
    tree = [P + j for j in range(64) if (tree_mask >> j) & 1]
    if dense_threshold > 0 and P + len(tree) < dense_threshold:
        return list(range(P)) + tree
    keys = set()
    for j in sel:
        if j >= 0:
            keys.update(range(j * bs, j * bs + bs))
    keys.update(range((P // bs) * bs, P))
    return sorted(keys) + tree


def attention(q_bits, k_rows, v_rows, keys, scale):
    """softmax(scale * q.k) v over the listed keys; returns (out list, lse)."""
    q = [bf16_value(x) for x in q_bits]
    s = [scale * math.fsum(a * bf16_value(b) for a, b in zip(q, k_rows[t])) for t in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    D = len(q_bits)
    out = [math.fsum(w[n] * bf16_value(v_rows[t][e]) for n, t in enumerate(keys)) / l for e in range(D)]
    return out, m + math.log(l)
