"""Workload descriptors for InfLLM v2 block-sparse attention.

Five synthetic workloads, named by what they are. Shapes follow the
MiniCPM4 pages' setting (an 8B-class model with 32 query heads sharing
8 KV heads, head_dim 128, 32K-128K contexts; MiniCPM4 report summary
(QbitAI), sections "Core performance: efficiency evaluation" and
"Long-context evaluation") plus one tiny prefill case that a CPU oracle
finishes in well under a second.

This module holds shapes only: no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

BLOCK = 64        # tokens per context block
KWIN = 32         # semantic-kernel window (tokens)
KSTRIDE = 16      # semantic-kernel stride (tokens)


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str               # "prefill" | "decode" | "tree"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int            # prefill: tokens T; decode: kv_len; tree: prefix P
    top_k: int
    dense_threshold: int
    n_plant: int            # planted relevant blocks per (batch, KV head)
    n_tree: int = 0         # tree: draft nodes
    tree_depth: int = 0     # tree: exact depth (root = depth 1)
    block_size: int = BLOCK
    kernel_size: int = KWIN
    kernel_stride: int = KSTRIDE

    # ---- derived shapes (bookkeeping only) ----
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_q(self) -> int:
        """Query rows per head in one call."""
        if self.mode == "prefill":
            return self.seq_len
        if self.mode == "decode":
            return 1
        return self.n_tree

    @property
    def kv_len(self) -> int:
        if self.mode == "tree":
            return self.seq_len + self.n_tree
        return self.seq_len

    @property
    def kv_cap(self) -> int:
        bs = self.block_size
        return (self.kv_len + bs - 1) // bs * bs

    @property
    def q_pos0(self) -> int:
        """Absolute position of query row 0 (tree: every node's prefix length P)."""
        if self.mode == "prefill":
            return 0
        if self.mode == "decode":
            return self.kv_len - 1
        return self.seq_len

    @property
    def n_cand_max(self) -> int:
        """Complete blocks strictly before the latest query's own block."""
        bs = self.block_size
        if self.mode == "prefill":
            return (self.seq_len - 1) // bs
        if self.mode == "decode":
            return (self.kv_len - 1) // bs
        return self.seq_len // bs

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # B1, 2 query heads on 1 KV head, D64, 2048 tokens, K=8, dense below 1024.
    "tiny_prefill_2k": Workload("tiny_prefill_2k", "prefill", 1, 2, 1, 64, 2048, 8, 1024, 4),
    # One new token against a 32K cache, GQA 4, K=16.
    "decode_32k": Workload("decode_32k", "decode", 1, 32, 8, 128, 32768, 16, 1024, 16),
    # Causal sparse prefill of 32K tokens, K=16 plus the own (diagonal) block.
    "prefill_32k": Workload("prefill_32k", "prefill", 1, 32, 8, 128, 32768, 16, 1024, 16),
    # Eight sequences, one new token each, against 128K caches, K=32.
    "decode_128k_b8": Workload("decode_128k_b8", "decode", 8, 32, 8, 128, 131072, 32, 1024, 32),
    # A 16-node draft tree of depth 4 after a 128K prefix, K=32 per node.
    "tree_128k": Workload("tree_128k", "tree", 1, 32, 8, 128, 131072, 32, 1024, 32,
                          n_tree=16, tree_depth=4),
}

ORDER = ["tiny_prefill_2k", "decode_32k", "prefill_32k", "decode_128k_b8", "tree_128k"]
