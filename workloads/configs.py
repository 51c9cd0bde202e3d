"""The synthetic group shapes the path is tested and measured on (five groups,
the next rows' workloads, and the headline group in fp32).

Shapes follow the workloads the PrefixFlow page trains on (flat GRPO groups
[P || S_i], PrefixFlow §2.1; long-prefix RAG groups, §5.2 Claim 2.1; the
large-N prefix-ratio sweep, §5.4 Claim 3) and the rollout trees of the HARTS
page (§2.1, compact representation; §3.4, sharing windows whose consumers
read a producer's cached ancestor K/V).  Inputs are synthetic N(0,1) draws;
no dataset item is reproduced.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str                 # "f32" or "bf16": the dtype of every Q/K/V/O/dO tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prefix_len: int            # P (0 for the tree config)
    # flat groups: suffix lengths (fixed) or a (lo, hi) range drawn per seed
    n_suffix: int = 0
    suffix_len: Optional[int] = None
    suffix_len_range: Optional[Tuple[int, int]] = None
    microbatches: int = 1      # Phase B calls; microbatch k takes suffixes in index order
    # tree config: fan-out per level and node length per level (root first)
    tree_levels: Optional[Tuple[Tuple[int, int], ...]] = None
    # tree windows over the prefix: windows, nodes per window, node length range
    windows: int = 0
    window_nodes: int = 0
    node_len_range: Optional[Tuple[int, int]] = None
    window_calls: int = 0      # calls the windows are run in (0: one per window)
    # windows under the deepest nodes of a producer tree (tree_levels) instead
    # of over a flat prefix: each window reads its node's and ancestors' rows
    under_producer: bool = False
    # compact log-probabilities: vocabulary of the compact-row logits (the
    # rows and positions are those of tree_levels)
    logprob_vocab: int = 0
    seed: int = 0
    note: str = ""

    @property
    def is_tree(self) -> bool:
        return self.tree_levels is not None and not self.under_producer

    @property
    def is_windows(self) -> bool:
        return self.windows > 0 and not self.under_producer

    @property
    def is_ranges(self) -> bool:
        return self.windows > 0 and self.under_producer

    @property
    def is_logprob(self) -> bool:
        return self.logprob_vocab > 0

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS: List[Config] = [
    Config(1, "tiny-f32", "f32", 2, 2, 64, 256, n_suffix=4, suffix_len=64, seed=1,
           note="parity only; fp32 end to end"),
    Config(2, "gqa-bf16-p4096-n8x512", "bf16", 32, 8, 128, 4096, n_suffix=8, suffix_len=512,
           seed=2, note="89% prefix ratio; one Phase-B call with all 8 suffixes"),
    Config(3, "rag-bf16-p16384-n16-varlen", "bf16", 32, 8, 128, 16384, n_suffix=16,
           suffix_len_range=(256, 2048), microbatches=4, seed=3,
           note="suffix lengths uniform on [256, 2048] inclusive; 4 calls of 4 suffixes"),
    Config(4, "sweep-bf16-p8192-n64x256", "bf16", 32, 8, 128, 8192, n_suffix=64, suffix_len=256,
           microbatches=8, seed=4,
           note="8 calls of 8 suffixes; the stated 83% prefix ratio does not match these "
                "shapes (P/(P+S) = 97%); the shapes rule"),
    Config(5, "tree-bf16-4096-4x1024-16x256", "bf16", 16, 4, 128, 0,
           tree_levels=((1, 4096), (4, 1024), (4, 256)), seed=5,
           note="DFS-preorder compact rows: root 4096, 4 children of 1024, 4 leaves of 256 each; "
                "12288 compact rows, 16 trajectories"),
    Config(6, "windows-bf16-p4096-4x24-irregular", "bf16", 32, 8, 128, 4096, windows=4,
           window_nodes=24, node_len_range=(32, 256), window_calls=1, seed=6,
           note="the next row after the five groups: 4 sharing windows over one cached 4096-row "
                "prefix, each an irregular tree of 24 nodes (each node's parent uniform over the "
                "earlier nodes, lengths uniform on [32, 256]); the 4 trees run as one call (a "
                "forest over the prefix)"),
    Config(8, "windows-under-tree-bf16-2048-4x1024-8x512", "bf16", 32, 8, 128, 0,
           tree_levels=((1, 2048), (4, 1024), (2, 512)), windows=8, window_nodes=24,
           node_len_range=(32, 256), under_producer=True, seed=8,
           note="per-node caches: a producer rollout tree (root 2048 rows, 4 children of 1024, "
                "each with 2 children of 512; 10240 compact rows) and 8 consumer windows, each an "
                "irregular tree of 24 nodes hung under one of the 8 depth-2 nodes and reading the "
                "3584 rows of that node and its ancestors in place; producer forward, the 8 "
                "windows forward and backward adding into the producer rows' gK/gV, then the "
                "producer backward with them injected"),
    Config(9, "gqa-f32-p4096-n8x512", "f32", 32, 8, 128, 4096, n_suffix=8, suffix_len=512,
           seed=9,
           note="the config-2 group with fp32 tensors end to end: the fp32 kernels (matrix-core "
                "products in fp32) at the headline shape; one Phase-B call with all 8 suffixes"),
    Config(7, "logprob-bf16-tree5-v151936", "bf16", 16, 4, 128, 0,
           tree_levels=((1, 4096), (4, 1024), (4, 256)), logprob_vocab=151936, seed=7,
           note="compact log-probabilities of the config-5 tree: 12288 compact rows of bf16 "
                "logits over a 151936-token vocabulary, 86016 trajectory positions mapped to "
                "their rows, targets uniform; logits drawn on the device from the seed"),
]


def get_config(cid: int) -> Config:
    for c in CONFIGS:
        if c.cid == cid:
            return c
    raise KeyError(f"no config {cid}")
