"""CPU oracle for prefix/suffix attention: TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy implementations of what the GPU path
computes, in fp64 by default.  Nothing here is blocked, fused or reordered
beyond the textbook definitions; nothing here is shared with the HIP path,
and the product never imports this package.  Only `tests/`,
`__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may use it.

Pins (checked by `tests/test_oracle_*.py`, none of which compares the oracle
with itself): finite differences, torch CPU fp64 autograd and SDPA (math
path), closed forms (Q = 0, single visible key), the full-trajectory row
identity, prefix-gradient superposition via a packed-graph formulation,
GQA = MHA with repeated K/V, tree expanded-vs-direct, the reductions of
trees to flat groups and causal chains, and tree windows over a prefix
against per-trajectory flat Phase B (expansion with a split upstream), a
chain tree as one flat suffix, and P = 0 as a plain tree; a window over a
producer tree's ancestor rows with the producer backward against direct
attention over the combined tree; compact
log-probabilities against torch log_softmax and autograd on the expanded
per-position logits, and scipy's logsumexp.

Sources (page titles and sections):
  * PrefixFlow: Training-Time KV Caching for Schedule-Level Prefix Reuse in
    LLM RL Training — §2.1 (flat groups), §3.1 (three-phase schedule),
    §3.3 (KV boundary, linearity), §4.1 (Phase-B mask and positions),
    §4.2 (packed suffix layout).
  * HARTS: A Prefix-Sharing Training System for Agentic RL with
    Hybrid-Attention Models — §2.1 (rollout trees, compact rows), §2.2
    (full attention reads ancestor K/V through a tree mask), §3 (gather
    backward sums into shared rows; producer / consumer sharing windows,
    consumer gradients accumulated before one producer backward), §3.5
    (compact log-probability recovery).
"""
from .attention import attention_backward, attention_forward, head_map
from .logprob import compact_logprob, row_logsumexp
from .masks import causal_mask, suffix_rows_mask, tree_ancestor_mask, tree_node_of_row
from .phases import (
    prefix_backward_inject,
    prefix_forward,
    suffix_attention,
    suffix_attention_full_rows,
    tree_attention_direct,
    tree_attention_expanded,
    tree_backward_inject,
    tree_trajectories,
    tree_window_attention,
    tree_window_attention_ranges,
)

__all__ = [
    "compact_logprob",
    "row_logsumexp",
    "attention_backward",
    "attention_forward",
    "head_map",
    "causal_mask",
    "suffix_rows_mask",
    "tree_ancestor_mask",
    "tree_node_of_row",
    "prefix_backward_inject",
    "prefix_forward",
    "suffix_attention",
    "suffix_attention_full_rows",
    "tree_attention_direct",
    "tree_attention_expanded",
    "tree_trajectories",
    "tree_window_attention",
    "tree_window_attention_ranges",
    "tree_backward_inject",
]
