"""Seeded input generation for the synthetic groups.

Every tensor is drawn as fp32 N(0,1) from numpy's PCG64 generator seeded with
the config number, then (for bf16 configs) rounded to bf16 with
round-to-nearest-even.  The rounded bits are what both sides consume: the GPU
gets the bf16 bits, the oracle gets the same values widened exactly.

Draw order: varlen suffix lengths first (if any), then Q_P, K_P, V_P, dO_P,
Q_S, K_S, V_S, dO_S.  Tree configs draw Q, K, V, dO over the compact rows.
"""
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import Config


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of x after storage in `dtype` ("f32" or "bf16"), as fp32."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x))
    raise ValueError(dtype)


def tree_layout(levels: Sequence[Sequence[int]]):
    """DFS-preorder node table for a complete tree.

    levels[i] = (fan_out, node_len): the root level has fan_out 1.  Returns
    (node_off[n+1], parent[n]) with nodes numbered in preorder: a node's own
    rows come first, then its subtrees left to right.
    """
    node_len: List[int] = []
    parent: List[int] = []

    def visit(depth: int, par: int):
        idx = len(node_len)
        node_len.append(int(levels[depth][1]))
        parent.append(par)
        if depth + 1 < len(levels):
            for _ in range(int(levels[depth + 1][0])):
                visit(depth + 1, idx)

    assert int(levels[0][0]) == 1, "the root level has one node"
    visit(0, -1)
    node_off = np.zeros(len(node_len) + 1, dtype=np.int32)
    node_off[1:] = np.cumsum(node_len)
    return node_off, np.asarray(parent, dtype=np.int32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_dtype(x, dtype)


def suffix_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.suffix_len is not None:
        return np.full(cfg.n_suffix, cfg.suffix_len, dtype=np.int32)
    lo, hi = cfg.suffix_len_range
    return rng.integers(lo, hi + 1, size=cfg.n_suffix, dtype=np.int64).astype(np.int32)


def generate(cfg: Config, include_prefix_q: bool = True) -> Dict[str, np.ndarray]:
    """All input tensors of one group, as fp32 arrays holding dtype-exact values.

    Flat groups: q_p, k_p, v_p, do_p [P, H, d]; q_s, k_s, v_s, do_s [T, H, d];
    cu_seqlens [N+1] (int32, over the packed suffix rows) and `microbatches`,
    a list of (first_suffix, last_suffix_exclusive).
    Tree groups: q, k, v, do [C, H, d]; node_off [n+1]; parent [n].
    Tree windows: q_p, k_p, v_p, do_p of the prefix and `windows`, a list of
    dicts with node_off, parent, q, k, v, do per window.
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    out: Dict[str, np.ndarray] = {}
    if cfg.is_windows:
        # the cached prefix, then each window's tree (from its own seed,
        # 100 seed + w) and rows
        p = cfg.prefix_len
        if include_prefix_q:
            out["q_p"] = _normal(rng, (p, hq, d), cfg.dtype)
        else:
            _normal(rng, (p, hq, d), cfg.dtype)
        out["k_p"] = _normal(rng, (p, hkv, d), cfg.dtype)
        out["v_p"] = _normal(rng, (p, hkv, d), cfg.dtype)
        out["do_p"] = _normal(rng, (p, hq, d), cfg.dtype)
        lo, hi = cfg.node_len_range
        wins = []
        for w in range(cfg.windows):
            node_off, parent = random_tree(100 * cfg.seed + w, cfg.window_nodes, max_len=hi,
                                           min_len=lo)
            c = int(node_off[-1])
            wins.append({"node_off": node_off, "parent": parent,
                         "q": _normal(rng, (c, hq, d), cfg.dtype),
                         "k": _normal(rng, (c, hkv, d), cfg.dtype),
                         "v": _normal(rng, (c, hkv, d), cfg.dtype),
                         "do": _normal(rng, (c, hq, d), cfg.dtype)})
        out["windows"] = wins
        return out
    if cfg.is_ranges:
        # the producer tree's rows, then each window's tree (seed 100 seed + w)
        # and rows; window w hangs under the w-th deepest node
        node_off, parent = tree_layout(cfg.tree_levels)
        c = int(node_off[-1])
        out["node_off"], out["parent"] = node_off, parent
        out["q"] = _normal(rng, (c, hq, d), cfg.dtype)
        out["k"] = _normal(rng, (c, hkv, d), cfg.dtype)
        out["v"] = _normal(rng, (c, hkv, d), cfg.dtype)
        out["do"] = _normal(rng, (c, hq, d), cfg.dtype)
        depth = node_depths(parent)
        deepest = [int(x) for x in np.flatnonzero(depth == depth.max())]
        lo, hi = cfg.node_len_range
        wins = []
        for w in range(cfg.windows):
            u = deepest[w % len(deepest)]
            wno, wpa = random_tree(100 * cfg.seed + w, cfg.window_nodes, max_len=hi, min_len=lo)
            rows = int(wno[-1])
            wins.append({"under": u, "ranges": ancestor_row_ranges(node_off, parent, u),
                         "node_off": wno, "parent": wpa,
                         "q": _normal(rng, (rows, hq, d), cfg.dtype),
                         "k": _normal(rng, (rows, hkv, d), cfg.dtype),
                         "v": _normal(rng, (rows, hkv, d), cfg.dtype),
                         "do": _normal(rng, (rows, hq, d), cfg.dtype)})
        out["windows"] = wins
        return out
    if cfg.is_logprob:
        # structure only; the C x V logits are drawn on the device by the caller
        node_off, parent = tree_layout(cfg.tree_levels)
        m = np.concatenate(tree_paths(node_off, parent)).astype(np.int32)
        out["node_off"], out["parent"], out["m"] = node_off, parent, m
        out["y"] = rng.integers(0, cfg.logprob_vocab, size=len(m)).astype(np.int32)
        out["row_ptr"], out["pos"] = positions_by_row(m, int(node_off[-1]))
        out["dlogp"] = rng.standard_normal(len(m)).astype(np.float32)
        return out
    if cfg.is_tree:
        node_off, parent = tree_layout(cfg.tree_levels)
        c = int(node_off[-1])
        out["node_off"], out["parent"] = node_off, parent
        out["q"] = _normal(rng, (c, hq, d), cfg.dtype)
        out["k"] = _normal(rng, (c, hkv, d), cfg.dtype)
        out["v"] = _normal(rng, (c, hkv, d), cfg.dtype)
        out["do"] = _normal(rng, (c, hq, d), cfg.dtype)
        return out
    lens = suffix_lengths(cfg, rng)
    cu = np.zeros(cfg.n_suffix + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    t = int(cu[-1])
    p = cfg.prefix_len
    out["cu_seqlens"] = cu
    q_p = _normal(rng, (p, hq, d), cfg.dtype)
    if include_prefix_q:
        out["q_p"] = q_p
    del q_p
    out["k_p"] = _normal(rng, (p, hkv, d), cfg.dtype)
    out["v_p"] = _normal(rng, (p, hkv, d), cfg.dtype)
    out["do_p"] = _normal(rng, (p, hq, d), cfg.dtype)
    out["q_s"] = _normal(rng, (t, hq, d), cfg.dtype)
    out["k_s"] = _normal(rng, (t, hkv, d), cfg.dtype)
    out["v_s"] = _normal(rng, (t, hkv, d), cfg.dtype)
    out["do_s"] = _normal(rng, (t, hq, d), cfg.dtype)
    per = cfg.n_suffix // cfg.microbatches
    out["microbatches"] = np.asarray(
        [(i * per, (i + 1) * per if i + 1 < cfg.microbatches else cfg.n_suffix)
         for i in range(cfg.microbatches)], dtype=np.int32)
    return out


def random_small_group(seed: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       prefix_len: int, suffix_lens: Sequence[int], dtype: str = "f32",
                       scale_q: float = 1.0) -> Dict[str, np.ndarray]:
    """A small flat group with arbitrary (possibly ragged or empty) suffixes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    t = int(np.sum(suffix_lens))
    cu = np.zeros(len(suffix_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(suffix_lens, dtype=np.int64))
    out = {"cu_seqlens": cu}
    out["q_p"] = _normal(rng, (prefix_len, num_q_heads, head_dim), dtype) * np.float32(scale_q)
    out["k_p"] = _normal(rng, (prefix_len, num_kv_heads, head_dim), dtype)
    out["v_p"] = _normal(rng, (prefix_len, num_kv_heads, head_dim), dtype)
    out["do_p"] = _normal(rng, (prefix_len, num_q_heads, head_dim), dtype)
    out["q_s"] = _normal(rng, (t, num_q_heads, head_dim), dtype) * np.float32(scale_q)
    out["k_s"] = _normal(rng, (t, num_kv_heads, head_dim), dtype)
    out["v_s"] = _normal(rng, (t, num_kv_heads, head_dim), dtype)
    out["do_s"] = _normal(rng, (t, num_q_heads, head_dim), dtype)
    return out


def random_tree(seed: int, n_nodes: int, max_len: int, min_len: int = 1):
    """A random tree in DFS preorder: (node_off, parent).  parent[i] < i."""
    rng = np.random.Generator(np.random.PCG64(seed))
    # build a random rooted tree, then renumber it in preorder
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, n_nodes)]
    children: List[List[int]] = [[] for _ in range(n_nodes)]
    for i in range(1, n_nodes):
        children[par[i]].append(i)
    order: List[int] = []
    stack = [0]
    while stack:
        v = stack.pop()
        order.append(v)
        stack.extend(reversed(children[v]))
    new_id = {v: i for i, v in enumerate(order)}
    parent = np.asarray([-1 if par[v] < 0 else new_id[par[v]] for v in order], dtype=np.int32)
    lens = rng.integers(min_len, max_len + 1, size=n_nodes)
    node_off = np.zeros(n_nodes + 1, dtype=np.int32)
    node_off[1:] = np.cumsum(lens)
    return node_off, parent


def random_tree_group(seed: int, node_off: np.ndarray, num_q_heads: int, num_kv_heads: int,
                      head_dim: int, dtype: str = "f32") -> Dict[str, np.ndarray]:
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    c = int(node_off[-1])
    return {
        "q": _normal(rng, (c, num_q_heads, head_dim), dtype),
        "k": _normal(rng, (c, num_kv_heads, head_dim), dtype),
        "v": _normal(rng, (c, num_kv_heads, head_dim), dtype),
        "do": _normal(rng, (c, num_q_heads, head_dim), dtype),
    }


def positions_by_row(m: np.ndarray, n_rows: int):
    """(row_ptr [C+1], pos [S]) grouping positions s by their compact row m(s),
    in increasing s within a row (the layout the compact log-probability
    calls take)."""
    m = np.asarray(m, dtype=np.int64)
    order = np.argsort(m, kind="stable")
    counts = np.bincount(m, minlength=n_rows)
    row_ptr = np.zeros(n_rows + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr, order.astype(np.int32)


def random_logprob_case(seed: int, n_rows: int, vocab: int, n_pos: int, dtype: str = "f32"):
    """Compact-row logits z [C, V] (N(0, 3^2), rounded to dtype), a random row
    m(s) and target y_s per position (some rows unread, some (row, target)
    pairs repeated), the grouped layout, and an upstream dlogp [S]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    z = round_to_dtype(rng.standard_normal((n_rows, vocab), dtype=np.float32) * 3.0, dtype)
    m = rng.integers(0, max(1, n_rows - 1), size=n_pos)      # the last row is never read
    y = rng.integers(0, vocab, size=n_pos)
    if n_pos >= 4:
        m[1], y[1] = m[0], y[0]                                # a repeated (row, target)
        m[3] = m[2]                                            # a shared row, other target
    row_ptr, pos = positions_by_row(m, n_rows)
    dlogp = rng.standard_normal(n_pos).astype(np.float32)
    return {"z": z, "m": m.astype(np.int32), "y": y.astype(np.int32), "row_ptr": row_ptr,
            "pos": pos, "dlogp": dlogp}


def tree_paths(node_off: np.ndarray, parent: np.ndarray) -> List[np.ndarray]:
    """Compact rows of every root-to-leaf trajectory of a DFS-preorder tree, in
    leaf order: position t of a trajectory reads compact row path[t]."""
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    has_child[np.asarray(parent[1:], dtype=np.int64)] = True
    paths = []
    for leaf in np.flatnonzero(~has_child):
        chain = []
        u = int(leaf)
        while u >= 0:
            chain.append(u)
            u = int(parent[u])
        paths.append(np.concatenate([np.arange(node_off[u], node_off[u + 1]) for u in reversed(chain)]))
    return paths



def ancestor_row_ranges(node_off: np.ndarray, parent: np.ndarray, u: int):
    """(start, length) of the compact rows of node u and of each of its
    ancestors, root first: the rows a consumer window attached under u reads
    (in trajectory order)."""
    chain = []
    while u >= 0:
        chain.append(int(u))
        u = int(parent[u])
    return [(int(node_off[a]), int(node_off[a + 1] - node_off[a])) for a in reversed(chain)]


def node_depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int64)
    for v in range(1, len(parent)):
        d[v] = d[parent[v]] + 1
    return d


def forest(trees):
    """One node table for several trees numbered one after another (each
    root's parent -1): (node_off, parent)."""
    parent, node_off = [], [0]
    for no, pa in trees:
        base = len(parent)
        parent += [int(x) + base if x >= 0 else -1 for x in pa]
        node_off += [int(x) + node_off[-1] for x in no[1:]]
    return np.asarray(node_off, dtype=np.int32), np.asarray(parent, dtype=np.int32)
