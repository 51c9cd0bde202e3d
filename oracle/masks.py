"""Visibility masks, each built from its definition on the pages.

* Causal: key k is visible to query q iff k <= q (standard causal LM; the
  diagonal is inclusive).
* Suffix rows of a trajectory [P || S_i]: suffix row j sits at trajectory
  position P + j and sees positions 0 .. P + j, i.e. every prefix token and
  its own suffix up to itself (PrefixFlow §4.1, the three conditions on the
  Phase-B mask; rows are aligned bottom-right, as HARTS §4 states for its
  packed Q/KV views).
* Trees: a compact row of node v sees the rows of every strict ancestor of v
  and the rows of v up to itself (HARTS §2.1 and §2.2: positions with equal
  token prefixes share a row, and full attention reads ancestor K/V through
  a tree mask).  This is the ancestor definition; the GPU path uses a
  preorder-interval rule that the tests check against it.

Test infrastructure only.
"""
import numpy as np


def causal_mask(n: int) -> np.ndarray:
    idx = np.arange(n)
    return idx[None, :] <= idx[:, None]


def suffix_rows_mask(prefix_len: int, suffix_len: int) -> np.ndarray:
    """[S, P+S] visibility of suffix rows over trajectory positions."""
    pos_q = prefix_len + np.arange(suffix_len)
    pos_k = np.arange(prefix_len + suffix_len)
    return pos_k[None, :] <= pos_q[:, None]


def tree_node_of_row(node_off: np.ndarray) -> np.ndarray:
    n_rows = int(node_off[-1])
    node = np.zeros(n_rows, dtype=np.int64)
    for v in range(len(node_off) - 1):
        node[node_off[v]:node_off[v + 1]] = v
    return node


def tree_ancestors(parent: np.ndarray):
    """anc[v] = set of strict ancestors of node v."""
    anc = []
    for v in range(len(parent)):
        s = set()
        u = int(parent[v])
        while u >= 0:
            s.add(u)
            u = int(parent[u])
        anc.append(s)
    return anc


def tree_ancestor_mask(node_off: np.ndarray, parent: np.ndarray) -> np.ndarray:
    """[C, C] visibility over compact rows: ancestor rows, plus own node causally."""
    node = tree_node_of_row(node_off)
    anc = tree_ancestors(parent)
    n = len(parent)
    # node-level relation: is node u a strict ancestor of node v
    is_anc = np.zeros((n, n), dtype=bool)          # [v, u]
    for v in range(n):
        for u in anc[v]:
            is_anc[v, u] = True
    rows = np.arange(len(node))
    same = node[:, None] == node[None, :]
    own_causal = same & (rows[None, :] <= rows[:, None])
    return own_causal | is_anc[node[:, None], node[None, :]]
