"""The benchmark's work counts, which every reported TFLOP/s rests on, against
brute-force counts of the oracle's visibility masks.

A Phase-B suffix row j sees the P prefix keys and its own keys 0..j; a prefix
row q sees keys 0..q; a tree row sees its own node up to itself and every
ancestor node; a tree-window row also sees the whole prefix.  The benchmark
prices a visible (query, key) pair per query head at 12 d FLOP (forward 4 d,
backward 8 d)."""
import numpy as np
import pytest

import bench
from oracle import causal_mask, suffix_rows_mask, tree_ancestor_mask
from workloads import get_config
from workloads.gen import random_tree


@pytest.mark.parametrize("seed", range(6))
def test_flat_pairs_match_the_masks(seed):
    rng = np.random.default_rng(seed)
    p = int(rng.integers(0, 40))
    lens = rng.integers(0, 25, size=int(rng.integers(1, 6)))
    phase_b, prefix = bench.flat_pairs(p, lens)
    assert phase_b == sum(int(suffix_rows_mask(p, int(s)).sum()) for s in lens)
    assert prefix == int(causal_mask(p).sum())


@pytest.mark.parametrize("seed", range(6))
def test_tree_and_window_pairs_match_the_masks(seed):
    node_off, parent = random_tree(seed, 9, max_len=12, min_len=0)
    c = int(node_off[-1])
    vis = tree_ancestor_mask(node_off, parent)
    assert bench.tree_pairs(node_off, parent) == int(vis.sum())
    p = 7 + seed
    assert bench.window_pairs(p, node_off, parent) == c * p + int(vis.sum())


def test_phase_b_work_at_the_headline_group():
    """GQA 32/8, d 128, P 4096, 8 suffixes of 512: 570 490 880 visible pairs
    over all query heads, 876.27 GFLOP of forward and backward."""
    cfg = get_config(2)
    pairs, _ = bench.flat_pairs(cfg.prefix_len, [cfg.suffix_len] * cfg.n_suffix)
    assert pairs * cfg.num_q_heads == 570_490_880
    flops = 12.0 * cfg.head_dim * pairs * cfg.num_q_heads
    assert round(flops / 1e9, 2) == 876.27


@pytest.mark.parametrize("seed", range(4))
def test_ranges_window_pairs_match_the_masks(seed):
    """A window under a producer node sees every row of its cached ranges plus
    its own tree pairs: brute force over the combined tree's ancestor mask
    (the consumer's root a child of the node)."""
    from workloads.gen import ancestor_row_ranges
    node_off_p, parent_p = random_tree(30 + seed, 8, max_len=6, min_len=1)
    u = int(np.argmax(np.arange(len(parent_p))))      # the last node
    ranges = ancestor_row_ranges(node_off_p, parent_p, u)
    no_c, pa_c = random_tree(40 + seed, 6, max_len=5, min_len=0)
    cp = int(node_off_p[-1])
    n_p = len(parent_p)
    parent = np.concatenate([parent_p, np.where(pa_c < 0, u, pa_c + n_p)]).astype(np.int32)
    node_off = np.concatenate([node_off_p, no_c[1:] + cp]).astype(np.int32)
    vis = tree_ancestor_mask(node_off, parent)
    w = {"node_off": no_c, "parent": pa_c, "ranges": ranges}
    assert bench.ranges_window_pairs(w) == int(vis[cp:].sum())


def test_profiler_names_are_recovered():
    """rocprofv3 leaves a template over __bf16 mangled; the summaries find the
    kernel's name in it, and leave demangled names alone."""
    mangled = ("_ZN2pf16prep_dsum_kernelIDF16bLi128EEEvNS_8SegTableENS_9HeadTableENS_7RowInfo"
               "ENS_8AttnArgsEi")
    plain = bench.plain_name(mangled)
    assert "prep_dsum_kernel" in plain.split("::")
    assert bench._pick({plain: (5.0, 2)}, "prep_dsum_kernel", whole=True) == (5.0, 2)
    demangled = "void pf::(anonymous namespace)::fwd_kernel<1>(pf::AttnArgs)"
    assert bench.plain_name(demangled) == demangled
    # a whole-identifier match: fwd_kernel is not logprob_fwd_kernel
    assert bench._pick({"pf::logprob_fwd_kernel(int)": (1.0, 1)}, "fwd_kernel", whole=True) is None


def test_stored_figures_are_keyed_to_their_kernel_family(tmp_path, monkeypatch):
    """A stored counter figure carries a hash of its family's kernel file and
    the common sources: editing another family's kernel file keeps it, editing
    its own or a common file does not."""
    assert bench.config_family(2) == "bf16"
    assert bench.config_family(9) == "f32"
    assert bench.config_family(7) == "logprob"
    csrc = tmp_path / "shared_prefix_attention_pf_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("pf_attn_bf16.hip", "pf_attn_f32.hip", "pf_logprob.hip", "pf_api.cpp",
                 "pf_internal.h"):
        (csrc / name).write_text(name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {f: bench.kernel_source_hash(f) for f in ("bf16", "f32", "logprob")}
    assert len(set(before.values())) == 3
    (csrc / "pf_attn_f32.hip").write_text("changed")
    after = {f: bench.kernel_source_hash(f) for f in ("bf16", "f32", "logprob")}
    assert after["bf16"] == before["bf16"] and after["logprob"] == before["logprob"]
    assert after["f32"] != before["f32"]
    (csrc / "pf_api.cpp").write_text("changed")
    assert all(bench.kernel_source_hash(f) != after[f] for f in after)


def test_counter_phases_cover_both_families():
    """The SQ counter summary labels a kernel's dispatches by the phases a flat
    group's step runs it in; every kernel a flat group launches in more than
    one phase, in either dtype family, must be listed, or its last (Phase C)
    dispatch would be labelled Phase B."""
    two_phase = {"fwd_kernel", "bwd_dkv_kernel", "bwd_dq_ds_kernel", "fwd_f32_kernel",
                 "dkv_f32_kernel", "dq_ds_f32_kernel", "prep_dsum_kernel", "partial_sums_kernel"}
    assert two_phase <= set(bench.PHASES_OF)
    assert set(bench.PHASES_OF) <= set(bench.KERNEL_SYMBOL.values())
    for k in ("fwd_kernel", "fwd_f32_kernel"):
        assert bench.PHASES_OF[k] == ("A", "B")
    for k in ("bwd_dkv_kernel", "dkv_f32_kernel", "bwd_dq_ds_kernel", "dq_ds_f32_kernel"):
        assert bench.PHASES_OF[k] == ("B", "C")
