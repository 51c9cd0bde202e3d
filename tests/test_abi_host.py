"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/pf.h declares, and
reject invalid arguments with the documented status before any HIP call.
The tree helper is checked against the oracle's ancestor mask.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import shared_prefix_attention_pf_amd as pf
from oracle import tree_ancestor_mask
from workloads.gen import random_tree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000   # a 16-byte aligned address that validation-failing calls never dereference


def _header_functions():
    src = open(os.path.join(ROOT, "include", "pf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pf_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(pf.LIB_PATH)
    names = _header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pf.EXPORTED)


def test_abi_version_and_status_strings():
    assert pf.pf_abi_version() == 1
    for s in range(5):
        assert pf._lib.pf_status_string(s).decode().startswith("PF_")


def _t(rows_heads_d=None, addr=FAKE, st=None, sh=None, heads=8, d=128):
    st = heads * d if st is None else st
    sh = d if sh is None else sh
    return pf._Tensor(addr, st, sh)


def _desc(hq=32, hkv=8, d=128, dtype=pf.PF_BF16, q_to_kv=None):
    return pf.AttnDesc(hq, hkv, d, dtype, 0.0, q_to_kv)._c()


def _suffix_fwd(desc_keep, cu, ws=FAKE, ws_bytes=1 << 30, q=None, kp=None, lse=FAKE):
    d, _keep = desc_keep
    cu_arr = np.asarray(cu, dtype=np.int32)
    cu_p = cu_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    q = q or _t(heads=d.num_q_heads, d=d.head_dim)
    kv = _t(heads=d.num_kv_heads, d=d.head_dim)
    kp = kp or kv
    return pf._lib.pf_suffix_attn_fwd(ctypes.byref(d), 64, kp, kv, len(cu) - 1, cu_p, q, kv, kv, q,
                                      ctypes.c_void_p(lse), ctypes.c_void_p(ws), ws_bytes,
                                      ctypes.c_void_p(0))


def test_binding_constants_match_the_header():
    src = open(os.path.join(ROOT, "include", "pf.h")).read()
    defs = dict(re.findall(r"#define\s+(PF_MAX_[A-Z]+)\s+(\d+)", src))
    assert int(defs["PF_MAX_SEGMENTS"]) == pf.PF_MAX_SEGMENTS
    assert int(defs["PF_MAX_HEADS"]) == pf.PF_MAX_HEADS
    m = re.search(r"#define\s+PF_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == pf.PF_NOALLOC_SCRATCH_BYTES


def test_rejects_bad_head_config():
    h = pf.PF_MAX_HEADS + 1
    assert _suffix_fwd(_desc(hq=h, hkv=h), [0, 4]) == pf.PF_ERR_UNSUPPORTED
    assert _suffix_fwd(_desc(hq=30, hkv=8), [0, 4]) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(_desc(hq=0, hkv=8), [0, 4]) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(_desc(d=96), [0, 4]) == pf.PF_ERR_UNSUPPORTED
    assert _suffix_fwd(_desc(d=64), [0, 4]) == pf.PF_ERR_UNSUPPORTED          # bf16 needs 128
    assert _suffix_fwd(_desc(hq=4, hkv=2, q_to_kv=[0, 0, 0, 1]), [0, 4]) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(_desc(hq=4, hkv=2, q_to_kv=[0, 1, 2, 1]), [0, 4]) == pf.PF_ERR_INVALID_ARG
    msg = pf._lib.pf_last_error().decode()
    assert "q_to_kv" in msg


def test_rejects_bad_cu_seqlens():
    assert _suffix_fwd(_desc(), [1, 4]) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(_desc(), [0, 8, 4]) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(_desc(), list(range(pf.PF_MAX_SEGMENTS + 2))) == pf.PF_ERR_UNSUPPORTED


def test_rejects_bad_tensors():
    d = _desc()
    assert _suffix_fwd(d, [0, 4], q=_t(addr=FAKE + 8, heads=32)) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(d, [0, 4], q=_t(addr=0, heads=32)) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(d, [0, 4], q=_t(st=32 * 128 + 3, heads=32)) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(d, [0, 4], q=_t(st=64, sh=64, heads=32)) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(d, [0, 4], kp=_t(addr=0)) == pf.PF_ERR_INVALID_ARG
    assert _suffix_fwd(d, [0, 4], lse=0) == pf.PF_ERR_INVALID_ARG


def test_rejects_small_workspace():
    d = pf.AttnDesc(32, 8, 128)
    need = pf.pf_workspace_size(pf.PF_OP_SUFFIX_FWD, d, 64, 4)
    assert need > 0
    assert _suffix_fwd(d._c(), [0, 4], ws_bytes=need - 1) == pf.PF_ERR_WORKSPACE
    assert _suffix_fwd(d._c(), [0, 4], ws=0) == pf.PF_ERR_WORKSPACE


def test_workspace_sizes():
    d = pf.AttnDesc(32, 8, 128)
    assert pf.pf_workspace_size(pf.PF_OP_SUFFIX_FWD, d, 4096, 0) == 0
    small = pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, d, 4096, 512)
    big = pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, d, 4096, 4096)
    assert big >= small > 0
    # fp32: the full workspace adds the fp32 dS buffer, Hq x (ceil256(P) +
    # ceil256(rows)) keys x ceil256(rows) rows of 4 bytes, twice the bf16 one;
    # the minimal one (dQ recomputes S and dP) has neither it nor partials here
    f = pf.AttnDesc(2, 2, 64, pf.PF_F32)
    fb = pf.AttnDesc(2, 2, 128, pf.PF_BF16)
    full = pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, f, 256, 256)
    low = pf.pf_workspace_size_min(pf.PF_OP_SUFFIX_BWD, f, 256, 256)
    assert low < 64 * 1024
    assert full - low >= 2 * 512 * 256 * 4
    assert (full - low) - (pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, fb, 256, 256) -
                           pf.pf_workspace_size_min(pf.PF_OP_SUFFIX_BWD, fb, 256, 256)) \
        >= 2 * 512 * 256 * 2
    bad = pf.AttnDesc(3, 2, 128)
    assert pf.pf_workspace_size(pf.PF_OP_SUFFIX_FWD, bad, 16, 16) == 0


def test_rejects_bad_trees():
    def subtree(node_off, parent):
        no = np.asarray(node_off, dtype=np.int32)
        pa = np.asarray(parent, dtype=np.int32)
        out = np.zeros(len(pa), dtype=np.int32)
        p32 = ctypes.POINTER(ctypes.c_int32)
        return pf._lib.pf_tree_subtree_end(len(pa), no.ctypes.data_as(p32), pa.ctypes.data_as(p32),
                                           out.ctypes.data_as(p32))
    assert subtree([0, 4, 6], [-1, 0]) == pf.PF_OK
    assert subtree([0, 4, 6], [0, 0]) == pf.PF_ERR_INVALID_ARG          # root must have -1
    assert subtree([0, 4, 6, 7], [-1, 2, 0]) == pf.PF_ERR_INVALID_ARG   # parent after child
    assert subtree([0, 4, 3], [-1, 0]) == pf.PF_ERR_INVALID_ARG          # offsets decrease
    # 0 -> 1 -> 2 and 0 -> 3, then node 4 claiming parent 1 breaks preorder
    assert subtree([0, 1, 2, 3, 4, 5], [-1, 0, 1, 0, 1]) == pf.PF_ERR_INVALID_ARG
    # a forest: node 2 starts a second tree; node 3 may not reach into the first
    assert subtree([0, 4, 6, 9], [-1, 0, -1]) == pf.PF_OK
    assert subtree([0, 4, 6, 9, 10], [-1, 0, -1, 1]) == pf.PF_ERR_INVALID_ARG


def test_forest_visibility_rule_matches_ancestor_mask():
    """Several random trees numbered one after another (each root's parent -1):
    the subtree-end rule equals the oracle's ancestor mask, so rows of
    different trees never see each other."""
    for seed in range(30):
        rng = np.random.default_rng(100 + seed)
        parent, node_off = [], [0]
        for t in range(int(rng.integers(2, 5))):
            no, pa = random_tree(1000 * seed + t, int(rng.integers(1, 7)), max_len=4, min_len=0)
            base = len(parent)
            parent += [x + base if x >= 0 else -1 for x in pa]
            node_off += [int(x) + node_off[-1] for x in no[1:]]
        node_off = np.asarray(node_off, dtype=np.int32)
        parent = np.asarray(parent, dtype=np.int32)
        if node_off[-1] == 0:
            continue
        end = pf.pf_tree_subtree_end(node_off, parent)
        c = int(node_off[-1])
        node = np.searchsorted(node_off, np.arange(c), side="right") - 1
        rows = np.arange(c)
        rule = (rows[None, :] <= rows[:, None]) & (rows[:, None] < end[node][None, :])
        np.testing.assert_array_equal(rule, tree_ancestor_mask(node_off, parent), err_msg=str(seed))


def test_tree_visibility_rule_matches_ancestor_mask():
    """The library's subtree ends give k <= q < end(node(k)) == the oracle's ancestor mask."""
    for seed in range(60):
        rng = np.random.default_rng(seed)
        node_off, parent = random_tree(seed, int(rng.integers(1, 14)), max_len=5, min_len=0)
        if node_off[-1] == 0:
            continue
        end = pf.pf_tree_subtree_end(node_off, parent)
        c = int(node_off[-1])
        node = np.searchsorted(node_off, np.arange(c), side="right") - 1
        rows = np.arange(c)
        rule = (rows[None, :] <= rows[:, None]) & (rows[:, None] < end[node][None, :])
        np.testing.assert_array_equal(rule, tree_ancestor_mask(node_off, parent), err_msg=str(seed))


def test_prefix_bwd_rejects_bad_dkv_dtype():
    d, _keep = _desc()
    t = _t(heads=32)
    kv = _t()
    st = pf._lib.pf_prefix_bwd_inject(ctypes.byref(d), 64, t, kv, kv, t, ctypes.c_void_p(FAKE), t,
                                      ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), t, kv, kv, 7,
                                      ctypes.c_void_p(FAKE), 1 << 30, ctypes.c_void_p(0))
    assert st == pf.PF_ERR_INVALID_ARG


def test_tree_window_entry_points_validate_on_the_host():
    """The tree-window calls reject a bad tree or a short workspace before any
    launch, and size their workspace like a suffix call over the same rows."""
    d, _keep = _desc()
    p32 = ctypes.POINTER(ctypes.c_int32)

    def fwd(node_off, parent, ws_bytes=1 << 30):
        no = np.asarray(node_off, dtype=np.int32)
        pa = np.asarray(parent, dtype=np.int32)
        rows = int(no[-1])
        q, kv, kp = _t(heads=32), _t(), _t()
        return pf._lib.pf_tree_suffix_attn_fwd(ctypes.byref(d), 64, kp, kp, len(pa),
                                               no.ctypes.data_as(p32), pa.ctypes.data_as(p32), q,
                                               kv, kv, q, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                               ws_bytes, ctypes.c_void_p(0)), rows
    assert fwd([0, 4, 6], [0, 0])[0] == pf.PF_ERR_INVALID_ARG
    assert fwd([0, 4, 6, 7], [-1, 2, 0])[0] == pf.PF_ERR_INVALID_ARG
    desc = pf.AttnDesc(32, 8, 128)
    rows = 6
    need = pf.pf_workspace_size(pf.PF_OP_TREE_SUFFIX_FWD, desc, 64, rows)
    # a suffix call's workspace plus the table of cached-row tiles (8 B per 32
    # keys, rounded to 256 B)
    assert need == pf.pf_workspace_size(pf.PF_OP_SUFFIX_FWD, desc, 64, rows) + 256
    assert fwd([0, 4, 6], [-1, 0], ws_bytes=need - 1)[0] == pf.PF_ERR_WORKSPACE
    full = pf.pf_workspace_size(pf.PF_OP_TREE_SUFFIX_BWD, desc, 4096, 2048)
    least = pf.pf_workspace_size_min(pf.PF_OP_TREE_SUFFIX_BWD, desc, 4096, 2048)
    assert full > least > 0


def test_logprob_entry_points_validate_on_the_host():
    """Bad dtype, vocabulary, alignment or stride is rejected before any launch."""
    lib = pf._lib
    f = lambda n_rows, vocab, z, stride, dtype=pf.PF_BF16: lib.pf_compact_logprob_fwd(
        n_rows, vocab, ctypes.c_void_p(z), stride, dtype, ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 4, ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(0))
    assert f(4, 100, FAKE, 104, dtype=7) == pf.PF_ERR_INVALID_ARG
    assert f(4, 0, FAKE, 104) == pf.PF_ERR_INVALID_ARG
    assert f(4, 100, FAKE + 2, 104) == pf.PF_ERR_INVALID_ARG          # z not 16-byte aligned
    assert f(4, 100, FAKE, 100) == pf.PF_ERR_INVALID_ARG              # 200-byte rows
    assert f(4, 100, FAKE, 96) == pf.PF_ERR_INVALID_ARG               # stride < vocab
    assert f(0, 100, 0, 0) == pf.PF_OK                                # nothing to do



def test_noalloc_rejects_a_call_beyond_its_scratch():
    """The no-alloc backward checks its scratch need on the host: a call whose
    per-row tables and D / LSE exceed the static scratch is refused with
    PF_ERR_UNSUPPORTED before any HIP call (placeholder pointers are never
    touched), and so is an invalid argument."""
    d, _keep = _desc()
    rows = 1 << 17        # 8 x 32 x 131072 bytes of D and LSE alone: past 16 MiB
    cu = np.asarray([0, rows], dtype=np.int32)
    cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    q = _t(heads=32)
    kv = _t(heads=8)
    args = [ctypes.byref(d), 64, kv, kv, 1, cu_p, q, kv, kv, q, ctypes.c_void_p(FAKE), q, q, kv,
            kv, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(0)]
    assert pf._lib.pf_suffix_attn_bwd_accum_noalloc(*args) == pf.PF_ERR_UNSUPPORTED
    assert b"scratch" in pf._lib.pf_last_error()
    args[1] = -1
    assert pf._lib.pf_suffix_attn_bwd_accum_noalloc(*args) == pf.PF_ERR_INVALID_ARG


def test_ranges_entry_points_validate_on_the_host():
    """The windows over producer row ranges reject a range outside the
    producer, overlapping ranges (each cached row is one key, and two
    workgroups would add into the same gK/gV rows) and a short workspace
    before any launch, in both dtypes; the padded key count that sizes their
    workspace rounds each range to 32; the injected tree backward needs both
    accumulators."""
    assert pf.pf_ranges_cached_keys([100, 0, 32, 1]) == 128 + 0 + 32 + 32
    assert pf.pf_ranges_cached_keys([]) == 0
    p32 = ctypes.POINTER(ctypes.c_int32)

    def call(starts, lens, c_rows=1000, dtype=pf.PF_BF16, ws_bytes=1 << 30):
        d, _keep = _desc(dtype=dtype, d=128)
        rs = np.asarray(starts, dtype=np.int32)
        rl = np.asarray(lens, dtype=np.int32)
        no = np.asarray([0, 4, 6], dtype=np.int32)
        pa = np.asarray([-1, 0], dtype=np.int32)
        q, kv = _t(heads=32), _t()
        return pf._lib.pf_tree_suffix_attn_fwd_ranges(
            ctypes.byref(d), c_rows, kv, kv, len(rs), rs.ctypes.data_as(p32),
            rl.ctypes.data_as(p32), len(pa), no.ctypes.data_as(p32), pa.ctypes.data_as(p32), q,
            kv, kv, q, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ws_bytes, ctypes.c_void_p(0))
    assert call([990], [20]) == pf.PF_ERR_INVALID_ARG
    assert call([-1], [5]) == pf.PF_ERR_INVALID_ARG
    assert call([0], [-5]) == pf.PF_ERR_INVALID_ARG
    assert call([0, 50], [100, 40]) == pf.PF_ERR_INVALID_ARG          # overlap
    n = pf.PF_MAX_SEGMENTS + 1
    assert call(list(range(0, 2 * n, 2)), [1] * n, c_rows=2 * n) == pf.PF_ERR_UNSUPPORTED
    assert call([100, 0], [40, 101]) == pf.PF_ERR_INVALID_ARG         # overlaps a later start
    for dtype in (pf.PF_BF16, pf.PF_F32):
        desc = pf.AttnDesc(32, 8, 128, dtype=dtype)
        need = pf.pf_workspace_size(pf.PF_OP_TREE_SUFFIX_FWD, desc,
                                    pf.pf_ranges_cached_keys([100, 40]), 6)
        assert call([0, 500], [100, 40], dtype=dtype, ws_bytes=need - 1) == pf.PF_ERR_WORKSPACE
        # adjacent ranges and an empty range inside another are not overlaps
        assert call([100, 0, 50], [40, 100, 0], dtype=dtype, ws_bytes=need - 1) == \
            pf.PF_ERR_WORKSPACE
    d, _keep = _desc()
    no = np.asarray([0, 4, 6], dtype=np.int32)
    pa = np.asarray([-1, 0], dtype=np.int32)
    q, kv = _t(heads=32), _t()
    st = pf._lib.pf_tree_attn_bwd_inject(
        ctypes.byref(d), 2, no.ctypes.data_as(p32), pa.ctypes.data_as(p32), q, kv, kv, q,
        ctypes.c_void_p(FAKE), q, None, ctypes.c_void_p(FAKE), q, kv, kv, pf.PF_BF16,
        ctypes.c_void_p(FAKE), 1 << 30, ctypes.c_void_p(0))
    assert st == pf.PF_ERR_INVALID_ARG


def test_last_error_is_per_thread_and_bounded():
    """pf_last_error is the calling thread's message of its last failing call,
    kept in a fixed thread-local buffer."""
    import threading
    pf._lib.pf_last_error.restype = ctypes.c_char_p
    got = {}

    def other():
        assert _suffix_fwd(_desc(hq=6, hkv=4), [0, 4]) == pf.PF_ERR_INVALID_ARG
        got["other"] = pf._lib.pf_last_error().decode()

    assert _suffix_fwd(_desc(), [0, 5, 3]) == pf.PF_ERR_INVALID_ARG
    mine = pf._lib.pf_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "cu_seqlens" in mine and "not a multiple" in got["other"]
    assert pf._lib.pf_last_error().decode() == mine
    # overlapping row ranges: the message names the range and fits the buffer
    d, _keep = _desc()
    long_ranges = [(0, 5)] * 3
    rs = np.asarray([r[0] for r in long_ranges], np.int32)
    rl = np.asarray([r[1] for r in long_ranges], np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    no = np.asarray([0, 4], np.int32)
    pa = np.asarray([-1], np.int32)
    q, kv = _t(heads=32), _t()
    st = pf._lib.pf_tree_suffix_attn_fwd_ranges(
        ctypes.byref(d), 100, kv, kv, 3, rs.ctypes.data_as(p32), rl.ctypes.data_as(p32), 1,
        no.ctypes.data_as(p32), pa.ctypes.data_as(p32), q, kv, kv, q, ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), 1 << 30, ctypes.c_void_p(0))
    assert st == pf.PF_ERR_INVALID_ARG
    msg = pf._lib.pf_last_error().decode()
    assert "overlaps" in msg and len(msg) < 512
