"""Device-memory plumbing around the binding: allocate outputs and workspaces
with torch on the caller's device and call the library entry points.

Nothing here computes attention; each helper allocates what its entry point
writes and forwards the call.
"""
from typing import Optional, Sequence

import torch

from . import (
    PF_BF16,
    PF_F32,
    PF_OP_PREFIX_BWD,
    PF_OP_PREFIX_FWD,
    PF_OP_SUFFIX_BWD,
    PF_OP_SUFFIX_FWD,
    PF_OP_TREE_BWD,
    PF_OP_TREE_FWD,
    PF_OP_TREE_SUFFIX_BWD,
    PF_OP_TREE_SUFFIX_FWD,
    AttnDesc,
    pf_prefix_bwd_inject,
    pf_prefix_fwd,
    pf_suffix_attn_bwd_accum,
    pf_suffix_attn_fwd,
    pf_tree_attn_bwd,
    pf_tree_attn_fwd,
    pf_ranges_cached_keys,
    pf_tree_attn_bwd_inject,
    pf_tree_suffix_attn_bwd_accum,
    pf_tree_suffix_attn_bwd_accum_ranges,
    pf_tree_suffix_attn_fwd,
    pf_tree_suffix_attn_fwd_ranges,
    pf_workspace_size,
)

TORCH_DTYPE = {PF_BF16: torch.bfloat16, PF_F32: torch.float32}


def desc_for(q: torch.Tensor, k: torch.Tensor, softmax_scale: float = 0.0,
             q_to_kv: Optional[Sequence[int]] = None) -> AttnDesc:
    dtype = PF_BF16 if q.dtype == torch.bfloat16 else PF_F32
    return AttnDesc(q.shape[1], k.shape[1], q.shape[2], dtype, softmax_scale, q_to_kv)


def workspace(op: int, desc: AttnDesc, prefix_len: int, rows: int, device) -> torch.Tensor:
    n = pf_workspace_size(op, desc, prefix_len, rows)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def prefix_fwd(desc, q_p, k_p, v_p, ws=None, stream=None):
    p = q_p.shape[0]
    o_p = torch.empty_like(q_p)
    lse_p = torch.empty(desc.num_q_heads, p, dtype=torch.float32, device=q_p.device)
    if ws is None:
        ws = workspace(PF_OP_PREFIX_FWD, desc, p, p, q_p.device)
    pf_prefix_fwd(desc, p, q_p, k_p, v_p, o_p, lse_p, ws, stream)
    return o_p, lse_p


def suffix_fwd(desc, k_p, v_p, cu_seqlens, q_s, k_s, v_s, ws=None, stream=None):
    rows = int(cu_seqlens[-1])
    o_s = torch.empty_like(q_s)
    lse_s = torch.empty(desc.num_q_heads, rows, dtype=torch.float32, device=q_s.device)
    if ws is None:
        ws = workspace(PF_OP_SUFFIX_FWD, desc, k_p.shape[0], rows, q_s.device)
    pf_suffix_attn_fwd(desc, k_p.shape[0], k_p, v_p, cu_seqlens, q_s, k_s, v_s, o_s, lse_s, ws,
                       stream)
    return o_s, lse_s


def suffix_bwd(desc, k_p, v_p, cu_seqlens, q_s, k_s, v_s, o_s, lse_s, do_s, gk_acc, gv_acc,
               ws=None, stream=None):
    rows = int(cu_seqlens[-1])
    dq_s = torch.empty_like(q_s)
    dk_s = torch.empty_like(k_s)
    dv_s = torch.empty_like(v_s)
    if ws is None:
        ws = workspace(PF_OP_SUFFIX_BWD, desc, k_p.shape[0], rows, q_s.device)
    pf_suffix_attn_bwd_accum(desc, k_p.shape[0], k_p, v_p, cu_seqlens, q_s, k_s, v_s, o_s, lse_s,
                             do_s, dq_s, dk_s, dv_s, gk_acc, gv_acc, ws, stream)
    return dq_s, dk_s, dv_s


def prefix_bwd(desc, q_p, k_p, v_p, o_p, lse_p, do_p, gk_acc, gv_acc, dkv_dtype=None, ws=None,
               stream=None):
    p = q_p.shape[0]
    if dkv_dtype is None:
        dkv_dtype = desc.dtype
    dq_p = torch.empty_like(q_p)
    dk_p = torch.empty(k_p.shape, dtype=TORCH_DTYPE[dkv_dtype], device=k_p.device)
    dv_p = torch.empty(v_p.shape, dtype=TORCH_DTYPE[dkv_dtype], device=v_p.device)
    if ws is None:
        ws = workspace(PF_OP_PREFIX_BWD, desc, p, p, q_p.device)
    pf_prefix_bwd_inject(desc, p, q_p, k_p, v_p, o_p, lse_p, do_p, gk_acc, gv_acc, dq_p, dk_p,
                         dv_p, dkv_dtype, ws, stream)
    return dq_p, dk_p, dv_p


def tree_fwd(desc, node_off, parent, q, k, v, ws=None, stream=None):
    rows = int(node_off[-1])
    o = torch.empty_like(q)
    lse = torch.empty(desc.num_q_heads, rows, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(PF_OP_TREE_FWD, desc, 0, rows, q.device)
    pf_tree_attn_fwd(desc, node_off, parent, q, k, v, o, lse, ws, stream)
    return o, lse


def tree_bwd(desc, node_off, parent, q, k, v, o, lse, dout, ws=None, stream=None):
    rows = int(node_off[-1])
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if ws is None:
        ws = workspace(PF_OP_TREE_BWD, desc, 0, rows, q.device)
    pf_tree_attn_bwd(desc, node_off, parent, q, k, v, o, lse, dout, dq, dk, dv, ws, stream)
    return dq, dk, dv


def tree_suffix_fwd(desc, k_p, v_p, node_off, parent, q, k, v, ws=None, stream=None):
    rows = int(node_off[-1])
    o = torch.empty_like(q)
    lse = torch.empty(desc.num_q_heads, rows, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(PF_OP_TREE_SUFFIX_FWD, desc, k_p.shape[0], rows, q.device)
    pf_tree_suffix_attn_fwd(desc, k_p.shape[0], k_p, v_p, node_off, parent, q, k, v, o, lse, ws,
                            stream)
    return o, lse


def tree_suffix_bwd(desc, k_p, v_p, node_off, parent, q, k, v, o, lse, dout, gk_acc, gv_acc,
                    ws=None, stream=None):
    rows = int(node_off[-1])
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if ws is None:
        ws = workspace(PF_OP_TREE_SUFFIX_BWD, desc, k_p.shape[0], rows, q.device)
    pf_tree_suffix_attn_bwd_accum(desc, k_p.shape[0], k_p, v_p, node_off, parent, q, k, v, o, lse,
                                  dout, dq, dk, dv, gk_acc, gv_acc, ws, stream)
    return dq, dk, dv



def tree_suffix_fwd_ranges(desc, k_c, v_c, ranges, node_off, parent, q, k, v, ws=None,
                           stream=None):
    """ranges: (start, length) row spans of k_c / v_c, in trajectory order."""
    starts = [int(s) for s, _ in ranges]
    lens = [int(n) for _, n in ranges]
    rows = int(node_off[-1])
    o = torch.empty_like(q)
    lse = torch.empty(desc.num_q_heads, rows, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(PF_OP_TREE_SUFFIX_FWD, desc, pf_ranges_cached_keys(lens), rows, q.device)
    pf_tree_suffix_attn_fwd_ranges(desc, k_c, v_c, starts, lens, node_off, parent, q, k, v, o, lse,
                                   ws, stream)
    return o, lse


def tree_suffix_bwd_ranges(desc, k_c, v_c, ranges, node_off, parent, q, k, v, o, lse, dout, gk_acc,
                           gv_acc, ws=None, stream=None):
    starts = [int(s) for s, _ in ranges]
    lens = [int(n) for _, n in ranges]
    rows = int(node_off[-1])
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if ws is None:
        ws = workspace(PF_OP_TREE_SUFFIX_BWD, desc, pf_ranges_cached_keys(lens), rows, q.device)
    pf_tree_suffix_attn_bwd_accum_ranges(desc, k_c, v_c, starts, lens, node_off, parent, q, k, v,
                                         o, lse, dout, dq, dk, dv, gk_acc, gv_acc, ws, stream)
    return dq, dk, dv


def tree_bwd_inject(desc, node_off, parent, q, k, v, o, lse, dout, gk_acc, gv_acc, dkv_dtype=None,
                    ws=None, stream=None):
    rows = int(node_off[-1])
    if dkv_dtype is None:
        dkv_dtype = desc.dtype
    dq = torch.empty_like(q)
    dk = torch.empty(k.shape, dtype=TORCH_DTYPE[dkv_dtype], device=k.device)
    dv = torch.empty(v.shape, dtype=TORCH_DTYPE[dkv_dtype], device=v.device)
    if ws is None:
        ws = workspace(PF_OP_TREE_BWD, desc, 0, rows, q.device)
    pf_tree_attn_bwd_inject(desc, node_off, parent, q, k, v, o, lse, dout, gk_acc, gv_acc, dq, dk,
                            dv, dkv_dtype, ws, stream)
    return dq, dk, dv
