"""Python binding of libpf.so, the gfx950 prefix/suffix attention library.

Argument marshalling only: every function here forwards torch tensors (as
device pointers and element strides), host metadata and the current HIP
stream to the C entry point of the same name declared in include/pf.h.  All
arithmetic runs in the library's HIP kernels; if the library is missing the
import fails loudly.  There is no fallback path.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpf.so")

PF_OK, PF_ERR_INVALID_ARG, PF_ERR_UNSUPPORTED, PF_ERR_WORKSPACE, PF_ERR_HIP = range(5)
PF_F32, PF_BF16 = 0, 1
(PF_OP_PREFIX_FWD, PF_OP_SUFFIX_FWD, PF_OP_SUFFIX_BWD, PF_OP_PREFIX_BWD, PF_OP_TREE_FWD,
 PF_OP_TREE_BWD, PF_OP_TREE_SUFFIX_FWD, PF_OP_TREE_SUFFIX_BWD) = range(8)
PF_MAX_SEGMENTS = 256
PF_MAX_HEADS = 256
PF_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = (
    "pf_workspace_size", "pf_workspace_size_min", "pf_prefix_fwd", "pf_suffix_attn_fwd", "pf_suffix_attn_bwd_accum",
    "pf_suffix_attn_bwd_accum_noalloc", "pf_prefix_bwd_inject", "pf_tree_attn_fwd", "pf_tree_attn_bwd", "pf_tree_suffix_attn_fwd",
    "pf_tree_suffix_attn_bwd_accum", "pf_tree_suffix_attn_fwd_ranges",
    "pf_tree_suffix_attn_bwd_accum_ranges", "pf_ranges_cached_keys", "pf_tree_attn_bwd_inject",
    "pf_compact_logprob_fwd", "pf_compact_logprob_bwd",
    "pf_tree_subtree_end",
    "pf_status_string", "pf_last_error", "pf_abi_version", "pf_set_launch_hook",
)


class PFError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_STATUS_NAMES = {0: "PF_OK", 1: "PF_ERR_INVALID_ARG", 2: "PF_ERR_UNSUPPORTED",
                 3: "PF_ERR_WORKSPACE", 4: "PF_ERR_HIP"}


class _Desc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("q_to_kv", ctypes.POINTER(ctypes.c_int32))]


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


# void (*)(const char* kernel, void* stream, int32_t end, void* user)
LAUNCH_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python shared_prefix_attention_pf_amd/build.py`")
    # torch ships its own HIP runtime under the same soname as ROCm's.  Loading
    # torch first makes libpf.so bind to that runtime; loading libpf.so first
    # would put a second HIP runtime in the process, which then sees no device
    # and rejects every launch against memory torch allocated.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    T, D, P = _Tensor, ctypes.POINTER(_Desc), ctypes.c_void_p
    i32, sz, fp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    ip = ctypes.POINTER(ctypes.c_int32)
    sigs = {
        "pf_workspace_size": (sz, [i32, D, i32, i32]),
        "pf_workspace_size_min": (sz, [i32, D, i32, i32]),
        "pf_prefix_fwd": (i32, [D, i32, T, T, T, T, fp, P, sz, P]),
        "pf_suffix_attn_fwd": (i32, [D, i32, T, T, i32, ip, T, T, T, T, fp, P, sz, P]),
        "pf_suffix_attn_bwd_accum": (i32, [D, i32, T, T, i32, ip, T, T, T, T, fp, T, T, T, T,
                                           fp, fp, P, sz, P]),
        "pf_suffix_attn_bwd_accum_noalloc": (i32, [D, i32, T, T, i32, ip, T, T, T, T, fp, T, T,
                                                   T, T, fp, fp, P]),
        "pf_prefix_bwd_inject": (i32, [D, i32, T, T, T, T, fp, T, fp, fp, T, T, T, i32, P, sz,
                                       P]),
        "pf_tree_attn_fwd": (i32, [D, i32, ip, ip, T, T, T, T, fp, P, sz, P]),
        "pf_tree_attn_bwd": (i32, [D, i32, ip, ip, T, T, T, T, fp, T, T, T, T, P, sz, P]),
        "pf_tree_suffix_attn_fwd": (i32, [D, i32, T, T, i32, ip, ip, T, T, T, T, fp, P, sz, P]),
        "pf_tree_suffix_attn_bwd_accum": (i32, [D, i32, T, T, i32, ip, ip, T, T, T, T, fp, T, T, T,
                                                T, fp, fp, P, sz, P]),
        "pf_tree_suffix_attn_fwd_ranges": (i32, [D, i32, T, T, i32, ip, ip, i32, ip, ip, T, T, T, T,
                                                 fp, P, sz, P]),
        "pf_tree_suffix_attn_bwd_accum_ranges": (i32, [D, i32, T, T, i32, ip, ip, i32, ip, ip, T, T,
                                                       T, T, fp, T, T, T, T, fp, fp, P, sz, P]),
        "pf_ranges_cached_keys": (i32, [i32, ip]),
        "pf_tree_attn_bwd_inject": (i32, [D, i32, ip, ip, T, T, T, T, fp, T, fp, fp, T, T, T, i32,
                                          P, sz, P]),
        "pf_compact_logprob_fwd": (i32, [i32, i32, P, ctypes.c_int64, i32, P, P, P, i32, fp, fp,
                                         P]),
        "pf_compact_logprob_bwd": (i32, [i32, i32, P, ctypes.c_int64, i32, fp, P, P, P, i32, fp,
                                         P, ctypes.c_int64, P]),
        "pf_tree_subtree_end": (i32, [i32, ip, ip, ip]),
        "pf_status_string": (ctypes.c_char_p, [i32]),
        "pf_last_error": (ctypes.c_char_p, []),
        "pf_abi_version": (i32, []),
        "pf_set_launch_hook": (None, [LAUNCH_HOOK, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


@dataclass
class AttnDesc:
    """Head configuration; mirrors pf_attn_desc."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: int = PF_BF16
    softmax_scale: float = 0.0
    q_to_kv: Optional[Sequence[int]] = None

    def _c(self):
        d = _Desc(self.num_q_heads, self.num_kv_heads, self.head_dim, self.dtype,
                  float(self.softmax_scale), None)
        keep = None
        if self.q_to_kv is not None:
            keep = (ctypes.c_int32 * len(self.q_to_kv))(*[int(x) for x in self.q_to_kv])
            d.q_to_kv = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
        return d, keep


def _t(x) -> _Tensor:
    """pf_tensor view of a [tokens, heads, head_dim] tensor (or None)."""
    if x is None or x.numel() == 0:
        return _Tensor(None, 0, 0)
    if x.dim() != 3 or (x.shape[2] > 1 and x.stride(2) != 1):
        raise ValueError("tensors must be [tokens, heads, head_dim] with head_dim contiguous")
    return _Tensor(x.data_ptr() if x.numel() else None, x.stride(0), x.stride(1))


def _p(x):
    return None if x is None or x.numel() == 0 else ctypes.c_void_p(x.data_ptr())


def _ints(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _check(status: int):
    if status != PF_OK:
        raise PFError(status, _lib.pf_last_error().decode())


def _ws(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


_hook_keepalive = None


def pf_set_launch_hook(fn) -> None:
    """Install fn(kernel: str, stream: int, end: int) around every kernel launch, or None."""
    global _hook_keepalive
    if fn is None:
        _hook_keepalive = None
        _lib.pf_set_launch_hook(LAUNCH_HOOK(), None)
        return
    _hook_keepalive = LAUNCH_HOOK(lambda k, s, e, u: fn(k.decode(), s or 0, e))
    _lib.pf_set_launch_hook(_hook_keepalive, None)


def pf_abi_version() -> int:
    return _lib.pf_abi_version()


def pf_workspace_size(op: int, desc: AttnDesc, prefix_len: int, rows: int) -> int:
    d, _keep = desc._c()
    return int(_lib.pf_workspace_size(op, ctypes.byref(d), prefix_len, rows))


def pf_workspace_size_min(op: int, desc: AttnDesc, prefix_len: int, rows: int) -> int:
    d, _keep = desc._c()
    return int(_lib.pf_workspace_size_min(op, ctypes.byref(d), prefix_len, rows))


def pf_tree_subtree_end(node_off, parent) -> np.ndarray:
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    out = np.zeros(len(pa), dtype=np.int32)
    _check(_lib.pf_tree_subtree_end(len(pa), no_p, pa_p,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out


def pf_prefix_fwd(desc, prefix_len, q_p, k_p, v_p, o_p, lse_p, workspace, stream=None):
    d, _keep = desc._c()
    ws, nws = _ws(workspace)
    _check(_lib.pf_prefix_fwd(ctypes.byref(d), prefix_len, _t(q_p), _t(k_p), _t(v_p), _t(o_p),
                              _p(lse_p), ws, nws, _stream(stream)))


def pf_suffix_attn_fwd(desc, prefix_len, k_p, v_p, cu_seqlens, q_s, k_s, v_s, o_s, lse_s,
                       workspace, stream=None):
    d, _keep = desc._c()
    cu, cu_p = _ints(cu_seqlens)
    ws, nws = _ws(workspace)
    _check(_lib.pf_suffix_attn_fwd(ctypes.byref(d), prefix_len, _t(k_p), _t(v_p), len(cu) - 1,
                                   cu_p, _t(q_s), _t(k_s), _t(v_s), _t(o_s), _p(lse_s), ws, nws,
                                   _stream(stream)))


def pf_suffix_attn_bwd_accum(desc, prefix_len, k_p, v_p, cu_seqlens, q_s, k_s, v_s, o_s, lse_s,
                             do_s, dq_s, dk_s, dv_s, gk_acc, gv_acc, workspace, stream=None):
    d, _keep = desc._c()
    cu, cu_p = _ints(cu_seqlens)
    ws, nws = _ws(workspace)
    _check(_lib.pf_suffix_attn_bwd_accum(
        ctypes.byref(d), prefix_len, _t(k_p), _t(v_p), len(cu) - 1, cu_p, _t(q_s), _t(k_s),
        _t(v_s), _t(o_s), _p(lse_s), _t(do_s), _t(dq_s), _t(dk_s), _t(dv_s), _p(gk_acc),
        _p(gv_acc), ws, nws, _stream(stream)))


def pf_suffix_attn_bwd_accum_noalloc(desc, prefix_len, k_p, v_p, cu_seqlens, q_s, k_s, v_s,
                                     o_s, lse_s, do_s, dq_s, dk_s, dv_s, gk_acc, gv_acc,
                                     stream=None):
    d, _keep = desc._c()
    cu, cu_p = _ints(cu_seqlens)
    _check(_lib.pf_suffix_attn_bwd_accum_noalloc(
        ctypes.byref(d), prefix_len, _t(k_p), _t(v_p), len(cu) - 1, cu_p, _t(q_s), _t(k_s),
        _t(v_s), _t(o_s), _p(lse_s), _t(do_s), _t(dq_s), _t(dk_s), _t(dv_s), _p(gk_acc),
        _p(gv_acc), _stream(stream)))


def pf_prefix_bwd_inject(desc, prefix_len, q_p, k_p, v_p, o_p, lse_p, do_p, gk_acc, gv_acc,
                         dq_p, dk_p, dv_p, dkv_dtype, workspace, stream=None):
    d, _keep = desc._c()
    ws, nws = _ws(workspace)
    _check(_lib.pf_prefix_bwd_inject(
        ctypes.byref(d), prefix_len, _t(q_p), _t(k_p), _t(v_p), _t(o_p), _p(lse_p), _t(do_p),
        _p(gk_acc), _p(gv_acc), _t(dq_p), _t(dk_p), _t(dv_p), dkv_dtype, ws, nws,
        _stream(stream)))


def pf_tree_attn_fwd(desc, node_off, parent, q, k, v, o, lse, workspace, stream=None):
    d, _keep = desc._c()
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_attn_fwd(ctypes.byref(d), len(pa), no_p, pa_p, _t(q), _t(k), _t(v), _t(o),
                                 _p(lse), ws, nws, _stream(stream)))


def pf_tree_attn_bwd(desc, node_off, parent, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                     stream=None):
    d, _keep = desc._c()
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_attn_bwd(ctypes.byref(d), len(pa), no_p, pa_p, _t(q), _t(k), _t(v), _t(o),
                                 _p(lse), _t(dout), _t(dq), _t(dk), _t(dv), ws, nws,
                                 _stream(stream)))


def pf_tree_suffix_attn_fwd(desc, prefix_len, k_p, v_p, node_off, parent, q, k, v, o, lse,
                            workspace, stream=None):
    d, _keep = desc._c()
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_suffix_attn_fwd(ctypes.byref(d), prefix_len, _t(k_p), _t(v_p), len(pa),
                                        no_p, pa_p, _t(q), _t(k), _t(v), _t(o), _p(lse), ws, nws,
                                        _stream(stream)))


def pf_tree_suffix_attn_bwd_accum(desc, prefix_len, k_p, v_p, node_off, parent, q, k, v, o, lse,
                                  dout, dq, dk, dv, gk_acc, gv_acc, workspace, stream=None):
    d, _keep = desc._c()
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_suffix_attn_bwd_accum(
        ctypes.byref(d), prefix_len, _t(k_p), _t(v_p), len(pa), no_p, pa_p, _t(q), _t(k), _t(v),
        _t(o), _p(lse), _t(dout), _t(dq), _t(dk), _t(dv), _p(gk_acc), _p(gv_acc), ws, nws,
        _stream(stream)))


def pf_ranges_cached_keys(range_len) -> int:
    ln, ln_p = _ints(range_len)
    n = int(_lib.pf_ranges_cached_keys(len(ln), ln_p))
    if n < 0:
        raise PFError(PF_ERR_INVALID_ARG, "invalid range lengths")
    return n


def pf_tree_suffix_attn_fwd_ranges(desc, k_c, v_c, range_start, range_len, node_off, parent, q, k,
                                   v, o, lse, workspace, stream=None):
    d, _keep = desc._c()
    rs, rs_p = _ints(range_start)
    rl, rl_p = _ints(range_len)
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_suffix_attn_fwd_ranges(
        ctypes.byref(d), k_c.shape[0], _t(k_c), _t(v_c), len(rs), rs_p, rl_p, len(pa), no_p, pa_p,
        _t(q), _t(k), _t(v), _t(o), _p(lse), ws, nws, _stream(stream)))


def pf_tree_suffix_attn_bwd_accum_ranges(desc, k_c, v_c, range_start, range_len, node_off, parent,
                                         q, k, v, o, lse, dout, dq, dk, dv, gk_acc, gv_acc,
                                         workspace, stream=None):
    d, _keep = desc._c()
    rs, rs_p = _ints(range_start)
    rl, rl_p = _ints(range_len)
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_suffix_attn_bwd_accum_ranges(
        ctypes.byref(d), k_c.shape[0], _t(k_c), _t(v_c), len(rs), rs_p, rl_p, len(pa), no_p, pa_p,
        _t(q), _t(k), _t(v), _t(o), _p(lse), _t(dout), _t(dq), _t(dk), _t(dv), _p(gk_acc),
        _p(gv_acc), ws, nws, _stream(stream)))


def pf_tree_attn_bwd_inject(desc, node_off, parent, q, k, v, o, lse, dout, gk_acc, gv_acc, dq, dk,
                            dv, dkv_dtype, workspace, stream=None):
    d, _keep = desc._c()
    no, no_p = _ints(node_off)
    pa, pa_p = _ints(parent)
    ws, nws = _ws(workspace)
    _check(_lib.pf_tree_attn_bwd_inject(
        ctypes.byref(d), len(pa), no_p, pa_p, _t(q), _t(k), _t(v), _t(o), _p(lse), _t(dout),
        _p(gk_acc), _p(gv_acc), _t(dq), _t(dk), _t(dv), dkv_dtype, ws, nws, _stream(stream)))


def _dtype_of(t):
    import torch
    return PF_BF16 if t.dtype == torch.bfloat16 else PF_F32


def pf_compact_logprob_fwd(z, row_ptr, pos, y, lse, logp, stream=None):
    """z [C, V] (bf16 or fp32, last dim contiguous); row_ptr [C+1], pos [S], y [S]
    int32 device tensors; lse [C], logp [S] fp32 outputs."""
    _check(_lib.pf_compact_logprob_fwd(z.shape[0], z.shape[1], _p(z), z.stride(0), _dtype_of(z),
                                       _p(row_ptr), _p(pos), _p(y), pos.shape[0], _p(lse),
                                       _p(logp), _stream(stream)))


def pf_compact_logprob_bwd(z, lse, row_ptr, pos, y, dlogp, dz, stream=None):
    _check(_lib.pf_compact_logprob_bwd(z.shape[0], z.shape[1], _p(z), z.stride(0), _dtype_of(z),
                                       _p(lse), _p(row_ptr), _p(pos), _p(y), pos.shape[0],
                                       _p(dlogp), _p(dz), dz.stride(0), _stream(stream)))


__all__ = [name for name in EXPORTED] + ["AttnDesc", "PFError", "PF_BF16", "PF_F32", "LIB_PATH"]
