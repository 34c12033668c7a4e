"""Python binding with the names of the C ABI (include/vmoba.h).

Each function checks tensor devices, dtypes, shapes and contiguity, allocates the
outputs and the workspace with torch (device memory plumbing), and passes raw
pointers and the current HIP stream to libvmoba.so.  All arithmetic runs in the
library's kernels.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from ._lib import CProblem, OPS, VMOBA_BF16, VMOBA_FP32, check, lib

_DTYPE_CODE = {torch.bfloat16: VMOBA_BF16, torch.float32: VMOBA_FP32}


@dataclass(frozen=True)
class Problem:
    """One layer: batch, heads, head_dim, latent (T, H, W), layer index, block shape."""
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    layer_idx: int
    block: Tuple[int, int, int]
    dtype: torch.dtype = torch.bfloat16
    grad_dtype: Optional[torch.dtype] = None   # dQ/dK/dV type; default: dtype

    @property
    def gdtype(self):
        return self.dtype if self.grad_dtype is None else self.grad_dtype

    @property
    def L(self):
        return self.T * self.H * self.W

    @property
    def groups(self):
        return self.batch * self.heads

    def c_struct(self):
        bt, bh, bw = self.block
        return CProblem(self.batch, self.heads, self.head_dim, self.T, self.H, self.W,
                        self.layer_idx, bt, bh, bw,
                        _DTYPE_CODE.get(self.dtype, 99), _DTYPE_CODE.get(self.gdtype, 99))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _want(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def vmoba_validate(p: Problem) -> int:
    s = p.c_struct()
    return lib().vmoba_validate(ctypes.byref(s))


def vmoba_num_blocks(p: Problem) -> int:
    s = p.c_struct()
    nb = ctypes.c_int32(0)
    check(lib().vmoba_num_blocks(ctypes.byref(s), ctypes.byref(nb)), "vmoba_num_blocks")
    return nb.value


def vmoba_workspace_size(p: Problem, op: str) -> int:
    s = p.c_struct()
    n = ctypes.c_size_t(0)
    check(lib().vmoba_workspace_size(ctypes.byref(s), OPS[op], ctypes.byref(n)),
          "vmoba_workspace_size")
    return n.value


def _workspace(p, op, device):
    n = vmoba_workspace_size(p, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def _tok_shape(p):
    return (p.batch, p.L, p.heads, p.head_dim)


def vmoba_partition_pool(p: Problem, q, k, q_pool=None, k_pool=None):
    """Block means of Q and K: returns fp32 (q_pool, k_pool) [B, Hh, N_b, d]."""
    dev = q.device
    _want(q, "q", _tok_shape(p), p.dtype, dev)
    _want(k, "k", _tok_shape(p), p.dtype, dev)
    nb = vmoba_num_blocks(p)
    shp = (p.batch, p.heads, nb, p.head_dim)
    q_pool = torch.empty(shp, dtype=torch.float32, device=dev) if q_pool is None else q_pool
    k_pool = torch.empty(shp, dtype=torch.float32, device=dev) if k_pool is None else k_pool
    _want(q_pool, "q_pool", shp, torch.float32, dev)
    _want(k_pool, "k_pool", shp, torch.float32, dev)
    s = p.c_struct()
    check(lib().vmoba_partition_pool(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(q_pool),
                                     _ptr(k_pool), _stream(dev)), "vmoba_partition_pool")
    return q_pool, k_pool


@dataclass
class Selection:
    """Selected block pairs of every head group g = b*Hh + h (device tensors)."""
    row_ptr: torch.Tensor      # int32 [G, N_b+1]
    col_idx: torch.Tensor      # int32 [G, N_b*N_b]
    col_ptr: torch.Tensor      # int32 [G, N_b+1]
    row_idx: torch.Tensor      # int32 [G, N_b*N_b]
    head_stats: torch.Tensor   # fp32 [G, 4]: k*, nnz, prefix mass, cutoff score
    norm_scores: Optional[torch.Tensor] = None  # fp32 [G, N_b, N_b]


SELECTION_MODES = {"threshold_global": 0, "topk_global": 1, "threshold_local": 2,
                   "topk_local": 3}


def vmoba_select(p: Problem, q_pool, k_pool, tau: float = None, want_scores=False,
                 mode: str = "threshold_global", k: int = None) -> Selection:
    """Block selection.  mode "threshold_global" (the default, tau) is vmoba_select; the
    other SELECTION_MODES go through vmoba_select_mode (tau for threshold_local, k for the
    top-k modes)."""
    if mode not in SELECTION_MODES:
        raise ValueError(f"unknown selection mode {mode!r}")
    dev = q_pool.device
    nb = vmoba_num_blocks(p)
    G = p.groups
    shp = (p.batch, p.heads, nb, p.head_dim)
    _want(q_pool, "q_pool", shp, torch.float32, dev)
    _want(k_pool, "k_pool", shp, torch.float32, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    sel = Selection(
        row_ptr=torch.empty((G, nb + 1), **i32), col_idx=torch.empty((G, nb * nb), **i32),
        col_ptr=torch.empty((G, nb + 1), **i32), row_idx=torch.empty((G, nb * nb), **i32),
        head_stats=torch.empty((G, 4), dtype=torch.float32, device=dev),
        norm_scores=(torch.empty((G, nb, nb), dtype=torch.float32, device=dev)
                     if want_scores else None))
    ws, n = _workspace(p, "select", dev)
    s = p.c_struct()
    if mode == "threshold_global":
        check(lib().vmoba_select(ctypes.byref(s), _ptr(q_pool), _ptr(k_pool),
                                 ctypes.c_float(tau), _ptr(sel.row_ptr), _ptr(sel.col_idx),
                                 _ptr(sel.col_ptr), _ptr(sel.row_idx), _ptr(sel.head_stats),
                                 _ptr(sel.norm_scores), _ptr(ws), n, _stream(dev)),
              "vmoba_select")
    else:
        check(lib().vmoba_select_mode(ctypes.byref(s), _ptr(q_pool), _ptr(k_pool),
                                      SELECTION_MODES[mode],
                                      ctypes.c_float(0.0 if tau is None else tau),
                                      ctypes.c_int32(0 if k is None else int(k)),
                                      _ptr(sel.row_ptr), _ptr(sel.col_idx), _ptr(sel.col_ptr),
                                      _ptr(sel.row_idx), _ptr(sel.head_stats),
                                      _ptr(sel.norm_scores), _ptr(ws), n, _stream(dev)),
              "vmoba_select_mode")
    return sel


def _check_lists(p, dev, *lists):
    nb = vmoba_num_blocks(p)
    G = p.groups
    for name, t, width in lists:
        _want(t, name, (G, width(nb)), torch.int32, dev)


def vmoba_sparse_attn_fwd(p: Problem, q, k, v, row_ptr, col_idx, o=None, lse=None):
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n))
    o = torch.empty(_tok_shape(p), dtype=p.dtype, device=dev) if o is None else o
    lse = torch.empty((p.batch, p.heads, p.L), dtype=torch.float32, device=dev) if lse is None else lse
    _want(o, "o", _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    ws, n = _workspace(p, "sparse_fwd", dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse),
                                      _ptr(ws), n, _stream(dev)), "vmoba_sparse_attn_fwd")
    return o, lse


def vmoba_sparse_attn_bwd(p: Problem, q, k, v, o, lse, dout, row_ptr, col_idx, col_ptr,
                          row_idx, dq=None, dk=None, dv=None):
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n),
                 ("col_ptr", col_ptr, lambda n: n + 1),
                 ("row_idx", row_idx, lambda n: n * n))
    outs = [torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if t is None else t
            for t in (dq, dk, dv)]
    for name, t in zip(("dq", "dk", "dv"), outs):
        _want(t, name, _tok_shape(p), p.gdtype, dev)
    ws, n = _workspace(p, "sparse_bwd", dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(lse), _ptr(dout), _ptr(row_ptr), _ptr(col_idx),
                                      _ptr(col_ptr), _ptr(row_idx), _ptr(outs[0]),
                                      _ptr(outs[1]), _ptr(outs[2]), _ptr(ws), n,
                                      _stream(dev)), "vmoba_sparse_attn_bwd")
    return tuple(outs)


def vmoba_sparse_attn_bwd_noalloc(p: Problem, q, k, v, o, lse, dout, row_ptr, col_idx,
                                  col_ptr, row_idx, dq, dk, dv):
    """vmoba_sparse_attn_bwd into caller-allocated dq, dk, dv with no workspace: the
    library keeps delta in a fixed per-GPU device array, and this call allocates nothing."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n),
                 ("col_ptr", col_ptr, lambda n: n + 1),
                 ("row_idx", row_idx, lambda n: n * n))
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _want(t, name, _tok_shape(p), p.gdtype, dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_bwd_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(o), _ptr(lse), _ptr(dout), _ptr(row_ptr),
                                              _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
                                              _ptr(dq), _ptr(dk), _ptr(dv), _stream(dev)),
          "vmoba_sparse_attn_bwd_noalloc")
    return dq, dk, dv


def vmoba_sparse_attn_bwd_delta(p: Problem, o, dout, delta=None):
    dev = o.device
    _want(o, "o", _tok_shape(p), p.dtype, dev)
    _want(dout, "dout", _tok_shape(p), p.dtype, dev)
    delta = torch.empty((p.batch, p.heads, p.L), dtype=torch.float32, device=dev) if delta is None else delta
    _want(delta, "delta", (p.batch, p.heads, p.L), torch.float32, dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_bwd_delta(ctypes.byref(s), _ptr(o), _ptr(dout), _ptr(delta),
                                            _stream(dev)), "vmoba_sparse_attn_bwd_delta")
    return delta


def _bwd_inputs(p, dev, q, k, v, lse, delta, dout):
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    _want(delta, "delta", (p.batch, p.heads, p.L), torch.float32, dev)


def vmoba_sparse_attn_bwd_dkdv(p: Problem, q, k, v, lse, delta, dout, col_ptr, row_idx,
                               dk=None, dv=None):
    dev = q.device
    _bwd_inputs(p, dev, q, k, v, lse, delta, dout)
    _check_lists(p, dev, ("col_ptr", col_ptr, lambda n: n + 1),
                 ("row_idx", row_idx, lambda n: n * n))
    dk = torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if dk is None else dk
    dv = torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if dv is None else dv
    _want(dk, "dk", _tok_shape(p), p.gdtype, dev)
    _want(dv, "dv", _tok_shape(p), p.gdtype, dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_bwd_dkdv(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(lse), _ptr(delta), _ptr(dout), _ptr(col_ptr),
                                           _ptr(row_idx), _ptr(dk), _ptr(dv), _stream(dev)),
          "vmoba_sparse_attn_bwd_dkdv")
    return dk, dv


def vmoba_sparse_attn_bwd_dq(p: Problem, q, k, v, lse, delta, dout, row_ptr, col_idx,
                             dq=None):
    dev = q.device
    _bwd_inputs(p, dev, q, k, v, lse, delta, dout)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n))
    dq = torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if dq is None else dq
    _want(dq, "dq", _tok_shape(p), p.gdtype, dev)
    s = p.c_struct()
    check(lib().vmoba_sparse_attn_bwd_dq(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(lse),
                                         _ptr(delta), _ptr(dout), _ptr(row_ptr),
                                         _ptr(col_idx), _ptr(dq), _stream(dev)),
          "vmoba_sparse_attn_bwd_dq")
    return dq


def vmoba_dense_attn_fwd(p: Problem, q, k, v, o=None, lse=None):
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    o = torch.empty(_tok_shape(p), dtype=p.dtype, device=dev) if o is None else o
    lse = torch.empty((p.batch, p.heads, p.L), dtype=torch.float32, device=dev) if lse is None else lse
    ws, n = _workspace(p, "dense_fwd", dev)
    s = p.c_struct()
    check(lib().vmoba_dense_attn_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), _ptr(ws), n, _stream(dev)),
          "vmoba_dense_attn_fwd")
    return o, lse


def vmoba_dense_attn_bwd(p: Problem, q, k, v, o, lse, dout, dq=None, dk=None, dv=None):
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    outs = [torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if t is None else t
            for t in (dq, dk, dv)]
    for name, t in zip(("dq", "dk", "dv"), outs):
        _want(t, name, _tok_shape(p), p.gdtype, dev)
    ws, n = _workspace(p, "dense_bwd", dev)
    s = p.c_struct()
    check(lib().vmoba_dense_attn_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), _ptr(dout), _ptr(outs[0]), _ptr(outs[1]),
                                     _ptr(outs[2]), _ptr(ws), n, _stream(dev)),
          "vmoba_dense_attn_bwd")
    return tuple(outs)


@dataclass
class TokenSelection:
    """Token-granular selection of every head group g = b*Hh + h (device tensors)."""
    token_mask: torch.Tensor   # int32 bits [G, L, ceil(N_b/32)]: bit j%32 of word j//32
    row_ptr: torch.Tensor      # union lists per query block (CSR), int32 [G, N_b+1]
    col_idx: torch.Tensor      # int32 [G, N_b*N_b]
    col_ptr: torch.Tensor      # and per key block (CSC)
    row_idx: torch.Tensor
    head_stats: torch.Tensor   # fp32 [G, 4]: k*, selected (token, block) pairs, mass, cutoff


def _mask_shape(p, nb):
    return (p.groups, p.L, (nb + 31) // 32)


def vmoba_select_tokens(p: Problem, q, k_pool, tau: float) -> TokenSelection:
    """Token-granular selection: the pool of a head is every (query token, key block)
    pair; q [B, L, Hh, d] bf16, k_pool from vmoba_partition_pool."""
    dev = q.device
    nb = vmoba_num_blocks(p)
    G = p.groups
    _want(q, "q", _tok_shape(p), p.dtype, dev)
    _want(k_pool, "k_pool", (p.batch, p.heads, nb, p.head_dim), torch.float32, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    sel = TokenSelection(
        token_mask=torch.empty(_mask_shape(p, nb), **i32),
        row_ptr=torch.empty((G, nb + 1), **i32), col_idx=torch.empty((G, nb * nb), **i32),
        col_ptr=torch.empty((G, nb + 1), **i32), row_idx=torch.empty((G, nb * nb), **i32),
        head_stats=torch.empty((G, 4), dtype=torch.float32, device=dev))
    ws, n = _workspace(p, "select_tokens", dev)
    s = p.c_struct()
    check(lib().vmoba_select_tokens(ctypes.byref(s), _ptr(q), _ptr(k_pool), ctypes.c_float(tau),
                                    _ptr(sel.token_mask), _ptr(sel.row_ptr), _ptr(sel.col_idx),
                                    _ptr(sel.col_ptr), _ptr(sel.row_idx), _ptr(sel.head_stats),
                                    _ptr(ws), n, _stream(dev)), "vmoba_select_tokens")
    return sel


def vmoba_token_attn_fwd(p: Problem, q, k, v, row_ptr, col_idx, token_mask, o=None, lse=None):
    dev = q.device
    nb = vmoba_num_blocks(p)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n))
    _want(token_mask, "token_mask", _mask_shape(p, nb), torch.int32, dev)
    o = torch.empty(_tok_shape(p), dtype=p.dtype, device=dev) if o is None else o
    lse = torch.empty((p.batch, p.heads, p.L), dtype=torch.float32, device=dev) if lse is None else lse
    _want(o, "o", _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    ws, n = _workspace(p, "token_fwd", dev)
    s = p.c_struct()
    check(lib().vmoba_token_attn_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                     _ptr(col_idx), _ptr(token_mask), _ptr(o), _ptr(lse),
                                     _ptr(ws), n, _stream(dev)), "vmoba_token_attn_fwd")
    return o, lse


def vmoba_token_attn_bwd(p: Problem, q, k, v, o, lse, dout, row_ptr, col_idx, col_ptr,
                         row_idx, token_mask, dq=None, dk=None, dv=None):
    dev = q.device
    nb = vmoba_num_blocks(p)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, name, _tok_shape(p), p.dtype, dev)
    _want(lse, "lse", (p.batch, p.heads, p.L), torch.float32, dev)
    _check_lists(p, dev, ("row_ptr", row_ptr, lambda n: n + 1),
                 ("col_idx", col_idx, lambda n: n * n),
                 ("col_ptr", col_ptr, lambda n: n + 1),
                 ("row_idx", row_idx, lambda n: n * n))
    _want(token_mask, "token_mask", _mask_shape(p, nb), torch.int32, dev)
    outs = [torch.empty(_tok_shape(p), dtype=p.gdtype, device=dev) if t is None else t
            for t in (dq, dk, dv)]
    for name, t in zip(("dq", "dk", "dv"), outs):
        _want(t, name, _tok_shape(p), p.gdtype, dev)
    ws, n = _workspace(p, "token_bwd", dev)
    s = p.c_struct()
    check(lib().vmoba_token_attn_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), _ptr(dout), _ptr(row_ptr), _ptr(col_idx),
                                     _ptr(col_ptr), _ptr(row_idx), _ptr(token_mask),
                                     _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(ws), n,
                                     _stream(dev)), "vmoba_token_attn_bwd")
    return tuple(outs)
