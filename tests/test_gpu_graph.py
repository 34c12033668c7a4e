"""The whole step (pool, select, forward, backward) captured in one HIP graph.

The library allocates nothing and issues no memset (its selection clears its tables with
a fill kernel), and the backward's second stream is made on an eager call before the
capture, so a caller can capture a step and replay it.  Every
kernel is deterministic (the selection's atomics add integers), so each replay must
reproduce the eager step bit for bit.  Replays alternate with eager steps on the same
buffers' neighbours, and every replay is checked.
"""

import pytest
import torch

from synthetic import make_layer_inputs
from block_sparse_attention_layer_amd import (
    Problem, vmoba_partition_pool, vmoba_select, vmoba_select_tokens, vmoba_sparse_attn_bwd,
    vmoba_sparse_attn_fwd, vmoba_token_attn_bwd, vmoba_token_attn_fwd)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(T=8, H=12, W=16, block=(4, 6, 8), heads=3):
    over = dict(T=T, H=H, W=W, heads=heads, head_dim=128, batch=1)
    inp = make_layer_inputs("l3d_55k", 0, backward=True, shape_override=over, dtype="bf16")
    p = Problem(1, heads, 128, T, H, W, 2, block, torch.bfloat16, torch.bfloat16)
    return p, {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}


def _block_step(p, d):
    qp, kp = vmoba_partition_pool(p, d["q"], d["k"])
    sel = vmoba_select(p, qp, kp, 0.25)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx)
    dq, dk, dv = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], sel.row_ptr,
                                       sel.col_idx, sel.col_ptr, sel.row_idx)
    return [sel.row_ptr, sel.col_idx, sel.col_ptr, sel.row_idx, sel.head_stats, o, lse, dq,
            dk, dv]


def _token_step(p, d):
    _, kp = vmoba_partition_pool(p, d["q"], d["k"])
    sel = vmoba_select_tokens(p, d["q"], kp, 0.25)
    o, lse = vmoba_token_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx,
                                  sel.token_mask)
    dq, dk, dv = vmoba_token_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], sel.row_ptr,
                                      sel.col_idx, sel.col_ptr, sel.row_idx, sel.token_mask)
    return [sel.token_mask, sel.row_ptr, sel.col_idx, sel.head_stats, o, lse, dq, dk, dv]


def _canon(outs, lists):
    """Outputs with each index list cut to its written length (entries past a head group's
    last offset are left unwritten by the library)."""
    out = []
    for i, t in enumerate(outs):
        if i in lists:
            ptr = outs[lists[i]]
            out.append([t[g, :int(ptr[g, -1])].clone() for g in range(t.shape[0])])
        else:
            out.append(t.clone())
    return out


def _same(a, b):
    if isinstance(a, list):
        return all(torch.equal(x, y) for x, y in zip(a, b))
    return torch.equal(a, b)


def _check_graph(step, p, d, lists):
    eager = _canon(step(p, d), lists)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(p, d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(p, d)
    for rep in range(4):
        for t in outs:
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_canon(outs, lists), eager)):
            assert _same(a, b), (rep, i)
        again = _canon(step(p, d), lists)        # eager work between the replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(again, eager)):
            assert _same(a, b), (rep, i)


def test_block_step_graph_replays_match_eager():
    print("[graph: block-granular step, 1536 tokens, 3 heads]", flush=True)
    p, d = _inputs()
    _check_graph(_block_step, p, d, {1: 0, 3: 2})


def test_large_pool_step_graph_replays_match_eager():
    print("[graph: block-granular step with the pool passes, 384 blocks]", flush=True)
    p, d = _inputs(T=8, H=12, W=32, block=(2, 2, 2), heads=2)
    _check_graph(_block_step, p, d, {1: 0, 3: 2})


def test_token_step_graph_replays_match_eager():
    print("[graph: token-granular step]", flush=True)
    p, d = _inputs()
    _check_graph(_token_step, p, d, {2: 1})
