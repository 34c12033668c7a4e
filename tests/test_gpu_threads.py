"""The fused backward called from several host threads.

vmoba_sparse_attn_bwd runs its dQ pass on a second stream of the device, one per calling
host thread, forked from the caller's stream and joined back.  Every kernel is
deterministic, so each thread's gradients must equal the single-thread result bit for
bit:
- threads that call it at the same time, each on a stream of its own;
- a thread whose first call is captured into a graph (the second stream is not made
  during a capture, so that call runs its passes one after the other), replayed, and then
  called eagerly.
"""

import threading

import pytest
import torch

from synthetic import make_layer_inputs
from block_sparse_attention_layer_amd import (
    Problem, vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd, vmoba_sparse_attn_fwd)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _problem(T=8, H=12, W=16, block=(4, 6, 8), heads=3):
    over = dict(T=T, H=H, W=W, heads=heads, head_dim=128, batch=1)
    inp = make_layer_inputs("l3d_55k", 0, backward=True, shape_override=over, dtype="bf16",
                            seed=21)
    p = Problem(1, heads, 128, T, H, W, 2, block, torch.bfloat16, torch.float32)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    qp, kp = vmoba_partition_pool(p, d["q"], d["k"])
    sel = vmoba_select(p, qp, kp, 0.25)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx)
    args = (p, d["q"], d["k"], d["v"], o, lse, d["do"], sel.row_ptr, sel.col_idx,
            sel.col_ptr, sel.row_idx)
    torch.cuda.synchronize()
    return args


def _run_threads(target, n):
    errors = []

    def wrap(i):
        try:
            target(i)
        except BaseException as e:   # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=wrap, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_fused_backward_from_concurrent_threads():
    print("[threads: fused backward, 4 threads x 3 calls, 1536 tokens, 3 heads]", flush=True)
    args = _problem()
    ref = [t.clone() for t in vmoba_sparse_attn_bwd(*args)]
    torch.cuda.synchronize()
    results = {}

    def work(i):
        s = torch.cuda.Stream(device=DEV)
        outs = []
        with torch.cuda.stream(s):
            for _ in range(3):
                outs.append(vmoba_sparse_attn_bwd(*args))
        s.synchronize()
        results[i] = outs

    _run_threads(work, 4)
    for i in range(4):
        for c, outs in enumerate(results[i]):
            for name, a, b in zip(("dq", "dk", "dv"), outs, ref):
                assert torch.equal(a, b), (i, c, name)


def test_first_call_of_a_thread_under_capture():
    print("[threads: a thread's first fused backward captured in a graph]", flush=True)
    args = _problem(T=8, H=12, W=32, heads=2)
    ref = [t.clone() for t in vmoba_sparse_attn_bwd(*args)]
    torch.cuda.synchronize()
    state = {}

    def work(_):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            outs = vmoba_sparse_attn_bwd(*args)
        replays = []
        for _ in range(3):
            for t in outs:
                t.fill_(0)
            graph.replay()
            torch.cuda.synchronize()
            replays.append([t.clone() for t in outs])
        eager = vmoba_sparse_attn_bwd(*args)   # this thread's second stream is made here
        torch.cuda.synchronize()
        state["replays"], state["eager"] = replays, eager

    _run_threads(work, 1)
    for r, outs in enumerate(state["replays"] + [state["eager"]]):
        for name, a, b in zip(("dq", "dk", "dv"), outs, ref):
            assert torch.equal(a, b), (r, name)
