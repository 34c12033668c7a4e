"""Out-of-bounds writes: every output and workspace buffer of every GPU entry point sits
between 64 KiB canary fills, and the fills must be untouched after the calls.  Entries
past a list's length (col_idx and row_idx beyond nnz), which the calls leave unwritten,
are canary-filled inside the buffers too.  Calls go through the C ABI directly, with
pointers into the padded buffers."""

import ctypes

import numpy as np
import pytest
import torch

from synthetic import make_layer_inputs
from block_sparse_attention_layer_amd import Problem, vmoba_num_blocks, vmoba_workspace_size
from block_sparse_attention_layer_amd._lib import check, lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD = 64 << 10
FILL = 0xA5


class Canaries:
    """Device buffers with PAD canary bytes on each side; view() hands out the middle."""

    def __init__(self):
        self.bufs = []

    def view(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((PAD + max(n, 1) + PAD,), FILL, dtype=torch.uint8, device=DEV)
        self.bufs.append((buf, n))
        return buf[PAD:PAD + n].view(dtype).view(shape)

    def intact(self):
        torch.cuda.synchronize()
        bad = []
        for i, (buf, n) in enumerate(self.bufs):
            lo, hi = buf[:PAD], buf[PAD + max(n, 1):]
            if not (bool((lo == FILL).all()) and bool((hi == FILL).all())):
                bad.append(i)
        return bad


def _p(x):
    return ctypes.c_void_p(x.data_ptr()) if x is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


# (name, T, H, W, heads, d, layer, block, batch): the 48-wide and split kernels (192-token
# blocks at d = 128), the 32-wide ones (d = 64, 216-token blocks), a 1D layer
CASES = [
    ("3d_192_d128", 8, 18, 32, 2, 128, 2, (4, 6, 8), 2),
    ("3d_216_d64", 6, 18, 16, 3, 64, 2, (3, 9, 8), 1),
    ("1d_d128", 6, 12, 16, 2, 128, 0, (2, 12, 16), 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_outputs_and_workspaces_stay_in_bounds(case):
    name, T, H, W, heads, d, layer, block, batch = case
    print(f"[canary {name}]", flush=True)
    inp = make_layer_inputs("l3d_55k", 0, backward=True, seed=77,
                            shape_override=dict(T=T, H=H, W=W, heads=heads, head_dim=d,
                                                batch=batch))
    bf = torch.bfloat16
    p = Problem(batch, heads, d, T, H, W, layer, block, bf, torch.float32)
    s = p.c_struct()
    sp = ctypes.byref(s)
    L = lib()
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    nb = vmoba_num_blocks(p)
    G = p.groups
    tok = (batch, p.L, heads, d)
    c = Canaries()
    i32, f32 = torch.int32, torch.float32

    qp, kp = c.view((batch, heads, nb, d), f32), c.view((batch, heads, nb, d), f32)
    check(L.vmoba_partition_pool(sp, _p(q), _p(k), _p(qp), _p(kp), _stream()), "pool")

    rp, cp = c.view((G, nb + 1), i32), c.view((G, nb + 1), i32)
    ci, ri = c.view((G, nb * nb), i32), c.view((G, nb * nb), i32)
    ci.view(torch.uint8).fill_(FILL)
    ri.view(torch.uint8).fill_(FILL)
    hs, ns = c.view((G, 4), f32), c.view((G, nb, nb), f32)
    nsel = vmoba_workspace_size(p, "select")
    ws = c.view((nsel,), torch.uint8)
    for mode in range(4):
        kk = max(1, nb * nb // 5) if mode == 1 else max(1, nb // 5)
        check(L.vmoba_select_mode(sp, _p(qp), _p(kp), mode, ctypes.c_float(0.25),
                                  ctypes.c_int32(kk), _p(rp), _p(ci), _p(cp), _p(ri), _p(hs),
                                  _p(ns), _p(ws), nsel, _stream()), f"select mode {mode}")
    # the strategies above wrote lists of other lengths: refill before the global one
    ci.view(torch.uint8).fill_(FILL)
    ri.view(torch.uint8).fill_(FILL)
    check(L.vmoba_select(sp, _p(qp), _p(kp), ctypes.c_float(0.25), _p(rp), _p(ci), _p(cp),
                         _p(ri), _p(hs), _p(ns), _p(ws), nsel, _stream()), "select")
    torch.cuda.synchronize()
    # list entries past each head's nnz keep the fill (the calls leave them unwritten)
    nnz = rp[:, -1].cpu().numpy()
    cib, rib = ci.cpu().numpy().view(np.uint8), ri.cpu().numpy().view(np.uint8)
    for g in range(G):
        assert (cib[g, 4 * nnz[g]:] == FILL).all() and (rib[g, 4 * nnz[g]:] == FILL).all()

    o, lse = c.view(tok, bf), c.view((batch, heads, p.L), f32)
    check(L.vmoba_sparse_attn_fwd(sp, _p(q), _p(k), _p(v), _p(rp), _p(ci), _p(o), _p(lse),
                                  ctypes.c_void_p(0), 0, _stream()), "sparse fwd")
    dq, dk, dv = c.view(tok, f32), c.view(tok, f32), c.view(tok, f32)
    nb_ws = vmoba_workspace_size(p, "sparse_bwd")
    wsb = c.view((nb_ws,), torch.uint8)
    check(L.vmoba_sparse_attn_bwd(sp, _p(q), _p(k), _p(v), _p(o), _p(lse), _p(do), _p(rp),
                                  _p(ci), _p(cp), _p(ri), _p(dq), _p(dk), _p(dv), _p(wsb),
                                  nb_ws, _stream()), "sparse bwd")
    check(L.vmoba_sparse_attn_bwd_noalloc(sp, _p(q), _p(k), _p(v), _p(o), _p(lse), _p(do),
                                          _p(rp), _p(ci), _p(cp), _p(ri), _p(dq), _p(dk),
                                          _p(dv), _stream()), "no-alloc bwd")
    od, lsed = c.view(tok, bf), c.view((batch, heads, p.L), f32)
    check(L.vmoba_dense_attn_fwd(sp, _p(q), _p(k), _p(v), _p(od), _p(lsed),
                                 ctypes.c_void_p(0), 0, _stream()), "dense fwd")
    check(L.vmoba_dense_attn_bwd(sp, _p(q), _p(k), _p(v), _p(od), _p(lsed), _p(do), _p(dq),
                                 _p(dk), _p(dv), _p(wsb), nb_ws, _stream()), "dense bwd")

    words = (nb + 31) // 32
    tm = c.view((G, p.L, words), i32)
    trp, tcp = c.view((G, nb + 1), i32), c.view((G, nb + 1), i32)
    tci, tri = c.view((G, nb * nb), i32), c.view((G, nb * nb), i32)
    ths = c.view((G, 4), f32)
    nts = vmoba_workspace_size(p, "select_tokens")
    wst = c.view((nts,), torch.uint8)
    check(L.vmoba_select_tokens(sp, _p(q), _p(kp), ctypes.c_float(0.25), _p(tm), _p(trp),
                                _p(tci), _p(tcp), _p(tri), _p(ths), _p(wst), nts, _stream()),
          "select tokens")
    ntf = vmoba_workspace_size(p, "token_fwd")
    wtf = c.view((ntf,), torch.uint8)
    ot, lset = c.view(tok, bf), c.view((batch, heads, p.L), f32)
    check(L.vmoba_token_attn_fwd(sp, _p(q), _p(k), _p(v), _p(trp), _p(tci), _p(tm), _p(ot),
                                 _p(lset), _p(wtf), ntf, _stream()), "token fwd")
    ntb = vmoba_workspace_size(p, "token_bwd")
    wtb = c.view((ntb,), torch.uint8)
    check(L.vmoba_token_attn_bwd(sp, _p(q), _p(k), _p(v), _p(ot), _p(lset), _p(do), _p(trp),
                                 _p(tci), _p(tcp), _p(tri), _p(tm), _p(dq), _p(dk), _p(dv),
                                 _p(wtb), ntb, _stream()), "token bwd")
    bad = c.intact()
    assert bad == [], f"canary bytes overwritten next to buffers {bad}"
    for t in (o, lse, dq, dk, dv, od, ot):
        assert torch.isfinite(t.float()).all()
