"""Pins of the oracle's DiT block (CPU only).

- Gradients: autograd through the block (the oracle attention's own backward inside)
  against central finite differences along random directions, selection held fixed.
- Full-attention step: the block equals the same block with torch's fp64
  scaled_dot_product_attention (a library routine) in place of the attention.
- Head split: heads whose query and key projections are zero score every pair alike,
  so their output is the plain mean of the values over the selected key blocks; with
  the output projection the identity and the MLP zero this is read off the block output.
- Warm-up rule and layer cycle: the count of full steps and the partition per layer.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import dit as odit
from synthetic import make_dit_input, make_dit_params

LAT = (2, 4, 4)
HEADS, DIM, HID = 2, 8, 16
BLOCK3D = (1, 2, 2)


def _params(dim=DIM, hid=HID, n=1, seed=7000):
    return [{k: v.double() for k, v in p.items()} for p in make_dit_params(dim, hid, n, seed)]


def _x(dim=DIM, lat=LAT, seed=7100):
    x, g = make_dit_input(1, lat, dim, seed)
    return x.double(), g.double()


def test_block_gradients_match_finite_differences():
    P = _params()[0]
    x, g = _x()
    _, info = odit.dit_block(x, P, LAT, HEADS, 2, BLOCK3D)
    mask = info["mask"]
    assert mask.sum() < mask.size   # a sparse selection

    def f(xx, pp):
        y, _ = odit.dit_block(xx, pp, LAT, HEADS, 2, BLOCK3D, mask=mask)
        return float((y * g).sum())

    xr = x.clone().requires_grad_()
    Pr = {k: v.clone().requires_grad_() for k, v in P.items()}
    y, _ = odit.dit_block(xr, Pr, LAT, HEADS, 2, BLOCK3D, mask=mask)
    (y * g).sum().backward()
    rng = np.random.default_rng(3)
    h = 1e-6
    for name in ["x"] + sorted(P):
        base = x if name == "x" else P[name]
        grad = xr.grad if name == "x" else Pr[name].grad
        u = torch.from_numpy(rng.standard_normal(tuple(base.shape)))
        def shifted(s):
            if name == "x":
                return f(x + s * u, P)
            return f(x, {**P, name: P[name] + s * u})
        fd = (shifted(h) - shifted(-h)) / (2 * h)
        an = float((grad * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def _sdpa_block(x, P, heads):
    B, L, dim = x.shape
    d = dim // heads
    F = torch.nn.functional
    h = F.layer_norm(x, (dim,), eps=1e-6)
    split = lambda t: t.reshape(B, L, heads, d).transpose(1, 2)
    q, k, v = (split(h @ P[w].T + P[b]) for w, b in (("wq", "bq"), ("wk", "bk"), ("wv", "bv")))
    a = F.scaled_dot_product_attention(q, k, v).transpose(1, 2).reshape(B, L, dim)
    x = x + a @ P["wo"].T + P["bo"]
    h = F.layer_norm(x, (dim,), eps=1e-6)
    return x + F.gelu(h @ P["w1"].T + P["b1"], approximate="tanh") @ P["w2"].T + P["b2"]


def test_full_step_equals_library_attention():
    P = _params()[0]
    x, g = _x()
    x1 = x.clone().requires_grad_()
    x2 = x.clone().requires_grad_()
    y1, info = odit.dit_block(x1, P, LAT, HEADS, 2, BLOCK3D, full=True)
    y2 = _sdpa_block(x2, P, HEADS)
    assert torch.allclose(y1, y2, rtol=0, atol=1e-12)
    (y1 * g).sum().backward()
    (y2 * g).sum().backward()
    assert torch.allclose(x1.grad, x2.grad, rtol=0, atol=1e-11)
    assert info["mask"].all()


@pytest.mark.parametrize("layer,block", [(0, (1, 4, 4)), (1, (2, 2, 2)), (2, (1, 2, 2))])
def test_heads_with_zero_query_key_average_selected_values(layer, block):
    heads, d = 3, 4
    dim = heads * d
    P = _params(dim, 8)[0]
    for w, b in (("wq", "bq"), ("wk", "bk")):
        P[w][d:, :] = 0.0            # heads 1 and 2: q = k = 0
        P[b][d:] = 0.0
    P["wo"] = torch.eye(dim, dtype=torch.float64)
    for n in ("bo", "w1", "b1", "w2", "b2"):
        P[n] = torch.zeros_like(P[n])
    x, _ = _x(dim)
    y, info = odit.dit_block(x, P, LAT, heads, layer, block, tau=0.3)
    a = (y - x).reshape(1, -1, heads, d).numpy()
    h = torch.nn.functional.layer_norm(x, (dim,), eps=1e-6)
    v = (h @ P["wv"].T + P["bv"]).reshape(1, -1, heads, d).numpy()
    members, mask = info["members"], info["mask"]
    for hh in (1, 2):
        for i in range(members.shape[0]):
            keys = members[np.nonzero(mask[0, hh, i])[0]].reshape(-1)
            want = v[0, keys, hh, :].mean(axis=0)
            got = a[0, members[i], hh, :]
            assert np.abs(got - want[None, :]).max() <= 1e-12


def test_warmup_rule_counts():
    count = lambda n: sum(odit.full_attention_step(s, n) for s in range(n))
    assert count(50) == 13 and count(40) == 10 and count(4) == 1 and count(8) == 2
    assert odit.full_attention_step(0, 50) and odit.full_attention_step(12, 50)
    assert not odit.full_attention_step(13, 50)


def test_stack_cycles_partitions_and_switches_to_full():
    lat, dim = (2, 4, 4), DIM
    blocks = [(2, 4, 4), (2, 2, 2), (1, 2, 2)]    # 1D: 1 block, 2D: 4, 3D: 8
    P = _params(dim, HID, n=4)
    x, _ = _x(dim, lat)
    _, infos = odit.dit_stack(x, P, lat, HEADS, blocks, step=1, num_steps=4)
    assert [inf["members"].shape[0] for inf in infos] == [1, 4, 8, 1]
    _, infos = odit.dit_stack(x, P, lat, HEADS, blocks, step=0, num_steps=4)
    assert all(inf["mask"].all() and inf["members"].shape == (1, 32) for inf in infos)
