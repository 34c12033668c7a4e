"""Oracle: masked softmax attention, forward and backward (test infrastructure only).

papernotes 方法详解/整体框架 (the layer keeps full attention's input/output
contract and computes attention only on the selected blocks; the heads are
concatenated); paperlayer §3.1 (Fig. 2).

With M[x, y] = 1 iff (block(x), block(y)) is a selected pair:

    z_xy   = q_x . k_y / sqrt(d)                     (M = 1; -inf elsewhere)
    O_x    = sum_y softmax_y(z_x) v_y
    LSE_x  = ln sum_y exp(z_xy)

Backward (the pages never describe it; reading taken: the gradient of this
function with the mask held constant, i.e. selection is not differentiated):

    P      = exp(z - LSE)
    dV     = P^T dO
    dP     = dO V^T
    delta  = rowsum(dO * O)
    dS     = P * (dP - delta)
    dQ     = dS K / sqrt(d)
    dK     = dS^T Q / sqrt(d)

The block-sparse forms below evaluate only the selected key columns of each
query block; that is the same function, because exp(-inf) = 0.

Layouts: q, k, v, o, dO are [B, L, Hh, d]; LSE is [B, Hh, L]; block masks are
[B, Hh, N_b, N_b] bool with rows = query blocks, columns = key blocks.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def token_mask(block_mask_bh, blk_of_tok):
    """Token-level mask [L, L] of one (b, h) from its block mask [N_b, N_b]."""
    return block_mask_bh[np.ix_(blk_of_tok, blk_of_tok)]


def dense_masked_attention_fwd(q, k, v, tok_mask):
    """Literal L x L form.  tok_mask: [B, Hh, L, L] bool.  Returns (O, LSE)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hh, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, Hh, L))
    for b in range(B):
        for h in range(Hh):
            z = q[b, :, h, :] @ k[b, :, h, :].T / np.sqrt(d)
            z = np.where(tok_mask[b, h], z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            ssum = e.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (e / ssum) @ v[b, :, h, :]
            lse[b, h] = (m + np.log(ssum))[:, 0]
    return o, lse


def dense_masked_attention_bwd(q, k, v, o, lse, do, tok_mask):
    """Literal L x L backward.  Returns (dQ, dK, dV)."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    B, L, Hh, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sc = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(Hh):
            z = q[b, :, h, :] @ k[b, :, h, :].T * sc
            p = np.where(tok_mask[b, h], np.exp(z - lse[b, h][:, None]), 0.0)
            dv[b, :, h, :] = p.T @ do[b, :, h, :]
            dp = do[b, :, h, :] @ v[b, :, h, :].T
            delta = (do[b, :, h, :] * o[b, :, h, :]).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[b, :, h, :] = ds @ k[b, :, h, :] * sc
            dk[b, :, h, :] = ds.T @ q[b, :, h, :] * sc
    return dq, dk, dv


def _selected_keys(members, mask_row):
    """Concatenated token list of the selected key blocks (ascending block id)."""
    cols = np.nonzero(mask_row)[0]
    return members[cols].reshape(-1)


def sparse_attention_fwd(q, k, v, members, block_mask):
    """Block-sparse form: per query block, softmax over the selected key blocks only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hh, d = q.shape
    nb = members.shape[0]
    o = np.zeros_like(q)
    lse = np.zeros((B, Hh, L))
    sc = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(Hh):
            for i in range(nb):
                qi = members[i]
                keys = _selected_keys(members, block_mask[b, h, i])
                z = q[b, qi, h, :] @ k[b, keys, h, :].T * sc
                m = z.max(axis=1, keepdims=True)
                e = np.exp(z - m)
                ssum = e.sum(axis=1, keepdims=True)
                o[b, qi, h, :] = (e / ssum) @ v[b, keys, h, :]
                lse[b, h, qi] = (m + np.log(ssum))[:, 0]
    return o, lse


def sparse_attention_bwd(q, k, v, o, lse, do, members, block_mask):
    """Block-sparse backward (same definition as the dense one, selected columns only)."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    lse = _f64(lse)
    B, L, Hh, d = q.shape
    nb = members.shape[0]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sc = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(Hh):
            for i in range(nb):
                qi = members[i]
                keys = _selected_keys(members, block_mask[b, h, i])
                qq, oo, dd = q[b, qi, h, :], o[b, qi, h, :], do[b, qi, h, :]
                kk, vv = k[b, keys, h, :], v[b, keys, h, :]
                p = np.exp(qq @ kk.T * sc - lse[b, h, qi][:, None])
                dv[b, keys, h, :] += p.T @ dd
                dp = dd @ vv.T
                delta = (dd * oo).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, qi, h, :] = ds @ kk * sc
                dk[b, keys, h, :] += ds.T @ qq * sc
    return dq, dk, dv


def _row_softmax_pieces(qrows, kk, vv, sc):
    z = qrows @ kk.T * sc
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    ssum = e.sum(axis=1, keepdims=True)
    return z, (e / ssum) @ vv, (m + np.log(ssum))[:, 0]


def sampled_query_rows(q, k, v, do, members, block_of_tok, block_mask, b, h, rows):
    """O, LSE and (if ``do`` is given) dQ of a few query tokens of one (b, h).

    Each row is computed on its own from the definition, so this scales to any L.
    Returns dict with o [n, d], lse [n], dq [n, d] or None.
    """
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d)
    n = len(rows)
    out_o = np.zeros((n, d))
    out_lse = np.zeros(n)
    out_dq = np.zeros((n, d)) if do is not None else None
    for r, x in enumerate(rows):
        keys = _selected_keys(members, block_mask[b, h, block_of_tok[x]])
        kk, vv = _f64(k[b, keys, h, :]), _f64(v[b, keys, h, :])
        qx = _f64(q[b, x, h, :])[None, :]
        z, ox, lx = _row_softmax_pieces(qx, kk, vv, sc)
        out_o[r], out_lse[r] = ox[0], lx[0]
        if do is not None:
            dx = _f64(do[b, x, h, :])[None, :]
            p = np.exp(z - lx[:, None])
            dp = dx @ vv.T
            delta = (dx * ox).sum(axis=1)
            ds = p * (dp - delta[:, None])
            out_dq[r] = (ds @ kk * sc)[0]
    return {"o": out_o, "lse": out_lse, "dq": out_dq}


def sampled_key_block_grads(q, k, v, do, members, block_mask, b, h, j):
    """dK and dV of every token of key block ``j`` of one (b, h), from the definition.

    Visits each query block i that selected (i, j), recomputes its full softmax
    rows (over all of row i's selected key blocks) and accumulates the
    contribution of block j's columns.  Returns (dk [S, d], dv [S, d]).
    """
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d)
    kj = members[j]
    S = kj.size
    dk = np.zeros((S, d))
    dv = np.zeros((S, d))
    for i in np.nonzero(block_mask[b, h, :, j])[0]:
        qi = members[i]
        keys_blocks = np.nonzero(block_mask[b, h, i])[0]
        keys = members[keys_blocks].reshape(-1)
        pos = int(np.nonzero(keys_blocks == j)[0][0]) * S
        qq = _f64(q[b, qi, h, :])
        kk, vv = _f64(k[b, keys, h, :]), _f64(v[b, keys, h, :])
        dd = _f64(do[b, qi, h, :])
        z, oo, ll = _row_softmax_pieces(qq, kk, vv, sc)
        p = np.exp(z - ll[:, None])
        delta = (dd * oo).sum(axis=1)
        pj = p[:, pos:pos + S]
        dpj = dd @ vv[pos:pos + S].T
        dsj = pj * (dpj - delta[:, None])
        dv += pj.T @ dd
        dk += dsj.T @ qq * sc
    return dk, dv
