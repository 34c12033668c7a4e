"""Oracle: the token-granular query pool (test infrastructure only).

papernotes 关键设计 2 writes the selection of one head as a mask over its query x key-block
products, with q_i the head's queries (all s of them, s x d) and b_i its key blocks
(N_b x d).  Read literally, the pool of a head is every (query token, key block) pair:
L x N_b entries, and papernotes 关键设计 3's threshold runs over that pool.  (The default
reading, block_scores / threshold_select, pools the queries of a block first.)

Readings, carried over from the block-granular selection:

* score s[x, j] = q_x . Kbar_j / sqrt(d) (Kbar_j the block mean of the keys);
* Shat = softmax over all L * N_b entries of the head;
* descending order with ties by ascending linear index x * N_b + j; the prefix is the
  shortest one whose running sum is >= tau (tau >= 1, or a sum that never reaches tau,
  takes the whole pool);
* every token also keeps its own block (x, block(x)), which does not count toward tau;
* token x attends to the tokens of its selected key blocks:
  M[x, y] = 1 iff (x, block(y)) is selected.  The forward and backward are those of the
  block-granular layer (masked softmax attention, mask held constant).
"""

import numpy as np

from .attention import dense_masked_attention_bwd, dense_masked_attention_fwd
from .selection import _ordered_prefix


def token_scores(q, k_pool):
    """s[b,h,x,j] = <q_x, Kbar_j> / sqrt(d), fp64.  q: [B,L,Hh,d]; k_pool: [B,Hh,N_b,d]."""
    q = np.asarray(q, dtype=np.float64)
    kp = np.asarray(k_pool, dtype=np.float64)
    d = q.shape[-1]
    return np.matmul(np.transpose(q, (0, 2, 1, 3)), np.swapaxes(kp, -1, -2)) / np.sqrt(d)


def normalise_token_pool(s):
    """Softmax over all L*N_b entries of each (b, h).  s: [B, Hh, L, N_b]."""
    s = np.asarray(s, dtype=np.float64)
    B, Hh, L, nb = s.shape
    flat = s.reshape(B, Hh, L * nb)
    e = np.exp(flat - flat.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).reshape(B, Hh, L, nb)


def token_select(shat, tau, blk_of_tok):
    """Select (token, key block) pairs of one head.  shat: [L, N_b] normalised over the
    whole pool; blk_of_tok: [L] block of every token.  Returns a dict with ``mask``
    [L, N_b] bool, ``k`` (prefix length), ``v`` (cutoff value), ``mass`` (prefix mass)."""
    shat = np.asarray(shat, dtype=np.float64)
    L, nb = shat.shape
    flat = shat.reshape(L * nb)
    order, k = _ordered_prefix(flat, tau=tau)
    mask = np.zeros(L * nb, dtype=bool)
    mask[order[:k]] = True
    mask = mask.reshape(L, nb)
    mask[np.arange(L), np.asarray(blk_of_tok)] = True
    vals = flat[order]
    return {"mask": mask, "k": k, "v": float(vals[k - 1]), "mass": float(vals[:k].sum())}


def select_tokens_all_heads(q, k_pool, tau, blk_of_tok):
    """Token pools of every (b, h).  Returns (mask [B,Hh,L,N_b] bool, shat [B,Hh,L,N_b],
    stats list of dicts k, v, mass, nnz in row-major (b, h) order)."""
    shat = normalise_token_pool(token_scores(q, k_pool))
    B, Hh, L, nb = shat.shape
    mask = np.zeros((B, Hh, L, nb), dtype=bool)
    stats = []
    for b in range(B):
        for h in range(Hh):
            r = token_select(shat[b, h], tau, blk_of_tok)
            mask[b, h] = r["mask"]
            stats.append({"k": r["k"], "v": r["v"], "mass": r["mass"],
                          "nnz": int(r["mask"].sum())})
    return mask, shat, stats


def union_block_mask(tok_mask, members):
    """Block mask [B,Hh,N_b,N_b]: query block i lists key block j iff some token of block i
    selected j (the lists a caller hands to the attention together with the token mask)."""
    tok_mask = np.asarray(tok_mask, dtype=bool)
    B, Hh, L, nb = tok_mask.shape
    out = np.zeros((B, Hh, nb, nb), dtype=bool)
    for i in range(members.shape[0]):
        out[:, :, i, :] = tok_mask[:, :, members[i], :].any(axis=2)
    return out


def token_level_mask(tok_mask, blk_of_tok):
    """[B,Hh,L,L] mask M[x, y] = tok_mask[x, block(y)]."""
    return np.asarray(tok_mask, dtype=bool)[:, :, :, np.asarray(blk_of_tok)]


def token_attention_fwd(q, k, v, tok_mask, blk_of_tok):
    """O, LSE of the token-granular selection (literal L x L form)."""
    return dense_masked_attention_fwd(q, k, v, token_level_mask(tok_mask, blk_of_tok))


def token_attention_bwd(q, k, v, o, lse, do, tok_mask, blk_of_tok):
    return dense_masked_attention_bwd(q, k, v, o, lse, do,
                                      token_level_mask(tok_mask, blk_of_tok))


def sampled_token_rows(q, k, v, do, tok_mask, members, blk_of_tok, b, h, rows):
    """O, LSE and dQ of the query tokens ``rows`` of one (b, h), each over the keys of its
    own selected blocks (for checks at sizes where the L x L form is too large)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d)
    out = []
    for x in rows:
        cols = np.nonzero(tok_mask[b, h, x])[0]
        keys = members[cols].reshape(-1)
        z = k[b, keys, h, :] @ q[b, x, h, :] * sc
        m = z.max()
        e = np.exp(z - m)
        ssum = e.sum()
        p = e / ssum
        o = p @ v[b, keys, h, :]
        dp = v[b, keys, h, :] @ do[b, x, h, :]
        ds = p * (dp - float(do[b, x, h, :] @ o))
        dq = ds @ k[b, keys, h, :] * sc
        out.append({"o": o, "lse": m + np.log(ssum), "dq": dq})
    return out
