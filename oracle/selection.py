"""Oracle: global block selection with a cumulative-mass threshold (test infrastructure only).

papernotes 关键设计 2 and 3; paperlayer §3.3 (Fig. 4) and §3.4 (Fig. 5).

For every (batch, head) the query-block x key-block similarities form one
global pool.  The pool is normalised, sorted in descending order, and the
dynamic block count k is the smallest prefix length whose cumulative
normalised similarity is >= tau (the threshold equation of 关键设计 3).

Readings taken where the pages are silent or ambiguous:

* score scale 1/sqrt(d), matching the attention scale;
* the normaliser is a softmax over all N_b^2 entries of the head's pool (a
  plain sum is not defined for dot products of either sign);
* comparison ">=" as in the threshold equation (the prose says "exceeds");
* exact ties in the descending order are broken by ascending linear index
  i*N_b + j;
* after the prefix is taken, every query block also keeps its own key block
  (the diagonal), which does not count toward tau; this guarantees that no
  query row has an empty softmax;
* if rounding keeps the cumulative sum below tau, every pair is selected;
  tau >= 1 selects every pair.
"""

import numpy as np


def block_scores(q_pool, k_pool):
    """s[b,h,i,j] = <Qbar_i, Kbar_j> / sqrt(d), fp64.  q_pool, k_pool: [B, Hh, N_b, d]."""
    q_pool = np.asarray(q_pool, dtype=np.float64)
    k_pool = np.asarray(k_pool, dtype=np.float64)
    d = q_pool.shape[-1]
    return np.matmul(q_pool, np.swapaxes(k_pool, -1, -2)) / np.sqrt(d)


def normalise_per_head(s):
    """Softmax over all N_b*N_b entries of each (b, h) pool.  s: [B, Hh, N_b, N_b]."""
    s = np.asarray(s, dtype=np.float64)
    B, Hh, nb, _ = s.shape
    flat = s.reshape(B, Hh, nb * nb)
    e = np.exp(flat - flat.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).reshape(B, Hh, nb, nb)


def threshold_select(shat, tau):
    """Select pairs of one head.  shat: [N_b, N_b] normalised scores.

    Returns a dict with
      ``mask``  [N_b, N_b] bool, selected pairs (prefix union diagonal),
      ``k``     prefix length k*,
      ``v``     value of the k*-th largest entry (the cutoff v*),
      ``mass``  cumulative normalised similarity of the prefix,
      ``order`` linear indices in descending order (ties by ascending index).
    """
    shat = np.asarray(shat, dtype=np.float64)
    nb = shat.shape[0]
    n = nb * nb
    flat = shat.reshape(n)
    # stable sort of the negated values: descending, ties keep ascending index
    order = np.argsort(-flat, kind="stable")
    vals = flat[order]
    csum = np.cumsum(vals)  # sequential left-to-right fp64 sums
    if tau >= 1.0:
        k = n
    else:
        hit = np.nonzero(csum >= tau)[0]
        k = int(hit[0]) + 1 if hit.size else n
    mask = np.zeros(n, dtype=bool)
    mask[order[:k]] = True
    mask = mask.reshape(nb, nb)
    mask[np.arange(nb), np.arange(nb)] = True
    return {"mask": mask, "k": k, "v": float(vals[k - 1]),
            "mass": float(csum[k - 1]), "order": order}


def select_all_heads(q_pool, k_pool, tau):
    """Scores, normalisation and selection for every (b, h).

    Returns (mask [B,Hh,N_b,N_b] bool, shat [B,Hh,N_b,N_b], stats list of dicts
    with keys k, v, mass, nnz per (b, h) in row-major (b, h) order).
    """
    s = block_scores(q_pool, k_pool)
    shat = normalise_per_head(s)
    B, Hh, nb, _ = shat.shape
    mask = np.zeros((B, Hh, nb, nb), dtype=bool)
    stats = []
    for b in range(B):
        for h in range(Hh):
            r = threshold_select(shat[b, h], tau)
            mask[b, h] = r["mask"]
            stats.append({"k": r["k"], "v": r["v"], "mass": r["mass"],
                          "nnz": int(r["mask"].sum())})
    return mask, shat, stats


def mask_to_csr(mask):
    """Row-compressed form of a [G, N_b, N_b] mask: (row_ptr [G, N_b+1], col_idx [G, N_b*N_b]).

    Columns within a row are ascending; unused capacity is filled with -1.
    """
    mask = np.asarray(mask, dtype=bool)
    G, nb, _ = mask.shape
    row_ptr = np.zeros((G, nb + 1), dtype=np.int32)
    col_idx = np.full((G, nb * nb), -1, dtype=np.int32)
    for g in range(G):
        pos = 0
        for i in range(nb):
            cols = np.nonzero(mask[g, i])[0]
            col_idx[g, pos:pos + cols.size] = cols
            pos += cols.size
            row_ptr[g, i + 1] = pos
    return row_ptr, col_idx


def mask_to_csc(mask):
    """Column-compressed form: (col_ptr [G, N_b+1], row_idx [G, N_b*N_b]), rows ascending."""
    return mask_to_csr(np.swapaxes(np.asarray(mask, dtype=bool), -1, -2))
