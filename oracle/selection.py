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

The ablation of paperlayer §4.4 (Table 3) and papernotes' ablation table also name three
other selection strategies, each dropping one or both of the two ingredients:

* top-k + global: a fixed number k of pairs from the head's global pool instead of the
  threshold;
* threshold + local: no global pool; every query block chooses its own key blocks, the
  threshold rule applied to that query block's row of scores;
* top-k + local: every query block takes its k highest-scoring key blocks (MoBA's rule).

The pages give no formula for them beyond that contrast.  Readings taken: a local pool
is normalised by a softmax over its own row (the row's share of mass, so that tau keeps
its meaning of a retained fraction); k counts pairs of the pool (k pairs per head for
global, k key blocks per query block for local) and is clamped to the pool size; order,
ties and the forced diagonal are as for the global threshold rule.
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


def _ordered_prefix(vals, tau=None, k=None):
    """Order a 1-D pool descending (ties by ascending index) and cut a prefix: the smallest
    one whose running sum is >= tau (tau >= 1, or a sum that never reaches tau, takes the
    whole pool), or the first k entries (k clamped to the pool).  Returns (order, length)."""
    vals = np.asarray(vals, dtype=np.float64)
    n = vals.size
    order = np.argsort(-vals, kind="stable")
    if k is not None:
        return order, int(min(max(int(k), 0), n))
    if tau >= 1.0:
        return order, n
    hit = np.nonzero(np.cumsum(vals[order]) >= tau)[0]
    return order, (int(hit[0]) + 1 if hit.size else n)


def topk_select(shat, k):
    """Top-k + global for one head: the k largest pairs of the [N_b, N_b] pool (ties by
    ascending linear index) union the diagonal.  Same keys as threshold_select."""
    shat = np.asarray(shat, dtype=np.float64)
    nb = shat.shape[0]
    flat = shat.reshape(nb * nb)
    order, kk = _ordered_prefix(flat, k=k)
    mask = np.zeros(nb * nb, dtype=bool)
    mask[order[:kk]] = True
    mask = mask.reshape(nb, nb)
    mask[np.arange(nb), np.arange(nb)] = True
    vals = flat[order]
    return {"mask": mask, "k": kk, "v": float(vals[kk - 1]) if kk else 0.0,
            "mass": float(vals[:kk].sum()), "order": order}


def normalise_per_row(s):
    """Softmax of every query-block row over its N_b key blocks.  s: [..., N_b, N_b]."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def local_select(shat_rows, tau=None, k=None):
    """Threshold + local (tau) or top-k + local (k) for one head: every row of the
    row-normalised [N_b, N_b] scores is its own pool.  Returns a dict with ``mask``,
    ``k`` (prefix lengths summed over rows), ``row_k``, ``row_v`` (each row's cutoff value)
    and ``row_mass`` (each row's prefix mass)."""
    shat_rows = np.asarray(shat_rows, dtype=np.float64)
    nb = shat_rows.shape[0]
    mask = np.zeros((nb, nb), dtype=bool)
    row_k = np.zeros(nb, dtype=np.int64)
    row_v = np.zeros(nb)
    row_mass = np.zeros(nb)
    for i in range(nb):
        order, kk = _ordered_prefix(shat_rows[i], tau=tau, k=k)
        mask[i, order[:kk]] = True
        row_k[i] = kk
        row_v[i] = shat_rows[i, order[kk - 1]] if kk else 0.0
        row_mass[i] = shat_rows[i, order[:kk]].sum()
    mask[np.arange(nb), np.arange(nb)] = True
    return {"mask": mask, "k": int(row_k.sum()), "row_k": row_k, "row_v": row_v,
            "row_mass": row_mass}


SELECTION_MODES = ("threshold_global", "topk_global", "threshold_local", "topk_local")


def select_all_heads(q_pool, k_pool, tau, mode="threshold_global", k=None):
    """Scores, normalisation and selection for every (b, h) under one of SELECTION_MODES
    (tau for the threshold modes, k for the top-k modes).

    Returns (mask [B,Hh,N_b,N_b] bool, shat [B,Hh,N_b,N_b], stats list of dicts with keys
    k, nnz (and v, mass for the global modes; row_k, row_v, row_mass for the local ones)
    per (b, h) in row-major (b, h) order).  shat is normalised over the mode's pool: the
    whole head for the global modes, each row for the local ones.
    """
    if mode not in SELECTION_MODES:
        raise ValueError(f"unknown selection mode {mode!r}")
    s = block_scores(q_pool, k_pool)
    local = mode.endswith("_local")
    shat = normalise_per_row(s) if local else normalise_per_head(s)
    B, Hh, nb, _ = shat.shape
    mask = np.zeros((B, Hh, nb, nb), dtype=bool)
    stats = []
    for b in range(B):
        for h in range(Hh):
            if mode == "threshold_global":
                r = threshold_select(shat[b, h], tau)
            elif mode == "topk_global":
                r = topk_select(shat[b, h], k)
            elif mode == "threshold_local":
                r = local_select(shat[b, h], tau=tau)
            else:
                r = local_select(shat[b, h], k=k)
            mask[b, h] = r["mask"]
            st = {key: r[key] for key in r if key not in ("mask", "order")}
            st["nnz"] = int(r["mask"].sum())
            stats.append(st)
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
