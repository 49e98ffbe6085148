"""fp64 masked softmax attention: the definition, written out.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed ("Accelerating Sparse Transformer Inference on GPU",
gist.science explainer, Technical summary > Problem statement: masks decide
which (query, key) pairs of MHA take part; Methodology > 1. Unified MHA
module: the masking is exact), for every batch b, head h and query row i:

    J_i   = { j : mask[i, j] }
    s_j   = tau * <Q[b,h,i,:], K[b,h,j,:]>              j in J_i
    O_i   = sum_j exp(s_j - m) V[b,h,j,:] / sum_j exp(s_j - m),  m = max s_j
    O_i   = 0                                            if J_i is empty

tau = 1/sqrt(d) unless given.  The mask may be one [S, S] matrix for every
(b, h) or a stack [Bm, Hm, S, S] with Bm in {1, B} and Hm in {1, H}: (b, h)
then uses mask[b if Bm > 1 else 0, h if Hm > 1 else 0] (a mask per sequence
and/or per head; the pages' masks decide per pair, for any mask).
Subtracting m changes no value; it only keeps exp from overflowing.  The empty-row convention (O = 0, never NaN) is a
reading: the pages are silent on rows with no valid key.

The dense score matrix is computed and masked afterwards, i.e. the
compute-then-reset approach the pages name as the wasteful fallback of prior
kernels; here it is the point, because it is obviously right.
"""
import math

import numpy as np


def _as_f64(x):
    if hasattr(x, "detach"):          # torch tensor (CPU): exact upcast
        x = x.detach().to("cpu")
        import torch
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _rows(q, k, v, mask_rows, tau):
    """Attention for a block of query rows of one (b, h).

    q: [R, d], k, v: [S, d], mask_rows: [R, S] bool.  Returns [R, d].
    """
    s = (q @ k.T) * tau                       # [R, S] dense scores
    s = np.where(mask_rows, s, -np.inf)       # reset the masked scores
    m = s.max(axis=1)                         # -inf for an empty row
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    w = np.exp(s - m[:, None])                # exactly 0 where masked
    den = w.sum(axis=1)
    num = w @ v
    out = np.zeros_like(num)
    ok = ~empty
    out[ok] = num[ok] / den[ok, None]
    return out


def mask_of(mask, b, h):
    """The [S, S] mask that batch b, head h uses (broadcast rule above)."""
    mask = np.asarray(mask)
    if mask.ndim == 2:
        return mask
    return mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]


def _check_mask(mask, B, H, S):
    if mask.ndim == 2:
        assert mask.shape == (S, S)
    else:
        assert mask.ndim == 4 and mask.shape[2:] == (S, S)
        assert mask.shape[0] in (1, B) and mask.shape[1] in (1, H)


def attention(q, k, v, mask, scale=None, row_block=1024):
    """Dense fp64 masked attention.

    q, k, v: [B, H, S, d] (numpy or CPU torch; upcast exactly to fp64).
    mask: bool, True = pair takes part: [S, S] shared by every (b, h), or
    a stack [Bm, Hm, S, S] (mask_of).
    scale: tau, default 1/sqrt(d).
    Returns a float64 numpy array [B, H, S, d].

    Rows are processed ``row_block`` at a time only to bound memory; each
    row's result depends on nothing but that row.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    mask = np.asarray(mask, dtype=bool)
    B, H, S, d = q.shape
    assert k.shape == (B, H, S, d) and v.shape == (B, H, S, d)
    _check_mask(mask, B, H, S)
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    out = np.empty((B, H, S, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            m = mask_of(mask, b, h)
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                out[b, h, r0:r1] = _rows(q[b, h, r0:r1], k[b, h], v[b, h],
                                         m[r0:r1], tau)
    return out


def attention_rows(q, k, v, mask, b, h, rows, scale=None, mask_rows=None):
    """The same definition for selected query rows of one (b, h).

    Used to check full-size workloads on a sample of outputs.  mask: as for
    attention; or None with mask_rows [len(rows), S] bool, the mask rows of
    those queries alone, for masks too large to hold whole.  Returns
    [len(rows), d] float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if hasattr(q, "detach"):
        import torch
        qb = _as_f64(q[b, h].index_select(0, torch.as_tensor(rows)))
    else:
        qb = _as_f64(np.asarray(q)[b, h][rows])
    kb = _as_f64(k[b, h])
    vb = _as_f64(v[b, h])
    d = qb.shape[1]
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    if mask_rows is not None:
        mask_rows = np.asarray(mask_rows, dtype=bool)
        assert mask_rows.shape == (len(rows), kb.shape[0])
        return _rows(qb, kb, vb, mask_rows, tau)
    m = np.asarray(mask_of(mask, b, h), dtype=bool)
    return _rows(qb, kb, vb, m[rows], tau)
