"""Oracle for masked softmax attention (TEST INFRASTRUCTURE ONLY; see package doc).

Plain float64 numpy.  Inputs are the exact values of the bf16 tensors the
GPU path receives (converted losslessly to float64); nothing is rounded on
the way.

Definitions followed (review Prompt 1.3.1, Step 0; paper §3 Eq.1 and Eq.2,
whose bodies were lost in extraction but are the standard forms):

* logits z[q, k] = scale * <Q[q], K[k]> for the keys k the mask allows, and
  -inf for the others (the mask M is added to the logits);
* P = softmax over k of z, O = P V, and LSE[q] = log sum_k exp(z[q, k])
  (natural log), i.e. LSE = m + log(sum exp(z - m)) with m = max_k z;
* gradients of O with respect to Q, K, V for an upstream gradient dO are the
  textbook ones: dV = P^T dO, dP = dO V^T, Delta[q] = sum_k P[q,k] dP[q,k]
  (= <dO[q], O[q]>), dS = P * (dP - Delta), dQ = scale dS K,
  dK = scale dS^T Q.

The mask is given as a set of key columns per query tile ("tile semantics",
review Step 5, paper §4.2: every token of a kept block is computed), or as a
boolean token mask for small problems.
"""

from __future__ import annotations

import numpy as np


def tile_columns(kept_row: np.ndarray, n: int, T: int) -> np.ndarray:
    """Key token indices of the kept tiles in one row of the tile map."""
    tiles = np.nonzero(kept_row)[0]
    cols = (tiles[:, None] * T + np.arange(T)[None, :]).reshape(-1)
    return cols[cols < n]


def _softmax_rows(z: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[:, 0]
    # every softmax row sums to one (review Step 0: P is a distribution)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-9)
    return p, lse


def fwd_rows(q_rows: np.ndarray, k_cols: np.ndarray, v_cols: np.ndarray,
             scale: float) -> tuple[np.ndarray, np.ndarray]:
    """O and LSE of some query rows over the keys they may attend: q_rows
    float64 [r, D] and the attended keys' K and V rows k_cols, v_cols
    float64 [c, D] (the definition, for rows whose allowed keys are given)."""
    z = scale * (q_rows @ k_cols.T)
    p, lse = _softmax_rows(z)
    return p @ v_cols, lse


def fwd_tile(q: np.ndarray, k: np.ndarray, v: np.ndarray, kept: np.ndarray,
             T: int, scale: float, u: int) -> tuple[np.ndarray, np.ndarray]:
    """O and LSE for the query rows of tile u of one (batch, head).

    q, k, v: float64 [n, D].  kept: boolean [nb, nb] tile map.
    Returns O [rows, D] and LSE [rows] with rows = the valid rows of tile u.
    """
    n = q.shape[0]
    rows = slice(u * T, min(n, (u + 1) * T))
    cols = tile_columns(kept[u], n, T)
    return fwd_rows(q[rows], k[cols], v[cols], scale)


def fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, kept: np.ndarray,
        T: int, scale: float, tiles=None) -> tuple[np.ndarray, np.ndarray]:
    """O [n, D] and LSE [n] for one (batch, head) under the tile map.

    ``tiles``: optional list of query tiles to compute; rows of other tiles
    are left as NaN.
    """
    n, d = q.shape
    nb = kept.shape[0]
    o = np.full((n, d), np.nan)
    lse = np.full(n, np.nan)
    for u in (range(nb) if tiles is None else tiles):
        rows = slice(u * T, min(n, (u + 1) * T))
        o[rows], lse[rows] = fwd_tile(q, k, v, kept, T, scale, u)
    return o, lse


def fwd_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
               scale: float) -> tuple[np.ndarray, np.ndarray]:
    """O and LSE for one (batch, head) under a boolean token mask [n, n]
    (True = allowed).  Every row must allow at least one key."""
    z = scale * (q @ k.T)
    z = np.where(mask, z, -np.inf)
    p, lse = _softmax_rows(z)
    return p @ v, lse


def bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
        kept: np.ndarray, T: int, scale: float):
    """dQ, dK, dV [n, D] for one (batch, head) under the tile map."""
    n, d = q.shape
    nb = kept.shape[0]
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for u in range(nb):
        rows = slice(u * T, min(n, (u + 1) * T))
        cols = tile_columns(kept[u], n, T)
        z = scale * (q[rows] @ k[cols].T)
        p, _ = _softmax_rows(z)
        dp = do[rows] @ v[cols].T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dv[cols] += p.T @ do[rows]
        dq[rows] += scale * (ds @ k[cols])
        dk[cols] += scale * (ds.T @ q[rows])
    return dq, dk, dv


def bwd_masked(q, k, v, do, mask, scale):
    """dQ, dK, dV for one (batch, head) under a boolean token mask [n, n]."""
    z = scale * (q @ k.T)
    z = np.where(mask, z, -np.inf)
    p, _ = _softmax_rows(z)
    dp = do @ v.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ do


def dq_masked(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, do_rows: np.ndarray,
              mask_rows: np.ndarray, scale: float) -> np.ndarray:
    """dQ of some query rows under their rows of a boolean token mask
    [r, n]: the first gradient of ``bwd_masked`` for those rows alone (a
    query row's gradient depends only on its own softmax row)."""
    z = np.where(mask_rows, scale * (q_rows @ k.T), -np.inf)
    p, _ = _softmax_rows(z)
    dp = do_rows @ v.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    return scale * ((p * (dp - delta)) @ k)


def dq_rows(q_rows: np.ndarray, k_cols: np.ndarray, v_cols: np.ndarray,
            do_rows: np.ndarray, scale: float) -> np.ndarray:
    """dQ of some query rows over the keys they may attend (as ``fwd_rows``):
    a query row's gradient depends only on its own softmax row."""
    z = scale * (q_rows @ k_cols.T)
    p, _ = _softmax_rows(z)
    dp = do_rows @ v_cols.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    return scale * ((p * (dp - delta)) @ k_cols)


def bwd_dq_tile(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                kept: np.ndarray, T: int, scale: float, u: int) -> np.ndarray:
    """dQ for the valid rows of query tile u only (same formulas as ``bwd``,
    restricted to one row block)."""
    n = q.shape[0]
    rows = slice(u * T, min(n, (u + 1) * T))
    cols = tile_columns(kept[u], n, T)
    return dq_rows(q[rows], k[cols], v[cols], do[rows], scale)


def row_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
              kept: np.ndarray, T: int, scale: float, u: int) -> tuple[np.ndarray, np.ndarray]:
    """LSE and Delta for the valid rows of query tile u: the log-sum-exp of
    each row's logits over all of its kept keys, and Delta = <dO, O> with
    O = P V over the same keys (the row terms of the textbook gradient)."""
    o, lse = fwd_tile(q, k, v, kept, T, scale, u)
    n = q.shape[0]
    rows = slice(u * T, min(n, (u + 1) * T))
    return lse, (do[rows] * o).sum(axis=1)


def bwd_dkdv_tile(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  kept: np.ndarray, T: int, scale: float, vt: int, stats=None):
    """dK and dV for the valid key rows of key tile vt only.

    The keys of tile vt receive gradient from every query row of every query
    tile u whose row keeps vt (the tile map's column vt).  For each such row
    the softmax runs over all of the row's own kept keys (its LSE), and the
    textbook formulas restricted to the keys of vt give
    dV_vt = sum_q P[q, vt]^T dO[q] and dK_vt = scale sum_q dS[q, vt]^T Q[q],
    with dS = P (dP - Delta), dP = dO V_vt^T and Delta = <dO, O> of the row.
    ``stats``: optional mapping u -> (LSE, Delta) of query tile u, as
    ``row_stats`` returns (computed here when absent).
    Returns dK, dV [keys, D] for the keys of vt below n.
    """
    n, d = q.shape
    keys = slice(vt * T, min(n, (vt + 1) * T))
    nk = keys.stop - keys.start
    dk = np.zeros((nk, d))
    dv = np.zeros((nk, d))
    for u in np.nonzero(kept[:, vt])[0]:
        rows = slice(u * T, min(n, (u + 1) * T))
        lse, delta = stats[u] if stats is not None else row_stats(q, k, v, do, kept, T, scale, u)
        p = np.exp(scale * (q[rows] @ k[keys].T) - lse[:, None])
        dp = do[rows] @ v[keys].T
        ds = p * (dp - delta[:, None])
        dv += p.T @ do[rows]
        dk += scale * (ds.T @ q[rows])
    return dk, dv


def row_stats_masked(q_rows: np.ndarray, k_cols: np.ndarray, v_cols: np.ndarray,
                     do_rows: np.ndarray, mask_rows: np.ndarray,
                     scale: float) -> tuple[np.ndarray, np.ndarray]:
    """LSE and Delta of some query rows under their rows of a boolean token
    mask, restricted to key columns that hold every key the rows may attend
    (k_cols, v_cols [c, D]; mask_rows [r, c]): the row terms of the textbook
    gradient, as ``row_stats`` gives them under the tile map."""
    o, lse = fwd_masked(q_rows, k_cols, v_cols, mask_rows, scale)
    return lse, (do_rows * o).sum(axis=1)


def dkdv_masked_keys(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                     keys: slice, blocks, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """dK and dV [keys, D] of the key rows ``keys`` under a boolean token mask.

    ``blocks``: tuples (rows, allowed, lse, delta) over groups of query rows
    that together hold every query row the mask lets attend one of these
    keys; ``allowed`` [len(rows), len(keys)] is the mask restricted to those
    rows and keys, and lse, delta are the rows' terms over all of their
    allowed keys (``row_stats_masked``).  The textbook formulas restricted
    to the keys: P = exp(scale <Q, K> - LSE) where allowed (0 elsewhere),
    dV = P^T dO and dK = scale (P (dP - Delta))^T Q with dP = dO V^T.
    """
    nk, d = keys.stop - keys.start, q.shape[1]
    dk = np.zeros((nk, d))
    dv = np.zeros((nk, d))
    for rows, allowed, lse, delta in blocks:
        z = scale * (q[rows] @ k[keys].T)
        p = np.where(allowed, np.exp(np.where(allowed, z, 0.0) - lse[:, None]), 0.0)
        dp = do[rows] @ v[keys].T
        ds = p * (dp - delta[:, None])
        dv += p.T @ do[rows]
        dk += scale * (ds.T @ q[rows])
    return dk, dv
