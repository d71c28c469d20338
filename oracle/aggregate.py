"""Neighbour aggregation of a partition's rows over inner and (dequantised) halo nodes, in float64.

GCN (SYLVIE guide, section 2): z_v = sum over u in N(v) and v itself of W h_u / sqrt(d_v d_u).
Aggregation and projection are separated by linearity: a_v = sum_u h_u / sqrt(d_v d_u) here, and
z_v = W a_v in ``dense``.  Readings used:
  * d is the degree counting the self-loop, d = |N(v)| + 1 (the renormalised adjacency A + I; the
    formula sums over N(v) and v, and this keeps isolated nodes finite);
  * for a halo node, d is its *global* degree, which the guide (section 7) insists on over the
    partition-local count; the caller passes it in ``deg``.
GraphSAGE is only named by the guide as another aggregation style; the mean form used is
a_v = [h_v || mean over u in N(v) of h_u] (no self term in the mean; an empty row gives 0).

Backward: the embedding gradient of a column node u is sum over rows v with u in N(v) and v of
g_v / sqrt(d_v d_u), the same dependencies walked in reverse (guide sections 3 and 11).
The sparse matrix products are scipy's CSR routines; the matrix is built here straight from the
definition.
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sp


def gcn_matrix(nbr_ptr: np.ndarray, nbr_idx: np.ndarray, deg: np.ndarray) -> sp.csr_matrix:
    """Rows are the n_in inner nodes, columns all inner + halo nodes; entry 1/sqrt(d_v d_u) on N(v) and v."""
    n_rows = nbr_ptr.size - 1
    n_cols = deg.size
    rows = np.repeat(np.arange(n_rows), np.diff(nbr_ptr))
    r = np.concatenate([rows, np.arange(n_rows)])
    c = np.concatenate([nbr_idx.astype(np.int64), np.arange(n_rows)])
    dd = deg.astype(np.float64) + 1.0
    w = 1.0 / np.sqrt(dd[r] * dd[c])
    return sp.csr_matrix((w, (r, c)), shape=(n_rows, n_cols))


def mean_matrix(nbr_ptr: np.ndarray, nbr_idx: np.ndarray, n_cols: int) -> sp.csr_matrix:
    n_rows = nbr_ptr.size - 1
    cnt = np.diff(nbr_ptr).astype(np.float64)
    rows = np.repeat(np.arange(n_rows), np.diff(nbr_ptr))
    w = 1.0 / cnt[rows]
    return sp.csr_matrix((w, (rows, nbr_idx.astype(np.int64))), shape=(n_rows, n_cols))


def gcn_aggregate(nbr_ptr, nbr_idx, deg, x_cols, rows=None) -> np.ndarray:
    """a_v for every inner row (or the listed ``rows``); ``x_cols`` holds inner then halo rows."""
    A = gcn_matrix(nbr_ptr, nbr_idx, deg)
    if rows is not None:
        A = A[np.asarray(rows)]
    return np.asarray(A @ np.asarray(x_cols, dtype=np.float64))


def gcn_aggregate_t(nbr_ptr, nbr_idx, deg, g, cols=None) -> np.ndarray:
    """Gradient w.r.t. every column node (or the listed ``cols``) of sum_v <a_v, g_v>."""
    A = gcn_matrix(nbr_ptr, nbr_idx, deg).tocsc()
    if cols is not None:
        A = A[:, np.asarray(cols)]
    return np.asarray(A.T @ np.asarray(g, dtype=np.float64))


def mean_aggregate(nbr_ptr, nbr_idx, x_cols, rows=None) -> np.ndarray:
    A = mean_matrix(nbr_ptr, nbr_idx, x_cols.shape[0])
    if rows is not None:
        A = A[np.asarray(rows)]
    return np.asarray(A @ np.asarray(x_cols, dtype=np.float64))


def mean_aggregate_t(nbr_ptr, nbr_idx, g, n_cols, cols=None) -> np.ndarray:
    A = mean_matrix(nbr_ptr, nbr_idx, n_cols).tocsc()
    if cols is not None:
        A = A[:, np.asarray(cols)]
    return np.asarray(A.T @ np.asarray(g, dtype=np.float64))


def add_received(dx_inner: np.ndarray, mirror: np.ndarray, received: np.ndarray) -> np.ndarray:
    """The owner's side of the backward exchange: each received halo gradient (already dequantised)
    is added to the gradient of the inner node it copies (guide section 11, backward loop)."""
    out = np.array(dx_inner, dtype=np.float64, copy=True)
    np.add.at(out, np.asarray(mirror), np.asarray(received, dtype=np.float64))
    return out
