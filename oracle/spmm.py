"""Batched N:M activation-sparse matmul, plain fp64 definition (test infrastructure only).

Q-Sparse replies (answer on batched inference): for large batches the
activations of every token are N:M sparse and multiply a dense weight; the
reply benchmarks that product against a dense matmul.
"""

from __future__ import annotations

import numpy as np


def nm_spmm(X, keep, wt) -> np.ndarray:
    """``Y[t][o] = sum_k (keep ⊙ X)[t][k] * W[o][k]`` in fp64.

    ``X``: fp16 ``[T][d_in]``; ``keep``: bool ``[T][d_in]``; ``wt``:
    ``WT[d_in][d_out]``.  Written per token as the sum over its kept columns.
    """
    X = np.asarray(X)
    keep = np.asarray(keep)
    wt = np.asarray(wt)
    Y = np.empty((X.shape[0], wt.shape[1]), dtype=np.float64)
    for t in range(X.shape[0]):
        idx = np.flatnonzero(keep[t])
        cols = wt[idx].astype(np.float64)
        Y[t] = (cols * X[t, idx].astype(np.float64)[:, None]).sum(axis=0)
    return Y


def masked_matmul(X, keep, wt) -> np.ndarray:
    """The same product as ``nm_spmm`` for every token at once:
    ``Y = (keep ⊙ X) @ WT`` in fp64, with numpy's matmul as the one library
    step (the masked activations, widened exactly, times the widened
    weight).  It serves the full-size workloads, where the per-token sums
    above would take minutes.  ``keep`` may be any boolean mask of ``X``'s
    shape (per-token N:M, or a tile-shared mask expanded to its tokens).
    """
    X = np.asarray(X)
    keep = np.asarray(keep, dtype=bool)
    if keep.shape != X.shape:
        raise ValueError("keep must have X's shape")
    xs = np.where(keep, X.astype(np.float64), 0.0)
    return xs @ np.asarray(wt).astype(np.float64)


def nm_shared_spmm(vals, tile_keep, tt: int, wt) -> np.ndarray:
    """The same product from the tile-shared compressed form: token t of tile
    ``g = t // tt`` holds its values at the kept positions of ``tile_keep[g]``
    (ascending), and ``Y[t] = sum_j vals[t][j] * WT[pos_g[j]]`` in fp64."""
    vals = np.asarray(vals)
    tile_keep = np.asarray(tile_keep)
    wt = np.asarray(wt)
    Y = np.empty((vals.shape[0], wt.shape[1]), dtype=np.float64)
    for t in range(vals.shape[0]):
        pos = np.flatnonzero(tile_keep[t // tt])
        Y[t] = (wt[pos].astype(np.float64) * vals[t].astype(np.float64)[:, None]).sum(axis=0)
    return Y


def nm_spmm_flops(T: int, d_in: int, d_out: int, n: int, m: int) -> int:
    """Algorithmic FLOPs: ``2 * T * d_out * d_in * n / m`` (kept columns only)."""
    return 2 * T * d_out * (d_in * n // m)
