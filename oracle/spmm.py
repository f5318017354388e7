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


def nm_spmm_flops(T: int, d_in: int, d_out: int, n: int, m: int) -> int:
    """Algorithmic FLOPs: ``2 * T * d_out * d_in * n / m`` (kept columns only)."""
    return 2 * T * d_out * (d_in * n // m)
