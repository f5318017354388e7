"""Sparse-input GEMV, plain fp64 definitions (test infrastructure only).

The weight is given as stored, ``WT[d_in][d_out]`` fp16 (``W`` column-major),
so row ``k`` of ``WT`` is the column of ``W`` that activation entry ``k``
multiplies.
"""

from __future__ import annotations

import numpy as np


def sparse_gemv(wt, idx, val) -> np.ndarray:
    """``y[o] = sum_j W[o][idx_j] * val_j`` in fp64.

    RaNA replies, Q5.1: once the activation is sparse, the products with the
    weight columns of its zero entries are skipped; only the listed columns
    take part.  ``idx``: kept column indices; ``val``: their activation values.
    """
    idx = np.asarray(idx, dtype=np.int64)
    val = np.asarray(val).astype(np.float64)
    cols = np.asarray(wt)[idx].astype(np.float64)  # [nnz][d_out]
    return (cols * val[:, None]).sum(axis=0)


def masked_gemv(wt, x, keep) -> np.ndarray:
    """``y = W (keep ⊙ x)`` for one row: the same sum over the kept entries."""
    idx = np.flatnonzero(np.asarray(keep))
    return sparse_gemv(wt, idx, np.asarray(x)[idx])


def batched_masked_gemv(wt, X, keep) -> np.ndarray:
    """Rows of ``X`` each with their own mask: ``Y[b] = W (keep_b ⊙ x_b)``.

    Each weight column in the union of the masks is read once for all rows
    by the GPU path; the definition is simply one masked GEMV per row.
    """
    X = np.asarray(X)
    keep = np.asarray(keep)
    return np.stack([masked_gemv(wt, X[b], keep[b]) for b in range(X.shape[0])])


def dense_gemv(wt, x) -> np.ndarray:
    """``y = W x`` with every column: the sparse sum over all indices."""
    x = np.asarray(x)
    return sparse_gemv(wt, np.arange(x.shape[-1]), x)


def union_columns(keep) -> int:
    """Number of weight columns a batched call must read: ``|∪_b keep_b|``."""
    return int(np.count_nonzero(np.any(np.asarray(keep), axis=0)))


def gemv_flops(d_out: int, nnz: int) -> int:
    """Matmul FLOPs of one sparse GEMV: ``2 * d_out * nnz``.

    Q-Sparse replies, A3 on FLOP counting: a ``d x d`` by ``d x 1`` product
    costs ``2 d^2`` and the Top-K selection is not counted; with only ``nnz``
    columns taking part that becomes ``2 d_out nnz``.
    """
    return 2 * int(d_out) * int(nnz)
