"""Activation sparsifiers, plain fp64 definitions (test infrastructure only).

A sparsifier decides, from an activation vector alone, which entries survive;
every later step multiplies only the surviving entries.  Magnitudes of fp16
values are compared exactly (widening fp16 to fp64 is exact), so -0 and +0 are
equal and an fp32 threshold is compared without rounding.
"""

from __future__ import annotations

import numpy as np


def _rows(x):
    x = np.asarray(x)
    return x[None, :] if x.ndim == 1 else x


def threshold_sparsify(x, t):
    """Per-tensor magnitude threshold.

    TEAL README, Abstract: entries of a hidden state are zeroed by magnitude.
    The comparator is ``>=``, the only one the pages print (RaNA replies, Q3,
    CATS and RaNA neuron masks).  An entry equal to zero is never kept, so the
    number kept equals the number of nonzeros of the result and the sparsity
    below is exact at ``t = 0``.

    ``x``: fp16 array ``[d]`` or ``[rows][d]``; ``t``: a float (fp32 value).
    Returns ``keep`` (bool, same shape), and per row the ascending kept
    indices, their values (fp16, unchanged) and the count.
    """
    x2 = _rows(x)
    xf = x2.astype(np.float64)
    keep = (np.abs(xf) >= float(t)) & (xf != 0.0)
    idx = [np.flatnonzero(keep[r]) for r in range(x2.shape[0])]
    val = [x2[r][idx[r]] for r in range(x2.shape[0])]
    nnz = np.array([len(i) for i in idx], dtype=np.int64)
    if np.asarray(x).ndim == 1:
        return keep[0], idx[0], val[0], int(nnz[0])
    return keep, idx, val, nnz


def topk_sparsify(x, k: int):
    """Per-token Top-K by magnitude.

    Q-Sparse replies (answer comparing with MoE): for each token the entries
    of smaller magnitude are pruned, keeping K.  Ties in magnitude go to the
    lower index.  Written as its definition: stable-sort the indices by
    descending magnitude (a stable sort keeps equal magnitudes in ascending
    index order), keep the first K, then list them in ascending order.
    """
    x2 = _rows(x)
    d = x2.shape[1]
    if not 0 <= k <= d:
        raise ValueError("k out of range")
    keep = np.zeros(x2.shape, dtype=bool)
    for r in range(x2.shape[0]):
        mag = np.abs(x2[r].astype(np.float64))
        order = np.argsort(-mag, kind="stable")
        keep[r, order[:k]] = True
    idx = [np.flatnonzero(keep[r]) for r in range(x2.shape[0])]
    val = [x2[r][idx[r]] for r in range(x2.shape[0])]
    nnz = np.array([len(i) for i in idx], dtype=np.int64)
    if np.asarray(x).ndim == 1:
        return keep[0], idx[0], val[0], int(nnz[0])
    return keep, idx, val, nnz


def nm_sparsify(x, n: int, m: int):
    """N:M activation sparsity: keep N of every M consecutive entries.

    Q-Sparse replies (answer on batched inference): Block Q-Sparse applies N:M
    sparsity over M consecutive elements.  The pages disagree on whether N
    counts kept or zeroed entries; the N:M summary's methodology section says
    N nonzeros are kept, and that reading is used.  The score is the absolute
    activation (ACT criterion, same section).  Within each aligned group the
    N largest magnitudes survive, ties to the lower position.

    ``x``: fp16 ``[T][d]`` with ``d % m == 0``.  Returns ``keep`` bool
    ``[T][d]`` and the compressed values ``[T][d*n/m]`` in position order.
    """
    x2 = _rows(x)
    T, d = x2.shape
    if d % m or not 1 <= n <= m:
        raise ValueError("bad N:M shape")
    groups = np.abs(x2.astype(np.float64)).reshape(T, d // m, m)
    order = np.argsort(-groups, axis=-1, kind="stable")[..., :n]
    keep = np.zeros(groups.shape, dtype=bool)
    np.put_along_axis(keep, order, True, axis=-1)
    keep = keep.reshape(T, d)
    vals = x2[keep].reshape(T, d * n // m)
    if np.asarray(x).ndim == 1:
        return keep[0], vals[0]
    return keep, vals


def nm_shared_sparsify(x, n: int, m: int, tt: int = 32):
    """Tile-shared (vector-wise) N:M: one N:M pattern for each run of ``tt``
    consecutive tokens.

    Q-Sparse replies (answer on batched inference): Block Q-Sparse keeps N of
    every M consecutive activations, and the batched kernel the reply times is
    nmSPARSE's VW32 form, in which one N:M pattern is shared by a vector of 32
    (the cited nmSPARSE paper defines the vector-wise form for weights; here
    the activations carry it).  The pages give no selection rule for a shared
    pattern.  Readings taken here:
    * the vector is ``tt`` consecutive tokens (rows of ``x``); the last tile
      holds the remaining ``T mod tt`` tokens when ``tt`` does not divide T;
    * a position's score is the sum of the tile's magnitudes at it (the ACT
      criterion of the N:M summary, section 2, summed over the tile: the L1
      norm of the column segment).  The fp64 sum is exact: every fp16
      magnitude is an integer multiple of 2^-24 below 2^16, so any partial sum
      of at most 256 of them is an integer multiple of 2^-24 below 2^24, which
      fp64 holds exactly; the order of the additions does not matter;
    * in each aligned group of ``m`` positions the ``n`` largest scores are
      kept, ties to the lower position (the per-token rule on the scores).

    ``x``: fp16 ``[T][d]``, ``d % m == 0``, ``1 <= tt <= 256``.  Returns
    ``keep`` bool ``[T][d]`` (equal rows within a tile), ``tile_keep`` bool
    ``[ceil(T/tt)][d]`` and the compressed values ``[T][d*n/m]``: each token's
    entries at its tile's kept positions, in position order.
    """
    x2 = _rows(x)
    T, d = x2.shape
    if d % m or not 1 <= n <= m or not 1 <= tt <= 256:
        raise ValueError("bad shared N:M shape")
    tiles = (T + tt - 1) // tt
    tile_keep = np.zeros((tiles, d), dtype=bool)
    for g in range(tiles):
        score = np.abs(x2[g * tt:(g + 1) * tt].astype(np.float64)).sum(axis=0)
        groups = score.reshape(d // m, m)
        order = np.argsort(-groups, axis=-1, kind="stable")[:, :n]
        kg = np.zeros(groups.shape, dtype=bool)
        np.put_along_axis(kg, order, True, axis=-1)
        tile_keep[g] = kg.reshape(d)
    keep = tile_keep[np.arange(T) // tt]
    vals = x2[keep].reshape(T, d * n // m)
    return keep, tile_keep, vals


def apply_mask(x, keep):
    """``keep ⊙ x`` as fp64 (the sparsified activation)."""
    return np.where(keep, np.asarray(x).astype(np.float64), 0.0)


def activation_sparsity(x_s) -> float:
    """Fraction of zero entries of the activation that enters the product.

    Q-Sparse replies (answer defining activation sparsity); the ProSparse
    summary, Overview, states the same definition.
    """
    x_s = np.asarray(x_s)
    return float(np.count_nonzero(x_s == 0)) / x_s.size


def pack_mask(keep) -> np.ndarray:
    """Bitmask words: bit ``j`` of word ``w`` of a row is entry ``32*w + j``.

    ``keep``: bool ``[..., d]`` -> uint32 ``[..., ceil(d/32)]``; padding bits
    past ``d`` are zero.
    """
    keep = np.asarray(keep, dtype=bool)
    d = keep.shape[-1]
    words = (d + 31) // 32
    padded = np.zeros(keep.shape[:-1] + (words * 32,), dtype=np.uint64)
    padded[..., :d] = keep
    bits = padded.reshape(keep.shape[:-1] + (words, 32))
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (bits * weights).sum(axis=-1).astype(np.uint32)


def unpack_mask(words, d: int) -> np.ndarray:
    """Inverse of :func:`pack_mask`."""
    words = np.asarray(words, dtype=np.uint32)
    bits = (words[..., None] >> np.arange(32, dtype=np.uint32)) & 1
    flat = bits.reshape(words.shape[:-1] + (words.shape[-1] * 32,))
    return flat[..., :d].astype(bool)
