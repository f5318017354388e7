"""Exhaustive enumeration for tiny inputs (test infrastructure only).

A third, independent statement of the selection rules: among all subsets of
the allowed size, take those with the largest total magnitude, and of those
the one whose ascending index list is lexicographically smallest.  That is
"largest magnitudes, ties to the lower index".  Sums of at most a few dozen
fp16 magnitudes are exact in fp64, so the maximum is found exactly.
"""

from __future__ import annotations

import itertools

import numpy as np


def _best_subset(mags, size: int):
    best, best_sum = None, -1.0
    # combinations() yields index tuples in lexicographic order, so the first
    # tuple reaching the maximum is the lexicographically smallest one.
    for comb in itertools.combinations(range(len(mags)), size):
        s = float(sum(mags[i] for i in comb))
        if s > best_sum:
            best, best_sum = comb, s
    return best


def topk_brute(x, k: int) -> np.ndarray:
    """Top-K mask of a short vector by enumerating all ``C(d, k)`` subsets."""
    x = np.asarray(x)
    mags = [abs(float(v)) for v in x]
    keep = np.zeros(len(mags), dtype=bool)
    best = _best_subset(mags, k)
    keep[list(best)] = True
    return keep


def nm_layouts(n: int, m: int):
    """All N:M keep-layouts of one group: every way to choose ``n`` of ``m``."""
    return list(itertools.combinations(range(m), n))


def nm_brute(x, n: int, m: int) -> np.ndarray:
    """N:M mask of one row by enumerating every layout of every group."""
    x = np.asarray(x)
    d = x.shape[0]
    keep = np.zeros(d, dtype=bool)
    layouts = nm_layouts(n, m)
    for g0 in range(0, d, m):
        mags = [abs(float(v)) for v in x[g0:g0 + m]]
        best, best_sum = None, -1.0
        for lay in layouts:
            s = float(sum(mags[i] for i in lay))
            if s > best_sum:
                best, best_sum = lay, s
        for i in best:
            keep[g0 + i] = True
    return keep


def threshold_loop(x, t: float) -> np.ndarray:
    """Threshold mask with a plain Python loop, one comparison per entry."""
    return np.array([abs(float(v)) >= t and float(v) != 0.0 for v in np.asarray(x)],
                    dtype=bool)


def rank_adapter_loop(bt, at, x, t: float) -> np.ndarray:
    """The rank adapter ``A (m ⊙ B x)`` as scalar loops: ``v_i`` summed in
    fp64 and stored as fp16, kept iff ``v_i * v_i >= t``, then each kept
    ``v_i`` times row ``i`` of ``AT`` added into ``y``."""
    d_in, r = len(bt), len(bt[0])
    d_out = len(at[0])
    y = [0.0] * d_out
    for i in range(r):
        s = 0.0
        for k in range(d_in):
            s += float(bt[k][i]) * float(x[k])
        vi = float(np.float16(s))
        if vi * vi >= t:
            for o in range(d_out):
                y[o] += vi * float(at[i][o])
    return np.array(y)
