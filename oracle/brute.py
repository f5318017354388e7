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
