"""Weight-aware selection with a static shift and a variance correction,
plain fp64 steps (test infrastructure only).

The flexible N:M activation-sparsity summary, section 2 (methodology), lists
the selection criteria and the light error corrections it benchmarks:
* WT: score an activation entry by the size of the weight it multiplies
  (Amber-Pruner also scores activations by weight size);
* S-PTS: a static per-token shift (centering) that brings activations close
  to zero before they are sparsified;
* VAR: a variance correction after sparsification that restores the scale
  of the output;
and section 3 names S-PTS and VAR as the strongest light corrections.

The page gives no formulas.  Readings taken here (the plainest the rest
supports):
* shift: a static vector ``mu[d]`` (fp16), the same for every token:
  ``x' = fp16(fp32(x) - fp32(mu))`` (one fp32 subtraction, rounded to
  nearest even); the output adds back the product with the shift,
  ``y = W s(x') + W mu``, so nothing is lost when nothing is dropped;
* weight size: ``c_i = ||W[:, i]||_2`` (the column entry i multiplies, as in
  the RaNA masker), ``score_i = |x'_i| * c_i`` (one fp64 multiply);
* selection on the score: a threshold (``score >= t`` and ``x' != 0``, as the
  magnitude threshold) or N of every M consecutive entries (largest scores,
  ties to the lower index);
* variance correction: the kept entries are scaled by
  ``alpha = sqrt(sum x'^2 / sum_kept x'^2)`` (1 when none is kept), which
  restores the row's second moment; applied to the output, ``y = alpha W s +
  W mu``.
"""

from __future__ import annotations

import numpy as np

from . import gemv, sparsify


def shift(x, mu) -> np.ndarray:
    """``x' = fp16(fp32(x) - fp32(mu))``; ``mu`` None means no shift."""
    x = np.asarray(x, dtype=np.float16)
    if mu is None:
        return x.copy()
    d = np.asarray(x, dtype=np.float32) - np.asarray(mu, dtype=np.float16).astype(np.float32)
    return d.astype(np.float16)


def scores(xs, colnorm) -> np.ndarray:
    """``|x'_i| * c_i`` in fp64 (``|x'_i|`` alone when ``colnorm`` is None)."""
    a = np.abs(np.asarray(xs, dtype=np.float16).astype(np.float64))
    return a if colnorm is None else a * np.asarray(colnorm, dtype=np.float64)


def threshold_keep(xs, colnorm, t: float) -> np.ndarray:
    """Keep entry i iff ``score_i >= t`` and ``x'_i != 0``."""
    xs = np.asarray(xs, dtype=np.float16)
    return (scores(xs, colnorm) >= float(t)) & (xs.astype(np.float64) != 0)


def nm_keep(xs, colnorm, n: int, m: int) -> np.ndarray:
    """N of every M consecutive entries: largest scores, ties to the lower
    index (a stable sort of each group by decreasing score)."""
    s = scores(xs, colnorm)
    d = len(s)
    assert d % m == 0
    keep = np.zeros(d, dtype=bool)
    for g in range(0, d, m):
        order = sorted(range(m), key=lambda j: (-s[g + j], j))
        keep[g + np.array(order[:n], dtype=np.int64)] = True
    return keep


def var_alpha(xs, keep) -> float:
    """``sqrt(sum x'^2 / sum_kept x'^2)``; 1 when no entry is kept."""
    v = np.asarray(xs, dtype=np.float16).astype(np.float64)
    kept = float(np.sum(v[np.asarray(keep)] ** 2))
    if kept == 0.0:
        return 1.0
    return float(np.sqrt(np.sum(v ** 2) / kept))


def column_norms(wt) -> np.ndarray:
    """``c_i = ||W[:, i]||_2`` = the norm of row i of ``WT`` (fp64)."""
    return np.sqrt(np.sum(np.asarray(wt).astype(np.float64) ** 2, axis=1))


def corrected_gemv(wt, x, mu, colnorm, keep_fn, var: bool):
    """One row: ``x' = shift(x, mu)``, ``keep = keep_fn(x', colnorm)``,
    ``y = alpha * W (keep ⊙ x') + W mu`` (alpha = 1 without ``var``).
    Returns ``(xs, keep, alpha, y)``."""
    xs = shift(x, mu)
    keep = keep_fn(xs, colnorm)
    alpha = var_alpha(xs, keep) if var else 1.0
    y = alpha * gemv.masked_gemv(wt, xs, keep)
    if mu is not None:
        y = y + gemv.dense_gemv(wt, np.asarray(mu, dtype=np.float16))
    return xs, keep, alpha, y


def plain_threshold_keep(xs, t):
    """The unshifted, unweighted rule, for the reductions the tests check."""
    return sparsify.threshold_sparsify(xs, t)[0]
