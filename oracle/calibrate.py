"""Threshold calibration from samples, plain fp64 definition (test infrastructure only).

TEAL README (Inference Usage; Accuracy Usage, step 1): thresholds for a target
sparsity come from per-layer activation histograms built offline.  The pages
give no binning; here the histogram has one bin per fp16 magnitude, so the
threshold is the exact empirical quantile of the sample magnitudes.
"""

from __future__ import annotations

import numpy as np


def quantile_linear(values, s: float) -> float:
    """Linearly interpolated empirical quantile, from its definition.

    Sort ascending: ``v_0 <= ... <= v_{n-1}``; position ``h = (n - 1) s``;
    ``q = v_lo + (h - lo) * (v_{lo+1} - v_lo)`` with ``lo = floor(h)``
    (``v_{lo+1}`` is ``v_lo`` when ``lo = n - 1``).  Each fp64 operation is
    done separately in the order written.
    """
    v = np.sort(np.asarray(values, dtype=np.float64))
    n = v.size
    if n == 0:
        raise ValueError("no samples")
    h = float(n - 1) * float(s)
    lo = int(np.floor(h))
    lo = min(max(lo, 0), n - 1)
    hi = min(lo + 1, n - 1)
    frac = h - float(lo)
    diff = float(v[hi]) - float(v[lo])
    return float(v[lo]) + frac * diff


def magnitude_threshold(samples, sparsity: float) -> np.float32:
    """Threshold ``t`` such that about ``sparsity`` of ``|samples|`` fall below.

    The ``sparsity``-quantile of the fp16 sample magnitudes, rounded to fp32.
    """
    mags = np.abs(np.asarray(samples).astype(np.float64))
    return np.float32(quantile_linear(mags, sparsity))
