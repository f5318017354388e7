"""Masked SwiGLU down projection, plain fp64 definitions (test infrastructure only).

RaNA replies, Q3, give two neuron masks on the input of the down projection
of a SwiGLU MLP (Eqn. 12 for RaNA):

* CATS:  keep neuron i iff ``|SiLU(gate_i)| >= t``
* RaNA:  keep neuron i iff ``|SiLU(gate_i) * up_i| * ||W_down[:, i]|| >= t``

and Q5.1 says the down projection then skips the weight columns of the
masked neurons.  ``gate`` and ``up`` are the fp16 outputs of the gate and up
projections, given as inputs.
"""

from __future__ import annotations

import numpy as np


def silu(z) -> np.ndarray:
    """``SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))`` in fp64.

    The pages use SiLU without defining it; this is its standard form.
    """
    z = np.asarray(z).astype(np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def column_norms(wdt) -> np.ndarray:
    """``c_i = ||W_down[:, i]||_2`` from the stored ``WdT[d_ff][d_model]``.

    RaNA replies, Q3 (Eqn. 12) write a Frobenius norm of the i-th part of the
    down weight; for one column that is its Euclidean norm.  Column ``i`` of
    ``W_down`` multiplies neuron ``i``, and is row ``i`` of ``WdT``.
    """
    w = np.asarray(wdt).astype(np.float64)
    return np.sqrt((w * w).sum(axis=1))


def hidden(g, u) -> np.ndarray:
    """``h = SiLU(g) ⊙ u``: the input of the down projection (fp64)."""
    return silu(g) * np.asarray(u).astype(np.float64)


def scores(g, u, mode: str, colnorm=None) -> np.ndarray:
    """Masker score per neuron: ``|SiLU(g)|`` (CATS) or ``|h| * c`` (RaNA)."""
    if mode == "cats":
        return np.abs(silu(g))
    if mode == "rana":
        return np.abs(hidden(g, u)) * np.asarray(colnorm, dtype=np.float64)
    raise ValueError(mode)


def masked_swiglu_down(g, u, wdt, t: float, mode: str, colnorm=None):
    """Masked down projection: ``y = sum_{kept i} W_down[:, i] * h_i``.

    Returns ``(keep, y)`` with ``y`` in fp64.  ``t`` is compared in fp64.
    """
    if mode == "rana" and colnorm is None:
        colnorm = column_norms(wdt)
    sc = scores(g, u, mode, colnorm)
    keep = sc >= float(t)
    h = hidden(g, u)
    idx = np.flatnonzero(keep)
    cols = np.asarray(wdt)[idx].astype(np.float64)
    y = (cols * h[idx][:, None]).sum(axis=0)
    return keep, y


def threshold_for_mask_rate(sc, rate: float) -> float:
    """Threshold that masks (about) ``rate`` of the neurons.

    The pages fix no threshold for a mask rate.  With the scores sorted
    ascending, the target cut is after ``floor(rate * n)`` entries; the
    threshold is the midpoint between the two adjacent *distinct* score values
    at the cut nearest that target, so no score lies within half a gap of it.
    """
    s = np.sort(np.asarray(sc, dtype=np.float64))
    n = s.size
    target = int(np.floor(rate * n))
    if target <= 0:
        return 0.0
    if target >= n:
        return float(s[-1] * 2.0 + 1.0)
    # distinct-value cuts: positions j where s[j-1] < s[j]
    cuts = np.flatnonzero(s[1:] > s[:-1]) + 1
    j = int(cuts[np.argmin(np.abs(cuts - target))])
    return float(0.5 * (s[j - 1] + s[j]))
