"""RaNA linear-layer rank adapter, plain fp64 steps (test infrastructure only).

RaNA replies:
* Q5.1 (Eq. 11): the rank adapter replaces each of the up, gate and QKV
  projections by the product ``A (m(x) ⊙ B x)``, where ``m(x)`` is a 0/1
  mask over the ``r`` entries of ``B x``; columns of ``A`` whose mask entry
  is zero take no part.
* Q4 (eqn. 9): the mask compares the element-wise square of ``B x`` with a
  threshold; the unsquared ``B x`` is what the masked product multiplies
  (eqn. 4).
* Q2 (two GEMVs in place of one): a plain GEMV computes ``v = B x``, then a
  masked GEMV computes ``A (m(x) ⊙ v)``.

Readings taken here (the pages leave them open):
* ``m_i = 1`` iff ``v_i ** 2 >= t`` (the comparator the pages print for
  their masks is ``>=``).
* ``v`` is the first GEMV's output in the layer's activation format, fp16.
  The mask is decided on those fp16 values (widened exactly), and the masked
  GEMV multiplies them.  Squaring an fp16 value is exact in fp32 and fp64, so
  the decision has one answer whatever precision computes it.

Both weights are given as stored, transposed: ``BT[d_in][r]`` and
``AT[r][d_out]`` (each row of a transposed weight is the column one
activation entry multiplies).
"""

from __future__ import annotations

import numpy as np

from . import gemv


def adapter_v(bt, x) -> np.ndarray:
    """Step 1: ``v = B x`` in fp64 (``x`` one row, ``BT[d_in][r]``)."""
    return gemv.dense_gemv(bt, x)


def adapter_mask(v16, t: float) -> np.ndarray:
    """Step 2 (eqn. 9): ``m_i = v_i ** 2 >= t`` on the fp16 ``v``."""
    v = np.asarray(v16, dtype=np.float16).astype(np.float64)
    return v * v >= float(t)


def rank_adapter(bt, at, x, t: float, v16=None):
    """``y = A (m(x) ⊙ B x)`` for one row ``x``.

    Returns ``(v, v16, keep, y)``: the fp64 ``B x``, the fp16 ``v`` the mask
    and the second GEMV use (``v16`` when given: the first GEMV's output as
    another implementation stored it; else ``v`` rounded to nearest even),
    the mask, and ``y`` in fp64 over the kept columns of ``A`` only.
    """
    v = adapter_v(bt, x)
    if v16 is None:
        v16 = v.astype(np.float16)
    v16 = np.asarray(v16, dtype=np.float16)
    keep = adapter_mask(v16, t)
    idx = np.flatnonzero(keep)
    y = gemv.sparse_gemv(at, idx, v16[idx])
    return v, v16, keep, y
