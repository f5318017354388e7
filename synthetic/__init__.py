"""Seeded synthetic inputs for the activation-sparse linear layers.

This module is the only code shared by the HIP path's callers (tests, bench,
smoke) and the CPU oracle.  It draws random numbers and casts them to fp16; it
holds none of the method's arithmetic (no thresholds, no quantiles, no masks,
no products).

Recipe (all draws use numpy's PCG64 ``default_rng(seed)``):

* values are drawn in fp32 and cast to fp16 with round-to-nearest-even;
* a weight ``W`` of shape ``d_out x d_in`` is produced directly in its stored
  transposed form ``WT[d_in][d_out]`` (entries are i.i.d., so the orientation
  of the draw does not change the distribution);
* ``N(0, s)`` means standard deviation ``s``; ``Laplace(0, b)`` means scale ``b``.

Seeds: the activation of case ``s`` uses seed ``s``; weight ``j`` of a layer
uses ``1000 + j`` in the order q, k, v, o, gate, up, down; the calibration
samples of projection input ``i`` use ``2000 + i``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "gaussian_f16",
    "laplace_f16",
    "weight_t",
    "LLAMA2_7B",
    "LLAMA2_7B_INPUTS",
    "LLAMA2_7B_FUSED",
    "fused_weight_t",
    "rank_adapter_weights",
    "LLAMA3_8B_MLP",
    "LLAMA3_8B_KV",
    "weight_seed",
    "calib_seed",
    "calibration_samples",
    "topk_k",
]


def gaussian_f16(shape, std: float, seed: int) -> np.ndarray:
    """i.i.d. N(0, std) draws, fp32 then rounded to fp16."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return v.astype(np.float16)


def laplace_f16(shape, scale: float, seed: int) -> np.ndarray:
    """i.i.d. Laplace(0, scale) draws, rounded to fp32 then to fp16."""
    rng = np.random.default_rng(seed)
    v = rng.laplace(0.0, scale, size=shape).astype(np.float32)
    return v.astype(np.float16)


def weight_t(d_out: int, d_in: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Transposed weight ``WT[d_in][d_out]`` (W stored column-major), N(0, std)."""
    return gaussian_f16((d_in, d_out), std, seed)


# Llama-2-7B decoder layer projections: name -> (d_out, d_in, input name).
LLAMA2_7B = {
    "q": (4096, 4096, "attn_in"),
    "k": (4096, 4096, "attn_in"),
    "v": (4096, 4096, "attn_in"),
    "o": (4096, 4096, "o_in"),
    "gate": (11008, 4096, "mlp_in"),
    "up": (11008, 4096, "mlp_in"),
    "down": (4096, 11008, "down_in"),
}
# Projection inputs: name -> (length, distribution).  Block inputs are N(0,1);
# the down-projection input is Laplace(0,1).
LLAMA2_7B_INPUTS = {
    "attn_in": (4096, "gaussian"),
    "o_in": (4096, "gaussian"),
    "mlp_in": (4096, "gaussian"),
    "down_in": (11008, "laplace"),
}
# Projections that read the same input, fused into one weight whose outputs
# are the members' outputs in order: name -> (members, input name).
LLAMA2_7B_FUSED = {
    "qkv": (("q", "k", "v"), "attn_in"),
    "gateup": (("gate", "up"), "mlp_in"),
}
_WEIGHT_ORDER = ["q", "k", "v", "o", "gate", "up", "down"]
_INPUT_ORDER = ["attn_in", "o_in", "mlp_in", "down_in"]

# Llama-3-8B MLP: d_model 4096, d_ff 14336.
LLAMA3_8B_MLP = {"d_model": 4096, "d_ff": 14336}
# Llama-3-8B k and v projections (grouped-query attention, 8 key/value heads
# of 128): d_out 1024, d_in 4096, input like the Llama-2-7B block input.
LLAMA3_8B_KV = {"d_out": 1024, "d_in": 4096, "input": "attn_in"}


def weight_seed(name: str) -> int:
    return 1000 + _WEIGHT_ORDER.index(name)


def fused_weight_t(name: str) -> np.ndarray:
    """``WT`` of a fused projection: the members' seeded ``WT[d_in][d_out]``
    side by side, so output block j is member j's output."""
    members, _ = LLAMA2_7B_FUSED[name]
    return np.concatenate(
        [weight_t(LLAMA2_7B[m][0], LLAMA2_7B[m][1], weight_seed(m)) for m in members], axis=1)


def rank_adapter_weights(d_out: int, d_in: int, r: int, seed: int, std: float = 0.02):
    """Seeded rank-adapter factors as stored: ``(BT[d_in][r], AT[r][d_out])``
    for ``y = A (m ⊙ B x)`` with ``B`` r x d_in and ``A`` d_out x r, both
    N(0, std) (the pages give no trained factors)."""
    return weight_t(r, d_in, seed, std), weight_t(d_out, r, seed + 1, std)


def calib_seed(input_name: str) -> int:
    return 2000 + _INPUT_ORDER.index(input_name)


def activation(shape, dist: str, seed: int) -> np.ndarray:
    """Activation draw: ``gaussian`` = N(0,1), ``laplace`` = Laplace(0,1)."""
    if dist == "gaussian":
        return gaussian_f16(shape, 1.0, seed)
    if dist == "laplace":
        return laplace_f16(shape, 1.0, seed)
    raise ValueError(dist)


def calibration_samples(input_name: str, n: int = 10_000) -> np.ndarray:
    """``n`` scalar samples from a projection input's distribution (fp16)."""
    _, dist = LLAMA2_7B_INPUTS[input_name]
    return activation((n,), dist, calib_seed(input_name))


def swiglu_gate_up(d_ff: int, d_model: int, seed: int):
    """Synthetic gate and up pre-activations ``g``, ``u`` (fp16).

    They stand in for ``W_g x`` and ``W_u x`` with ``W ~ N(0, 0.02)`` and
    ``x ~ N(0, 1)`` of length ``d_model``: each entry of such a product is
    N(0, 0.02 * sqrt(d_model)), and the draws here use that distribution
    directly so that no GEMV result enters the inputs.
    """
    std = 0.02 * float(np.sqrt(d_model))
    g = gaussian_f16((d_ff,), std, 3000 + seed)
    u = gaussian_f16((d_ff,), std, 4000 + seed)
    return g, u


def topk_k(pct: int, d: int) -> int:
    """K for a Top-K percentage: ``pct`` percent of ``d``, rounded half up."""
    return (pct * d + 50) // 100
