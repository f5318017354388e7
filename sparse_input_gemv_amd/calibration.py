"""Calibrated magnitude thresholds, kept in a JSON file between runs.

TEAL README, Inference Usage: thresholds are calibrated once per model and
shipped with it, and sparse inference loads them instead of calibrating
again.  Here the thresholds come from the library's calibration kernel
(``act_calibrate_threshold``) on samples of each projection input; this
module only runs that kernel, stores its results and reads them back.
Nothing here computes a threshold on the host.

File layout (one JSON object)::

    {"format": "sparse_act.thresholds", "version": 1,
     "inputs": {"<name>": {"samples": <n>,
                           "thresholds": {"<sparsity>": <t>, ...}}, ...},
     "meta": {...}}

Sparsity keys are the fractions as ``repr(float)``; thresholds are the
kernel's fp32 values as JSON numbers, which read back exactly.  ``meta`` is
free-form (model, dtype, date) and is not interpreted.
"""

from __future__ import annotations

import json
import math
import os
from typing import Mapping, Sequence

FORMAT = "sparse_act.thresholds"
VERSION = 1


def _key(sparsity: float) -> str:
    s = float(sparsity)
    if not (0.0 <= s <= 1.0):
        raise ValueError(f"sparsity {sparsity!r} is outside [0, 1]")
    return repr(s)


def calibrate(samples: Mapping[str, "object"], sparsities: Sequence[float],
              meta: Mapping | None = None) -> dict:
    """Thresholds for every input and sparsity, from the calibration kernel.

    ``samples`` maps an input name (e.g. "down_in") to a 1-D fp16 CUDA
    tensor of its calibration activations.  Returns the file's object.
    """
    import sparse_input_gemv_amd as sa

    inputs = {}
    for name, x in samples.items():
        if not isinstance(name, str) or not name:
            raise ValueError("input names must be non-empty strings")
        th = {}
        for s in sparsities:
            t = sa.act_calibrate_threshold(x, float(s))
            th[_key(s)] = float(t.cpu()[0])
        inputs[name] = {"samples": int(x.numel()), "thresholds": th}
    return {"format": FORMAT, "version": VERSION, "inputs": inputs, "meta": dict(meta or {})}


def validate(cal: Mapping) -> dict:
    """The object if it is a well-formed threshold file; else ValueError."""
    if not isinstance(cal, Mapping) or cal.get("format") != FORMAT:
        raise ValueError(f"not a {FORMAT} object")
    if cal.get("version") != VERSION:
        raise ValueError(f"unsupported version {cal.get('version')!r} (expected {VERSION})")
    inputs = cal.get("inputs")
    if not isinstance(inputs, Mapping):
        raise ValueError("'inputs' must be an object")
    for name, ent in inputs.items():
        if not isinstance(ent, Mapping) or not isinstance(ent.get("thresholds"), Mapping):
            raise ValueError(f"input {name!r}: 'thresholds' must be an object")
        n = ent.get("samples")
        if not isinstance(n, int) or isinstance(n, bool) or n < 1:
            raise ValueError(f"input {name!r}: 'samples' must be a positive integer")
        for k, t in ent["thresholds"].items():
            try:
                _key(float(k))
            except (TypeError, ValueError):
                raise ValueError(f"input {name!r}: bad sparsity key {k!r}") from None
            if (not isinstance(t, (int, float)) or isinstance(t, bool) or not math.isfinite(t)
                    or t < 0):
                raise ValueError(f"input {name!r}: threshold {t!r} is not a finite value >= 0")
    if not isinstance(cal.get("meta", {}), Mapping):
        raise ValueError("'meta' must be an object")
    return dict(cal)


def save(cal: Mapping, path: str | os.PathLike) -> None:
    """Write a validated threshold object (atomically: a temporary file, then rename)."""
    obj = validate(cal)
    tmp = f"{os.fspath(path)}.tmp"
    with open(tmp, "w") as f:
        json.dump(obj, f, indent=1, sort_keys=True)
        f.write("\n")
    os.replace(tmp, path)


def load(path: str | os.PathLike) -> dict:
    """Read and validate a threshold file."""
    with open(path) as f:
        return validate(json.load(f))


def threshold(cal: Mapping, name: str, sparsity: float) -> float:
    """The stored threshold of input ``name`` at ``sparsity`` (KeyError if absent)."""
    return float(cal["inputs"][name]["thresholds"][_key(sparsity)])
