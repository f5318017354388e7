"""Persisted thresholds (sparse_input_gemv_amd.calibration).

CPU tests: the file round-trips exactly and malformed files are refused.
GPU test: the stored thresholds are the calibration kernel's, bit for bit,
and a GEMV run with a reloaded threshold gives the same bits as one run
with the fresh threshold.
"""

import json
import math

import numpy as np
import pytest

from sparse_input_gemv_amd import calibration as cal


def _hand_made():
    return {
        "format": cal.FORMAT, "version": cal.VERSION,
        "inputs": {
            "down_in": {"samples": 10000,
                        "thresholds": {repr(0.5): 0.69873046875, repr(0.4): 0.5087890625}},
            "attn_in": {"samples": 10000, "thresholds": {repr(0.6): 0.841552734375}},
            "tiny": {"samples": 1, "thresholds": {repr(0.0): 0.0, repr(1.0): 6.103515625e-05}},
        },
        "meta": {"model": "synthetic llama-2-7b shapes", "dtype": "f16"},
    }


def test_round_trip_is_exact(tmp_path):
    obj = _hand_made()
    # fp32 values that are not short decimals survive too
    obj["inputs"]["down_in"]["thresholds"][repr(0.3)] = float(np.float32(1) / np.float32(3))
    p = tmp_path / "thresholds.json"
    cal.save(obj, p)
    back = cal.load(p)
    assert back == obj
    assert cal.threshold(back, "down_in", 0.5) == 0.69873046875
    assert cal.threshold(back, "down_in", 0.3) == float(np.float32(1) / np.float32(3))
    assert cal.threshold(back, "tiny", 1) == 6.103515625e-05
    assert not (tmp_path / "thresholds.json.tmp").exists()


def test_lookup_misses_raise_key_error():
    obj = cal.validate(_hand_made())
    with pytest.raises(KeyError):
        cal.threshold(obj, "mlp_in", 0.5)
    with pytest.raises(KeyError):
        cal.threshold(obj, "down_in", 0.7)
    with pytest.raises(ValueError):
        cal.threshold(obj, "down_in", 1.5)


@pytest.mark.parametrize("mutate", [
    lambda o: o.update(format="something else"),
    lambda o: o.update(version=2),
    lambda o: o.pop("inputs"),
    lambda o: o.update(inputs=[]),
    lambda o: o["inputs"]["down_in"].pop("thresholds"),
    lambda o: o["inputs"]["down_in"].update(samples=0),
    lambda o: o["inputs"]["down_in"].update(samples=True),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"abc": 0.5}),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"1.5": 0.5}),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"0.5": -1.0}),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"0.5": math.nan}),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"0.5": math.inf}),
    lambda o: o["inputs"]["down_in"]["thresholds"].update({"0.5": "0.7"}),
    lambda o: o.update(meta=[1, 2]),
])
def test_malformed_objects_are_refused(mutate, tmp_path):
    obj = _hand_made()
    mutate(obj)
    with pytest.raises(ValueError):
        cal.validate(obj)
    with pytest.raises(ValueError):
        cal.save(obj, tmp_path / "bad.json")
    (tmp_path / "bad2.json").write_text(json.dumps(obj, allow_nan=True))
    with pytest.raises(ValueError):
        cal.load(tmp_path / "bad2.json")


@pytest.mark.gpu
def test_stored_thresholds_are_the_kernels(tmp_path):
    import torch

    import sparse_input_gemv_amd as sa
    import synthetic as syn
    from oracle import calibrate as ocal

    dev = "cuda:0"
    names = ["attn_in", "o_in", "mlp_in", "down_in"]
    samples = {n: torch.from_numpy(syn.calibration_samples(n)).to(dev) for n in names}
    levels = [0.4, 0.5, 0.6]
    obj = cal.calibrate(samples, levels, meta={"what": "test"})
    p = tmp_path / "thr.json"
    cal.save(obj, p)
    back = cal.load(p)
    for n in names:
        assert back["inputs"][n]["samples"] == samples[n].numel()
        for s in levels:
            t = cal.threshold(back, n, s)
            assert t == float(sa.act_calibrate_threshold(samples[n], s).cpu()[0])
            assert t == float(ocal.magnitude_threshold(syn.calibration_samples(n), s))
    # a GEMV with the reloaded threshold: the same bits as with the fresh one
    wt = torch.from_numpy(syn.weight_t(4096, 11008, syn.weight_seed("down"))).to(dev)
    x = torch.from_numpy(syn.activation((11008,), "laplace", 0)).to(dev)
    t_fresh = float(sa.act_calibrate_threshold(samples["down_in"], 0.5).cpu()[0])
    y0 = sa.sparse_gemv_threshold(wt, x, t_fresh).clone()
    y1 = sa.sparse_gemv_threshold(wt, x, cal.threshold(back, "down_in", 0.5))
    assert torch.equal(y0, y1)
