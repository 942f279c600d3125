"""Stored expected values of one small fp32 layer (tests/golden/tiny_layer.json,
written by tests/golden/make_golden.py, which calls only the oracle).

The CPU test guards the oracle against unintended changes of its arithmetic
(a change must regenerate the file, and its commit names the passage that
justifies it); the GPU test checks the library against the stored values:
selection and dispatch bit-exact, the fp32 layer output within max-abs 1e-5.
Inputs are drawn on the CPU by workloads.make_inputs and copied to the device.
"""
import json
import os

import numpy as np
import pytest
import torch

from gpu_helpers import make_layer, need_gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load():
    import sys
    sys.path.insert(0, GOLDEN)
    import make_golden
    with open(os.path.join(GOLDEN, "tiny_layer.json")) as f:
        return make_golden, json.load(f)


def test_oracle_reproduces_the_stored_layer():
    mg, ref = _load()
    got = mg.compute()
    assert got["workload"] == ref["workload"]
    for key in ("ids", "counts", "offsets", "perm", "pos"):
        assert got[key] == ref[key], key
    for key in ("logits32", "weights", "out"):
        np.testing.assert_allclose(np.array(got[key]), np.array(ref[key]), rtol=1e-12, atol=1e-12, err_msg=key)
    # the case is not degenerate: two experts get no rows, every token's two
    # weights sum to 1 (renorm), and the output is not tiny
    assert ref["counts"].count(0) >= 1
    assert np.allclose(np.array(ref["weights"]).sum(1), 1.0)
    assert np.sqrt(np.mean(np.array(ref["out"]) ** 2)) > 0.1


@pytest.mark.gpu
def test_library_matches_the_stored_layer():
    need_gpu()
    mg, ref = _load()
    from workloads import make_inputs
    w = mg.WORKLOAD
    inp = {k: v.cuda() for k, v in make_inputs(w, device="cpu").items()}
    layer = make_layer(w, inp)
    out = layer.forward(inp["x"])
    torch.cuda.synchronize()
    s = layer.last
    assert s["ids"].cpu().tolist() == ref["ids"]
    for key in ("counts", "offsets", "perm", "pos"):
        assert s[key].cpu().tolist() == ref[key], key
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - np.array(ref["out"]))))
    assert err <= 1e-5, err
