"""Oracle regression against the fixture written by tests/golden/make_golden.py."""
import json
import os

import numpy as np

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_seed0_regression():
    with open(os.path.join(HERE, "golden", "tiny_seed0.json")) as f:
        doc = json.load(f)
    w = workloads.SCAN_WORKLOADS[doc["workload"]]
    x = workloads.make_scan_inputs(w, seed=doc["seed"])
    y, last = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                          x["softplus"], threads=1)
    np.testing.assert_allclose(y.ravel(), doc["y"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(last.ravel(), doc["last_state"], rtol=1e-13, atol=1e-15)


def test_generator_is_deterministic():
    a = workloads.make_scan_inputs(workloads.MID.with_shape(b=1, L=64, E=32), seed=5)
    b = workloads.make_scan_inputs(workloads.MID.with_shape(b=1, L=64, E=32), seed=5)
    for k in ("u", "delta", "z", "B", "C", "D", "A"):
        assert a[k].dtype == b[k].dtype and bool((a[k].float() == b[k].float()).all())
