"""Write the oracle regression fixtures in this folder.

Calls only ``oracle/`` (and the seeded generators in ``workloads/``).  The
fixtures freeze the oracle's output on the tiny workload so an accidental
change to the oracle's arithmetic shows up as a failing test; they are not an
independent pin (the pins live in tests/test_oracle_pins.py).  No page prints
input/output values for a reproducible worked example, so there is no
page-sourced golden.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.TINY
    x = workloads.make_scan_inputs(w, seed=0)
    y, last = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                          x["softplus"], threads=1)
    doc = {
        "what": "oracle regression fixture: tiny workload (b1 L64 E16 N4 fp32, softplus, D, no gate), seed 0",
        "source": "written by tests/golden/make_golden.py from oracle.scan; inputs from workloads.make_scan_inputs",
        "workload": w.name,
        "seed": 0,
        "y": [float(v) for v in y.ravel()],
        "last_state": [float(v) for v in last.ravel()],
    }
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote tiny_seed0.json")


if __name__ == "__main__":
    main()
