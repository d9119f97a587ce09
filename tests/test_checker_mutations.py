"""The parity checker must reject plausible wrong outputs at the bounds it is used with.

Wrong outputs are produced on the CPU by the oracle itself with a planted
mistake (zeroed last state, output shifted one step, the carry dropped at
chunk boundaries, one state coordinate omitted) on inputs drawn with the
mid-size (bf16) and block (fp32) workload recipes at reduced width.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.parity import TOL, within


def _inputs(w):
    x = workloads.make_scan_inputs(w, seed=3)
    return {k: (oracle.to_f64(v) if hasattr(v, "shape") else v) for k, v in x.items()}


def _scan(x, h0=None, n_keep=None, sl=slice(None)):
    A, B, C = x["A"], x["B"][:, sl], x["C"][:, sl]
    if n_keep is not None:
        A, B, C = A[:, :n_keep], B[..., :n_keep], C[..., :n_keep]
    return oracle.scan(x["u"][:, sl], x["delta"][:, sl], A, B, C, x["D"],
                       None if x["z"] is None else x["z"][:, sl], x["delta_bias"], x["softplus"], h0=h0)


def _dropped_carry(x, every):
    L = x["u"].shape[1]
    ys, last = [], None
    for t0 in range(0, L, every):
        y, last = _scan(x, sl=slice(t0, min(t0 + every, L)))  # every segment restarts from zero
        ys.append(y)
    return np.concatenate(ys, axis=1), last


CASES = [
    ("bf16", workloads.MID.with_shape(b=1, L=2048, E=32)),
    ("f32", workloads.BLOCK.with_shape(b=2, L=512, E=32)),
]


@pytest.mark.parametrize("kind,w", CASES, ids=[c[0] for c in CASES])
def test_checker_rejects_mutations(kind, w):
    x = _inputs(w)
    tol = TOL[kind]
    y_ref, last_ref = _scan(x)
    assert within(y_ref, y_ref, tol) and within(last_ref, last_ref, tol)
    # last_state = 0
    assert not within(np.zeros_like(last_ref), last_ref, tol)
    # y shifted by one step
    y_shift = np.concatenate([y_ref[:, :1], y_ref[:, :-1]], axis=1)
    assert not within(y_shift, y_ref, tol)
    # carry dropped at chunk boundaries
    for every in (64, 256):
        y_drop, last_drop = _dropped_carry(x, every)
        assert not within(y_drop, y_ref, tol), f"dropped carry every {every} not caught"
    # state n = N-1 omitted
    y_miss, last_miss = _scan(x, n_keep=w.N - 1)
    assert not within(y_miss, y_ref, tol)
