"""GPU parity of ssm_scan_fwd_save and ssm_scan_bwd_saved through the C ABI.

The forward keeps the state every 64 steps and the backward takes those states
in place of the chunk states it would otherwise recompute.

* saved states against the fp64 oracle: saved[:, k] is the last state of the
  oracle's scan over the first 64 (k + 1) steps;
* y and last_state of ssm_scan_fwd_save equal ssm_scan_fwd_from's bit for bit
  (same kernels; saving only adds stores);
* ssm_scan_bwd_saved's gradients against the oracle's backward, with the
  forward cut into chunks that do not line up with the 64-step interval
  (forced chunk lengths 40 and 200) and in one piece;
* lengths at the interval's edges (1, 64, 65, 128, 129);
* the long workload at full size (b1 L65536 E5120 N16 bf16), all channels.

Bounds as in the other parity tests: tol * (1 + |ref|) elementwise, tol = 1e-4
for fp32 I/O and 2e-2 for bf16 I/O.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import say, to_device
from tests.parity import TOL, max_normalised_error
from tests.test_gpu_bwd import NAMES, ORACLE_NAME, make, oracle_bwd

pytestmark = pytest.mark.gpu

BASE = workloads.ScanWorkload("saved_small", b=2, L=300, E=70, N=16, dtype="f32", u=workloads.N01,
                              delta=("normal", -1.0, 0.7), z=workloads.N01, B=workloads.N01, C=workloads.N01,
                              D=workloads.N01, delta_bias=("normal", 0.0, 0.3), softplus=True)


def fwd_save(x, tuning=None):
    import torch

    import selective_state_space_35_amd as ssm

    y, last, saved = ssm.ssm_scan_fwd_save(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                           x["delta_bias"], x["softplus"], initial_state=x["h0"], tuning=tuning)
    torch.cuda.synchronize()
    return y, last, saved


def bwd_saved(x, saved):
    import torch

    import selective_state_space_35_amd as ssm

    g = ssm.ssm_scan_bwd_saved(x["u"], x["delta"], x["A"], x["B"], x["C"], x["dy"], saved, x["D"], x["z"],
                               x["delta_bias"], x["softplus"], initial_state=x["h0"], d_last_state=x["dlast"])
    torch.cuda.synchronize()
    return g


def check_grads(got, ref, kind, what):
    worst = {}
    for name in NAMES:
        r = ref[ORACLE_NAME.get(name, name)]
        if r is None:
            assert got[name] is None, f"{what}: {name} returned without its input"
            continue
        worst[name] = max_normalised_error(oracle.to_f64(got[name]), r)
    print(f"[parity] {what}: " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()) + f" (bound {TOL[kind]:.0e})",
          flush=True)
    for name, err in worst.items():
        assert err <= TOL[kind], f"{what}: {name} error {err:.3e} > {TOL[kind]}"


def force_chunks(min_chunk):
    """The chunked form cut into chunks of min_chunk steps or more (None: the plan the sizes give)."""
    return {"path": "chunked", "min_chunk": min_chunk, "target_waves": 100000} if min_chunk else None


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("min_chunk", [None, 40, 200])
def test_saved_states_are_the_prefix_states(dtype, min_chunk):
    import torch

    import selective_state_space_35_amd as ssm

    tune = force_chunks(min_chunk)
    w = BASE.with_shape(dtype=dtype)
    x = make(w, seed=3, with_h0=True)
    say(f"saved states {dtype} min_chunk={min_chunk} plan={ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype, tune)}")
    y, last, saved = fwd_save(x, tune)
    assert saved.shape == ssm.saved_states_shape(w.b, w.L, w.E, w.N) == (w.b, 4, w.E, w.N)
    y0, last0 = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                 x["softplus"], initial_state=x["h0"], tuning=tune)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(last, last0)
    worst = 0.0
    for k in range(saved.shape[1]):
        Lk = 64 * (k + 1)
        _, ref = oracle.scan(x["u"][:, :Lk], x["delta"][:, :Lk], x["A"], x["B"][:, :Lk], x["C"][:, :Lk], x["D"],
                             x["z"][:, :Lk], x["delta_bias"], x["softplus"], h0=x["h0"])
        worst = max(worst, max_normalised_error(oracle.to_f64(saved[:, k]), ref))
    print(f"[parity] saved states {dtype} min_chunk={min_chunk}: {worst:.2e} (bound {TOL[dtype]:.0e})", flush=True)
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("dtype,with_h0,with_dlast,min_chunk", [
    ("f32", True, True, None), ("f32", False, False, 40), ("bf16", True, False, 200), ("bf16", False, True, 40)])
def test_backward_from_saved_states(dtype, with_h0, with_dlast, min_chunk):
    tune = force_chunks(min_chunk)
    w = BASE.with_shape(dtype=dtype)
    x = make(w, seed=5, with_h0=with_h0, with_dlast=with_dlast)
    say(f"bwd from saved states {dtype} h0={with_h0} dlast={with_dlast} min_chunk={min_chunk}")
    _, _, saved = fwd_save(x, tune)
    check_grads(bwd_saved(x, saved), oracle_bwd(x), dtype, f"bwd saved {dtype} h0={with_h0} min_chunk={min_chunk}")


@pytest.mark.parametrize("L", [1, 64, 65, 128, 129])
def test_interval_edges(L):
    w = BASE.with_shape(L=L, E=40)
    x = make(w, seed=L, with_h0=True, with_dlast=True)
    say(f"saved interval edge L={L}")
    _, _, saved = fwd_save(x)
    assert saved.shape[1] == max((L + 63) // 64 - 1, 0)
    check_grads(bwd_saved(x, saved), oracle_bwd(x), "f32", f"bwd saved L={L}")


def test_long_workload_full_size():
    """Forward with saved states and the backward from them, b1 L65536 E5120 N16 bf16, against the oracle."""
    w = workloads.LONG
    x = make(w, seed=0, backend="torch")
    say(f"saved fwd + bwd full size {w.description}")
    y, last, saved = fwd_save(x)
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                  x["softplus"])
    assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL["bf16"]
    assert max_normalised_error(oracle.to_f64(last), last_ref) <= TOL["bf16"]
    check_grads(bwd_saved(x, saved), oracle_bwd(x), "bf16", "bwd saved long, full size")
