"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the same inputs."""
import sys

import numpy as np

import oracle
import workloads
from tests.parity import TOL, max_normalised_error


def say(msg):
    """Name the case before each GPU step so a failing run can be traced."""
    print(f"[gpu-case] {msg}", flush=True)


def to_device(inputs, device="cuda"):
    return {k: (v.to(device) if hasattr(v, "to") else v) for k, v in inputs.items()}


def gpu_scan(x, return_last_state=True, tuning=None):
    import torch

    import selective_state_space_35_amd as ssm

    y, last = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                               x["softplus"], return_last_state=return_last_state, tuning=tuning)
    torch.cuda.synchronize()
    return y, last


def oracle_scan(x, channels=None, batches=None):
    """Oracle on the same tensors; optionally only on a subset of channels / batch rows.

    Channels and batch rows are independent chains, so the oracle of a subset is
    exactly the subset of the oracle.
    """
    def sel(t, ch_axis, b_axis=0):
        if t is None:
            return None
        if batches is not None:
            t = t.index_select(b_axis, batches)
        if channels is not None and ch_axis is not None:
            t = t.index_select(ch_axis, channels)
        return t

    u, delta, z = sel(x["u"], 2), sel(x["delta"], 2), sel(x["z"], 2)
    B, C = sel(x["B"], None), sel(x["C"], None)
    A = x["A"] if channels is None else x["A"].index_select(0, channels)
    D = x["D"] if (x["D"] is None or channels is None) else x["D"].index_select(0, channels)
    bias = x["delta_bias"]
    if bias is not None and channels is not None:
        bias = bias.index_select(0, channels)
    return oracle.scan(u, delta, A, B, C, D, z, bias, x["softplus"])


def pick(t, channels=None, batches=None, ch_axis=2):
    if batches is not None:
        t = t.index_select(0, batches)
    if channels is not None:
        t = t.index_select(ch_axis, channels)
    return oracle.to_f64(t)


def check_scan(x, kind, what, channels=None, batches=None, y=None, last=None, tuning=None):
    """Run GPU (unless outputs given) and oracle; assert the elementwise bound on y and last_state."""
    if y is None:
        y, last = gpu_scan(x, tuning=tuning)
    y_ref, last_ref = oracle_scan(x, channels, batches)
    ey = max_normalised_error(pick(y, channels, batches), y_ref)
    el = max_normalised_error(pick(last, channels, batches, ch_axis=1), last_ref)
    tol = TOL[kind]
    print(f"[parity] {what}: max normalised error y {ey:.3e}, last_state {el:.3e} (bound {tol:.0e})", flush=True)
    assert ey <= tol, f"{what}: y error {ey:.3e} > {tol}"
    assert el <= tol, f"{what}: last_state error {el:.3e} > {tol}"
    return ey, el


def sample_channels(E, device, k=64, seed=0):
    """First, last and middle 64-channel blocks plus random channels (sorted, unique)."""
    import torch

    rng = np.random.default_rng(seed)
    parts = [np.arange(0, min(64, E)), np.arange(max(0, E - 64), E), np.arange(E // 2, min(E, E // 2 + 64)),
             rng.choice(E, size=min(k, E), replace=False)]
    ch = np.unique(np.concatenate(parts))
    return torch.from_numpy(ch).to(device)
