"""GPU parity of ssm_ssd_fwd (the scan with a scalar transition per head, in chunks
of MFMA matrix products) against the fp64 oracle, through the C ABI.

The oracle is the scan's with the head's step, A, D and bias broadcast over the
head's channels; it is pinned against the dense structured mixing matrix in
tests/test_oracle_pins.py.  The GPU path takes bf16 operands in its matrix
products and accumulates in fp32; outputs are bf16, so the bf16 bound applies:
|x - x_ref| <= 2e-2 * (1 + |x_ref|), elementwise on y and on the last state.
Cases: state sizes 16..128, ragged lengths around the 128-step chunk (and 64) and the
1024-step segment the chunk states are chained along, every flag,
an initial state, the empty sequence, determinism, agreement with ssm_scan_fwd
on broadcast inputs, the mid-size workload in full and the long workload
(b1 L65536 H80 P64 N64) on sampled heads.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu

BASE = workloads.SsdWorkload("ssd_small", b=2, L=150, H=3, N=32, with_bias=True)


def make(w, seed, with_h0=False, backend="numpy"):
    import torch

    dev = "cpu" if backend == "numpy" else "cuda"
    x = to_device(workloads.make_ssd_inputs(w, seed=seed, device=dev, backend=backend))
    x["h0"] = (torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed + 5)).to("cuda")
               if with_h0 else None)
    return x


def gpu_ssd(x):
    import torch

    import selective_state_space_35_amd as ssm

    y, last = ssm.ssm_ssd_fwd(x["x"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                              x["softplus"], initial_state=x["h0"])
    torch.cuda.synchronize()
    return y, last


def check(x, what, heads=None):
    y, last = gpu_ssd(x)
    xs, dl, A, D, z, bias, h0 = x["x"], x["delta"], x["A"], x["D"], x["z"], x["delta_bias"], x["h0"]
    if heads is not None:  # heads are independent: the oracle on a subset of heads
        import torch

        P = 64
        ch = torch.cat([torch.arange(h * P, (h + 1) * P) for h in heads.tolist()]).to(xs.device)
        xs, y = xs.index_select(2, ch), y.index_select(2, ch)
        z = None if z is None else z.index_select(2, ch)
        last = last.index_select(1, ch)
        h0 = None if h0 is None else h0.index_select(1, ch)
        dl, A = dl.index_select(2, heads), A.index_select(0, heads)
        D = None if D is None else D.index_select(0, heads)
        bias = None if bias is None else bias.index_select(0, heads)
    y_ref, last_ref = oracle.ssd(xs, dl, A, x["B"], x["C"], D, z, bias, x["softplus"], h0=h0)
    ey = max_normalised_error(oracle.to_f64(y), y_ref)
    el = max_normalised_error(oracle.to_f64(last), last_ref)
    print(f"[parity] {what}: y {ey:.2e}, last_state {el:.2e} (bound {TOL['bf16']:.0e})", flush=True)
    assert ey <= TOL["bf16"], f"{what}: y error {ey:.3e}"
    assert el <= TOL["bf16"], f"{what}: last_state error {el:.3e}"


@pytest.mark.parametrize("N", [16, 32, 48, 64, 96, 128])
def test_state_sizes(N):
    w = BASE.with_shape(N=N)
    say(f"ssd N={N}")
    check(make(w, N, with_h0=True), f"ssd N={N}")


@pytest.mark.parametrize("gate,with_D,with_bias,softplus", [
    (False, False, False, True), (True, False, True, True), (False, True, False, False), (True, True, True, False)])
def test_flags(gate, with_D, with_bias, softplus):
    w = BASE.with_shape(gate=gate, with_D=with_D, with_bias=with_bias, softplus=softplus)
    x = make(w, 3, with_h0=True)
    if not softplus:  # the step as given: keep it positive (retention below one)
        x["delta"] = (x["delta"].float().abs() * 0.05 + 0.01).to(x["delta"].dtype)
        if x["delta_bias"] is not None:
            x["delta_bias"] = x["delta_bias"].abs()
    say(f"ssd flags gate={gate} D={with_D} bias={with_bias} softplus={softplus}")
    check(x, f"ssd flags z={gate} D={with_D} bias={with_bias} sp={softplus}")


@pytest.mark.parametrize("L", [1, 5, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 400])
def test_lengths(L):
    w = BASE.with_shape(L=L, H=2, N=64)
    say(f"ssd L={L}")
    check(make(w, 10 + L, with_h0=True), f"ssd L={L}")


@pytest.mark.parametrize("L,b,with_h0", [(1023, 1, True), (1024, 1, False), (1025, 2, True), (2049, 1, True),
                                         (3 * 1024 + 130, 1, False)])
def test_segment_edges(L, b, with_h0):
    """Lengths around the 1024-step segments of 8 chunks that the chunk states are chained along."""
    w = BASE.with_shape(L=L, b=b, H=1, N=32)
    say(f"ssd segment edge L={L} b={b} h0={with_h0}")
    check(make(w, 50 + L, with_h0=with_h0), f"ssd segment edge L={L}")


def test_empty_sequence_and_no_heads():
    import torch

    w = BASE.with_shape(L=0)
    x = make(w, 1, with_h0=True)
    say("ssd L=0")
    y, last = gpu_ssd(x)
    assert y.shape == (w.b, 0, w.E) and torch.equal(last, x["h0"])


def test_deterministic():
    import torch

    w = BASE.with_shape(L=500, H=4, N=64)
    x = make(w, 7, with_h0=True)
    say("ssd determinism")
    (y1, l1), (y2, l2) = gpu_ssd(x), gpu_ssd(x)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)


def test_agrees_with_the_general_scan():
    """The same problem through ssm_scan_fwd_from with broadcast inputs: both GPU paths agree."""
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=300, H=3, N=16)
    x = make(w, 8, with_h0=True)
    say("ssd vs general scan")
    y, last = gpu_ssd(x)
    P = 64
    rep = lambda v: v.repeat_interleave(P, dim=-1).contiguous()
    A_full = x["A"].repeat_interleave(P)[:, None].expand(w.E, w.N).contiguous()
    y2, last2 = ssm.ssm_scan_fwd(x["x"], rep(x["delta"]), A_full, x["B"], x["C"], rep(x["D"]), x["z"],
                                 rep(x["delta_bias"]), True, initial_state=x["h0"])
    torch.cuda.synchronize()
    assert max_normalised_error(oracle.to_f64(y), oracle.to_f64(y2)) <= TOL["bf16"]
    assert max_normalised_error(oracle.to_f64(last), oracle.to_f64(last2)) <= TOL["bf16"]


def test_mid_workload_full():
    w = workloads.SSD_MID
    say(f"ssd {w.description}")
    check(make(w, 0), "ssd mid")


def test_long_workload_all_heads():
    """b1 L65536 H80 P64 N64 bf16: every head against the oracle, 16 heads (1024 channels) per oracle call."""
    import torch

    w = workloads.SSD_LONG
    x = make(w, 0, backend="torch")
    for h0 in range(0, w.H, 16):
        heads = torch.arange(h0, min(h0 + 16, w.H), device="cuda")
        say(f"ssd {w.description}, heads {h0}..{int(heads[-1])}")
        check(x, f"ssd long (heads {h0}..{int(heads[-1])})", heads=heads)
