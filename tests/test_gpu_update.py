"""GPU parity of ssm_state_update against the fp64 oracle, through the C ABI.

Covers the generation workload (b256 E5120 N16, 128 successive updates,
state carried in HBM) at full size with every batch row checked, reduced
sizes with ragged channel counts, every state size 1..16, the vector and
the unaligned (scalar) memory paths, the path that stages x, step, z and y
through LDS (bit for bit against the per-lane one), both dtypes, flags, and
the identity "L token updates == one scan over L".
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import gpu_scan, say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu


def make(w, seed=0, backend="numpy"):
    dev = "cpu" if backend == "numpy" else "cuda"
    return to_device(workloads.make_decode_inputs(w, seed=seed, device=dev, backend=backend))


def run_steps(x, steps, check_rows=None, kind="bf16", what="", state=None):
    """Run `steps` GPU updates; check every y and the final state against the chained oracle."""
    import torch

    import selective_state_space_35_amd as ssm

    st = x["state0"].clone() if state is None else state
    rows = check_rows
    ref_state = oracle.to_f64(st if rows is None else st.index_select(0, rows))
    worst_y = 0.0
    for k in range(steps):
        y = ssm.ssm_state_update(st, x["x"][k], x["delta"][k], x["A"], x["B"][k], x["C"][k], x["D"],
                                 None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"])
        sel = (lambda t: t) if rows is None else (lambda t: t.index_select(0, rows))
        ref_state, y_ref = oracle.state_update(
            ref_state, sel(x["x"][k]), sel(x["delta"][k]), x["A"], sel(x["B"][k]), sel(x["C"][k]), x["D"],
            None if x["z"] is None else sel(x["z"][k]), x["delta_bias"], x["softplus"])
        torch.cuda.synchronize()
        worst_y = max(worst_y, max_normalised_error(oracle.to_f64(sel(y)), y_ref))
    es = max_normalised_error(oracle.to_f64(st if rows is None else st.index_select(0, rows)), ref_state)
    print(f"[parity] {what}: max normalised error y {worst_y:.3e} (all steps), state {es:.3e}", flush=True)
    assert worst_y <= TOL[kind] and es <= TOL[kind], what
    return st


def test_decode_full_size_all_rows():
    """b256 E5120 N16 bf16, 128 successive updates: every y and the final state of all 256 rows."""
    import torch

    say("decode full b256 E5120 N16 bf16, 128 steps (torch generator on device)")
    w = workloads.DECODE
    x = make(w, seed=0, backend="torch")
    run_steps(x, w.steps, what="decode full (all 256 rows)")
    del x
    torch.cuda.empty_cache()


def test_decode_from_nonzero_state():
    import torch

    say("decode from N(0,1) state")
    w = workloads.DECODE.with_shape(b=8, E=320, steps=12)
    x = make(w, seed=1)
    g = torch.Generator(device="cpu").manual_seed(3)
    st = torch.randn(w.b, w.E, w.N, generator=g).to("cuda")
    run_steps(x, w.steps, what="decode from random state", state=st)


@pytest.mark.parametrize("N", list(range(1, 17)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_every_state_size(N, dtype):
    say(f"update N={N} {dtype}")
    w = workloads.DECODE.with_shape(b=5, E=77, N=N, steps=6, dtype=dtype)
    run_steps(make(w, seed=2), w.steps, kind=dtype, what=f"update N={N} {dtype}")


@pytest.mark.parametrize("gate,with_D,with_bias,softplus",
                         [(False, False, False, False), (True, False, True, True), (False, True, False, True),
                          (True, True, True, False)])
def test_flags(gate, with_D, with_bias, softplus):
    say(f"update flags gate={gate} D={with_D} bias={with_bias} softplus={softplus}")
    w = workloads.DECODE.with_shape(b=4, E=130, steps=5, dtype="f32", z=workloads.N01 if gate else None,
                                    D=workloads.N01 if with_D else None,
                                    delta_bias=(("normal", -0.5, 0.3) if softplus else ("normal", -0.1, 0.02))
                                    if with_bias else None, softplus=softplus,
                                    delta=("normal", -2.0, 1.0) if softplus else ("normal", 0.3, 0.1))
    run_steps(make(w, seed=3), w.steps, kind="f32", what="update flags")


def test_unaligned_state_uses_scalar_path():
    """A state view offset by one float is 4-byte but not 16-byte aligned: the scalar path must agree."""
    import torch

    say("update, state offset by one float")
    w = workloads.DECODE.with_shape(b=3, E=70, steps=4, dtype="f32")
    x = make(w, seed=4)
    buf = torch.zeros(w.b * w.E * w.N + 1, device="cuda")
    st = buf[1:].view(w.b, w.E, w.N)
    assert st.data_ptr() % 16 != 0
    run_steps(x, w.steps, kind="f32", what="update unaligned", state=st)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("b,N", [(3, 16), (6, 12)])
def test_staged_inputs_and_outputs(dtype, gate, b, N):
    """E a multiple of 64 with aligned rows: x, step, z and y move through LDS in 16-byte pieces.

    Checked against the oracle over several steps (batch not a multiple of the 4 rows a
    workgroup covers; N = 12 takes the padded state layout), and bit for bit against the
    per-lane path, which an output whose base is not 16-byte aligned forces."""
    import torch

    import selective_state_space_35_amd as ssm

    say(f"update staged {dtype} gate={gate} b{b} N{N}")
    w = workloads.DECODE.with_shape(b=b, E=192, N=N, steps=5, dtype=dtype, z=workloads.N01 if gate else None)
    x = make(w, seed=b + N)
    run_steps(x, w.steps, kind=dtype, what=f"update staged {dtype} gate={gate} b{b} N{N}")
    st_a = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(b)).cuda()
    st_b, st_c = st_a.clone(), st_a.clone()
    io = x["x"].dtype
    y_a, y_c = (torch.empty((w.b, w.E), dtype=io, device="cuda") for _ in range(2))
    y_buf = torch.empty(w.b * w.E + 1, dtype=io, device="cuda")
    y_b = y_buf[1:].view(w.b, w.E)
    assert y_a.data_ptr() % 16 == 0 and y_b.data_ptr() % 16 != 0
    # B and C at a base 8 bytes (bf16) or 4 bytes (fp32) past 16-byte alignment: their rows are
    # then read per lane (bf16: 8-byte vector loads; fp32: the scalar-state path)
    off = 4 if dtype == "bf16" else 1
    bc_buf = torch.empty(2, w.b * w.N + off, dtype=io, device="cuda")
    B_c, C_c = bc_buf[0, off:].view(w.b, w.N), bc_buf[1, off:].view(w.b, w.N)
    assert B_c.data_ptr() % 16 != 0
    for k in range(w.steps):
        B_c.copy_(x["B"][k])
        C_c.copy_(x["C"][k])
        for st, y, Bk, Ck in ((st_a, y_a, x["B"][k], x["C"][k]), (st_b, y_b, x["B"][k], x["C"][k]),
                              (st_c, y_c, B_c, C_c)):
            ssm.ssm_state_update(st, x["x"][k], x["delta"][k], x["A"], Bk, Ck, x["D"],
                                 None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"], y=y)
        torch.cuda.synchronize()
        assert torch.equal(y_a, y_b), f"step {k}: staged and per-lane outputs differ"
        assert torch.equal(y_a, y_c), f"step {k}: staged and per-lane B / C outputs differ"
    assert torch.equal(st_a, st_b) and torch.equal(st_a, st_c), "staged and per-lane states differ"


def test_token_steps_equal_scan():
    """L single-token updates reproduce one scan over the L tokens (same recurrence)."""
    import torch

    import selective_state_space_35_amd as ssm

    say("token steps == scan")
    w = workloads.MID.with_shape(b=3, L=150, E=70)
    x = to_device(workloads.make_scan_inputs(w, seed=5))
    y_scan, last_scan = gpu_scan(x)
    st = torch.zeros(w.b, w.E, w.N, device="cuda")
    ys = []
    for t in range(w.L):
        ys.append(ssm.ssm_state_update(st, x["u"][:, t].contiguous(), x["delta"][:, t].contiguous(), x["A"],
                                       x["B"][:, t].contiguous(), x["C"][:, t].contiguous(), x["D"],
                                       x["z"][:, t].contiguous(), x["delta_bias"], x["softplus"]))
    y_steps = torch.stack(ys, dim=1)
    torch.cuda.synchronize()
    ey = max_normalised_error(oracle.to_f64(y_steps), oracle.to_f64(y_scan))
    es = max_normalised_error(oracle.to_f64(st), oracle.to_f64(last_scan))
    print(f"[parity] steps vs scan: y {ey:.3e} state {es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= 1e-4
