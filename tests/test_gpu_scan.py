"""GPU parity of ssm_scan_fwd against the fp64 oracle, through the C ABI.

Bounds: |y - y_ref| <= 1e-4 (1 + |y_ref|) for fp32 I/O and 2e-2 (1 + |y_ref|)
for bf16 I/O with fp32 state; last_state to the same bounds.

Coverage: the four scan workloads at full size (the long-sequence one on
sampled channels, in the launch configuration the benchmark times), reduced
sizes that span several channel blocks and chunks with ragged tails, forced
chunk splits down to 8 steps, every state size 1..16, flags off/on, both
dtypes, degenerate sizes (L=0, L=1, E=1, b=0), NaN propagation, determinism,
causality, and the page invariants (a zero step keeps the state bitwise, a
large step resets it).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import check_scan, gpu_scan, sample_channels, say, to_device
from tests.parity import TOL

pytestmark = pytest.mark.gpu


def make(w, seed=0, backend="numpy"):
    dev = "cpu" if backend == "numpy" else "cuda"
    return to_device(workloads.make_scan_inputs(w, seed=seed, device=dev, backend=backend))


REDUCED = [
    ("tiny", workloads.TINY),
    ("block_b2_L512_E96", workloads.BLOCK.with_shape(b=2, L=512, E=96)),
    ("mid_b2_L1000_E130", workloads.MID.with_shape(b=2, L=1000, E=130)),
    ("long_b1_L4100_E81", workloads.LONG.with_shape(b=1, L=4100, E=81)),
]


@pytest.mark.parametrize("name,w", REDUCED, ids=[r[0] for r in REDUCED])
def test_reduced_workloads(name, w):
    say(name)
    check_scan(make(w, seed=1), w.dtype, name)


@pytest.mark.parametrize("min_chunk", [8, 24, 64, 1000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forced_chunk_splits(min_chunk, dtype):
    """Carries across chunk boundaries: many chunks, ragged last chunk, chunk longer than L."""
    tune = {"path": "chunked", "min_chunk": min_chunk, "target_waves": 100000}
    base = workloads.MID if dtype == "bf16" else workloads.BLOCK
    w = base.with_shape(b=3, L=1003, E=70)
    say(f"forced chunks min_chunk={min_chunk} {dtype}")
    check_scan(make(w, seed=2), dtype, f"chunks>={min_chunk} {dtype}", tuning=tune)


@pytest.mark.parametrize("N", list(range(1, 17)))
def test_every_state_size(N):
    w = workloads.MID.with_shape(b=2, L=300, E=72, N=N)
    say(f"N={N}")
    check_scan(make(w, seed=3), "bf16", f"N={N} bf16")
    wf = workloads.BLOCK.with_shape(b=1, L=200, E=65, N=N)
    check_scan(make(wf, seed=4), "f32", f"N={N} f32")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 9, 15, 16])
@pytest.mark.parametrize("shift", [0, 1])
def test_bf16_rows_read_directly(N, shift):
    """A scan in one chunk reads bf16 B / C rows as 32-bit words split on the scalar unit: rows that start in
    the upper half of a word (odd N, or a tensor starting 2 bytes into a word) take the other half first."""
    import torch

    w = workloads.MID.with_shape(b=3, L=150, E=72, N=N)
    x = make(w, seed=50 + N)
    if shift:
        for k in ("B", "C"):
            t = x[k]
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
            v = buf[1:].view(t.shape)
            v.copy_(t)
            x[k] = v
        assert x["B"].data_ptr() % 4 == 2 and x["C"].data_ptr() % 4 == 2
    say(f"bf16 rows direct N={N} shift={shift}")
    check_scan(x, "bf16", f"bf16 rows N={N} shift={shift}", tuning={"path": "chunked", "target_waves": 1})


@pytest.mark.parametrize("softplus", [False, True])
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("with_D", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_flag_combinations(softplus, gate, with_D, with_bias):
    # without softplus the raw step must stay positive (retention <= 1), so step and bias are drawn accordingly
    if softplus:
        delta, bias = ("normal", -1.0, 1.0), ("normal", -1.0, 0.5)
    else:
        delta, bias = ("normal", 0.6, 0.05), ("normal", -0.2, 0.05)
    w = workloads.BLOCK.with_shape(b=2, L=257, E=67, z=workloads.N01 if gate else None,
                                   D=workloads.N01 if with_D else None,
                                   delta_bias=bias if with_bias else None, softplus=softplus, delta=delta)
    say(f"flags softplus={softplus} gate={gate} D={with_D} bias={with_bias}")
    check_scan(make(w, seed=5), "f32", "flags")


def test_degenerate_sizes():
    import torch

    import selective_state_space_35_amd as ssm

    dev = "cuda"
    # L == 0: last_state is written as zeros, y is empty
    say("L=0")
    A = torch.from_numpy(workloads.a_matrix(70, 16)).to(dev)
    e = torch.empty(2, 0, 70, device=dev)
    bc = torch.empty(2, 0, 16, device=dev)
    last = torch.full((2, 70, 16), 7.0, device=dev)
    y, last = ssm.ssm_scan_fwd(e, e, A, bc, bc, last_state=last)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 70) and bool((last == 0).all())
    # b == 0: no-op
    say("b=0")
    y, _ = ssm.ssm_scan_fwd(torch.empty(0, 5, 70, device=dev), torch.empty(0, 5, 70, device=dev), A,
                            torch.empty(0, 5, 16, device=dev), torch.empty(0, 5, 16, device=dev))
    assert y.shape == (0, 5, 70)
    # L == 1 and E == 1
    for shape in [dict(b=3, L=1, E=70), dict(b=2, L=50, E=1), dict(b=1, L=1, E=1)]:
        say(f"shape {shape}")
        w = workloads.MID.with_shape(**shape)
        check_scan(make(w, seed=6), "bf16", f"{shape}")


def test_zero_step_keeps_state_bitwise():
    """A vanishing step keeps the state exactly (retention 1, write 0)."""
    import torch

    one_chunk = {"path": "chunked", "target_waves": 1}  # both runs share their arithmetic order
    for softplus, fill in [(False, 0.0), (True, -200.0)]:
        say(f"zero step softplus={softplus}")
        w = workloads.MID.with_shape(b=2, L=200, E=100, softplus=softplus, delta=("normal", 0.2, 0.05))
        x = make(w, seed=7)
        x["delta"][:, 100:] = fill
        y, last = gpu_scan(x, tuning=one_chunk)
        half = {k: (v[:, :100].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
        _, last_half = gpu_scan(half, tuning=one_chunk)
        assert torch.equal(last, last_half)


def test_large_step_resets_state():
    """A large step with A <= -1 makes the retention underflow: the state becomes the write (d*x)*B exactly."""
    import torch

    say("reset")
    w = workloads.BLOCK.with_shape(b=1, L=40, E=64, softplus=False, delta=("normal", 0.1, 0.02), delta_bias=None)
    x = make(w, seed=8)
    x["delta"][:, -1] = 200.0
    _, last = gpu_scan(x)
    d = torch.tensor(200.0, device="cuda")
    expect = (d * x["u"][0, -1])[:, None] * x["B"][0, -1][None, :]
    assert torch.equal(last[0], expect)


def test_nan_propagates_along_its_channel_only():
    import torch

    say("nan")
    w = workloads.BLOCK.with_shape(b=1, L=300, E=128)
    x = make(w, seed=9)
    x["u"][0, 123, 70] = float("nan")
    y, last = gpu_scan(x)
    assert bool(torch.isnan(y[0, 123:, 70]).all()) and not bool(torch.isnan(y[0, :123, 70]).any())
    others = torch.cat([y[..., :70], y[..., 71:]], dim=-1)
    assert not bool(torch.isnan(others).any())
    y_ref, _ = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True)
    assert np.array_equal(np.isnan(y_ref), torch.isnan(y).cpu().numpy())


def test_deterministic_and_causal():
    import torch

    say("determinism / causality")
    w = workloads.MID.with_shape(b=2, L=3000, E=96)
    x = make(w, seed=10)
    y1, l1 = gpu_scan(x)
    y2, l2 = gpu_scan(x)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
    t0 = 1777
    for k in ("u", "delta", "z", "B", "C"):
        x[k][:, t0:] = -x[k][:, t0:]
    y3, _ = gpu_scan(x)
    assert torch.equal(y3[:, :t0], y1[:, :t0])
    assert not torch.equal(y3[:, t0:], y1[:, t0:])


# ----------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark uses
# ----------------------------------------------------------------------------
def test_full_tiny():
    say("full tiny b1 L64 E16 N4 f32")
    check_scan(make(workloads.TINY, seed=0), "f32", "tiny full")


def test_full_block():
    say("full block b32 L512 E512 N16 f32")
    check_scan(make(workloads.BLOCK, seed=0), "f32", "block full")


def test_full_mid():
    say("full mid b8 L2048 E1536 N16 bf16")
    check_scan(make(workloads.MID, seed=0), "bf16", "mid full")


def test_full_mid_no_D_no_gate():
    say("full mid, D=None, no gate")
    w = workloads.MID.with_shape(D=None, z=None)
    check_scan(make(w, seed=1), "bf16", "mid full no D / no gate")


def test_full_long_all_channels():
    """b1 L65536 E5120 N16 bf16, the headline workload: every channel against the oracle (1024 per oracle call)."""
    import torch

    say("full long b1 L65536 E5120 N16 bf16 (torch generator on device)")
    x = make(workloads.LONG, seed=0, backend="torch")
    y, last = gpu_scan(x)
    for c0 in range(0, workloads.LONG.E, 1024):
        ch = torch.arange(c0, c0 + 1024, device="cuda")
        say(f"oracle on channels {c0}..{c0 + 1023}")
        check_scan(x, "bf16", f"long full (channels {c0}..{c0 + 1023})", channels=ch, y=y, last=last)
    del x, y, last
    torch.cuda.empty_cache()


def test_full_long_no_D_no_gate_sampled():
    import torch

    say("full long, D=None, no gate")
    w = workloads.LONG.with_shape(D=None, z=None)
    x = make(w, seed=1, backend="torch")
    y, last = gpu_scan(x)
    ch = sample_channels(w.E, "cuda", k=32, seed=1)
    check_scan(x, "bf16", "long full no D / no gate (sampled)", channels=ch, y=y, last=last)
    del x, y, last
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# continuation from a given state (ssm_scan_fwd_from)
# ----------------------------------------------------------------------------
def _h0(w, seed):
    import torch

    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(w.b, w.E, w.N, generator=g).to("cuda")


@pytest.mark.parametrize("kind,w", [("bf16", workloads.MID.with_shape(b=2, L=700, E=130)),
                                    ("f32", workloads.BLOCK.with_shape(b=3, L=300, E=70, N=5))],
                         ids=["bf16", "f32_N5"])
def test_initial_state_parity(kind, w):
    import torch

    import selective_state_space_35_amd as ssm

    say(f"initial state {kind}")
    x = make(w, seed=11)
    h0 = _h0(w, 12)
    y, last = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                               x["softplus"], initial_state=h0)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                  x["softplus"], h0=h0)
    ey = max_err(y, y_ref)
    el = max_err(last, last_ref)
    print(f"[parity] initial state {kind}: y {ey:.3e} last {el:.3e}", flush=True)
    assert ey <= TOL[kind] and el <= TOL[kind]


def max_err(t, ref):
    from tests.parity import max_normalised_error

    return max_normalised_error(oracle.to_f64(t), ref)


@pytest.mark.parametrize("min_chunk", [None, 16])
def test_continuation_equals_whole_sequence(min_chunk):
    """scan(L1 + L2) == scan(L2, initial_state = last_state of scan(L1)), split inside a chunk."""
    import torch

    import selective_state_space_35_amd as ssm

    tune = {"path": "chunked", "min_chunk": min_chunk, "target_waves": 100000} if min_chunk else None
    say(f"continuation min_chunk={min_chunk}")
    w = workloads.MID.with_shape(b=2, L=1500, E=96)
    x = make(w, seed=13)
    y_all, last_all = gpu_scan(x, tuning=tune)
    L1 = 611
    part = lambda sl: {k: (v[:, sl].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    p1, p2 = part(slice(0, L1)), part(slice(L1, None))
    y1, last1 = gpu_scan(p1, tuning=tune)
    y2, last2 = ssm.ssm_scan_fwd(p2["u"], p2["delta"], p2["A"], p2["B"], p2["C"], p2["D"], p2["z"], p2["delta_bias"],
                                 p2["softplus"], initial_state=last1, tuning=tune)
    torch.cuda.synchronize()
    y_cat = torch.cat([y1, y2], dim=1)
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True)
    e_cat, e_last = max_err(y_cat, y_ref), max_err(last2, last_ref)
    e_self = max_err(y_cat, oracle.to_f64(y_all))
    print(f"[parity] continuation: y {e_cat:.3e} last {e_last:.3e} vs one call {e_self:.3e}", flush=True)
    assert e_cat <= TOL["bf16"] and e_last <= TOL["bf16"] and e_self <= TOL["bf16"]
    assert max_err(last2, oracle.to_f64(last_all)) <= 1e-4


def test_prefill_then_decode():
    """A prefill's last state handed to the token update continues the same recurrence."""
    import torch

    import selective_state_space_35_amd as ssm

    say("prefill -> decode")
    w = workloads.MID.with_shape(b=3, L=400, E=130)
    x = make(w, seed=14)
    L1 = 371
    part = {k: (v[:, :L1].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    _, st = gpu_scan(part)
    ys = []
    for t in range(L1, w.L):
        ys.append(ssm.ssm_state_update(st, x["u"][:, t].contiguous(), x["delta"][:, t].contiguous(), x["A"],
                                       x["B"][:, t].contiguous(), x["C"][:, t].contiguous(), x["D"],
                                       x["z"][:, t].contiguous(), x["delta_bias"], x["softplus"]))
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True)
    ey = max_err(torch.stack(ys, dim=1), y_ref[:, L1:])
    el = max_err(st, last_ref)
    print(f"[parity] prefill->decode: y {ey:.3e} state {el:.3e}", flush=True)
    assert ey <= TOL["bf16"] and el <= TOL["bf16"]


def test_empty_sequence_copies_initial_state():
    import torch

    import selective_state_space_35_amd as ssm

    say("L=0 with initial state")
    w = workloads.BLOCK.with_shape(b=2, L=0, E=70)
    A = torch.from_numpy(workloads.a_matrix(70, 16)).to("cuda")
    e = torch.empty(2, 0, 70, device="cuda")
    bc = torch.empty(2, 0, 16, device="cuda")
    h0 = _h0(w, 15)
    _, last = ssm.ssm_scan_fwd(e, e, A, bc, bc, initial_state=h0)
    torch.cuda.synchronize()
    assert torch.equal(last, h0)
