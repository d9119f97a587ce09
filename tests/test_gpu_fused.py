"""GPU parity of the single-pass form of the forward scan (scan_fused_kernel).

The single pass walks the sequence in blocks of W chunks of 8 steps per
workgroup: every chunk runs from zero with its retentions and writes kept in
registers, the lanes of chunk 0 chain the chunk maps through LDS, and every
chunk replays from its incoming state ("mamba, from scratch", "the scan";
abhik.ai page, "Compose the updates instead of waiting for every state").  The
cases force it (tuning path "single_pass") on seeded random shapes that it
accepts, so every variant runs on inputs the oracle checks in full:

* 1, 2 or 4 lanes per channel (N <= 4, <= 8, <= 16) with padded states
  (N not a multiple of 4), fp32 and bf16 I/O, every flag combination, an
  initial state, ragged channel groups (the last workgroup of a row holds fewer
  channels) and ragged blocks (L not a multiple of the block);
* W from 1 to 16 chunks per block, including the long workload's 11 (sampled
  channels at full size), and sequences that end inside a chunk or a block;
* the saved states for the backward;
* tensors that are not 8-byte aligned: the single pass refuses them when asked
  for and the automatic choice falls back to the chunked form.

Bounds as in the other parity tests: tol * (1 + |ref|) elementwise, tol = 1e-4
for fp32 I/O and 2e-2 for bf16 I/O.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import check_scan, sample_channels, say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu

N01 = ("normal", 0.0, 1.0)
SINGLE = {"path": "single_pass"}


def fused_case(seed):
    """A seeded shape the single pass accepts (the host-side plan query decides), and its flags."""
    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(7000 + seed)
    for _ in range(200):
        dtype = str(rng.choice(["f32", "bf16"]))
        # rows of u, delta, z, y, B and C must be whole 8-byte units
        N = int(rng.choice([4, 8, 12, 16] if dtype == "bf16" else [2, 4, 6, 8, 10, 12, 14, 16]))
        b = int(rng.choice([1, 2, 3, 8, 16, 32]))
        unit = 4 if dtype == "bf16" else 2
        E = int(rng.integers(64, 4097)) // unit * unit
        L = int(rng.integers(1, 700))
        if b * L * E * N > 1.2e8:
            continue
        try:
            path, _, _ = ssm.ssm_scan_plan(b, L, E, N, dtype, tuning=SINGLE)
        except ssm.SSMError:
            continue
        assert path == "single_pass"
        softplus = bool(rng.integers(2))
        w = workloads.ScanWorkload(
            f"fused{seed}", b=b, L=L, E=E, N=N, dtype=dtype, u=N01,
            delta=("normal", -1.0, 0.8) if softplus else ("normal", 0.5, 0.05),
            z=N01 if rng.integers(2) else None, B=N01, C=N01, D=N01 if rng.integers(2) else None,
            delta_bias=(("normal", 0.0, 0.3) if softplus else ("normal", 0.0, 0.05)) if rng.integers(2) else None,
            softplus=softplus)
        return w, bool(rng.integers(2))
    raise AssertionError(f"no single-pass shape drawn for seed {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_single_pass_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    w, with_h0 = fused_case(seed)
    x = to_device(workloads.make_scan_inputs(w, seed=seed))
    h0 = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda() if with_h0 else None
    say(f"single pass seed={seed}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype} z={w.z is not None} "
        f"D={w.D is not None} bias={w.delta_bias is not None} softplus={w.softplus} h0={with_h0}")
    y, last = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                               x["softplus"], initial_state=h0, tuning=SINGLE)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                  x["softplus"], h0=h0)
    ey = max_normalised_error(oracle.to_f64(y), y_ref)
    el = max_normalised_error(oracle.to_f64(last), last_ref)
    print(f"[parity] single pass seed={seed}: y {ey:.2e} last {el:.2e} (bound {TOL[w.dtype]:.0e})", flush=True)
    assert ey <= TOL[w.dtype] and el <= TOL[w.dtype]


@pytest.mark.parametrize("L", [41, 47, 48, 49, 87, 88, 89, 176, 177, 1000])
def test_single_pass_block_edges(L):
    """Lengths around a chunk (8 steps) and a block (W = 11 here: 88 steps; 6 chunks below 49 steps), with
    the long workload's channel group (20 channels per CU).  Shorter sequences leave too few lanes for the
    single pass (fewer than 8 compute waves)."""
    w = workloads.LONG.with_shape(b=1, L=L, E=5120)
    say(f"single pass edges L={L}")
    x = to_device(workloads.make_scan_inputs(w, seed=L))
    ch = sample_channels(w.E, "cuda", k=128, seed=L)
    check_scan(x, "bf16", f"single pass L={L}", channels=ch, tuning=SINGLE)


def test_single_pass_full_long_sampled_channels():
    """b1 L65536 E5120 N16 bf16 (W = 11 chunks per block) on sampled channels, forced single pass."""
    w = workloads.LONG
    say("single pass long")
    x = workloads.make_scan_inputs(w, seed=0, device="cuda", backend="torch")
    ch = sample_channels(w.E, "cuda", k=96, seed=5)
    check_scan(x, "bf16", "single pass long (sampled channels)", channels=ch, tuning=SINGLE)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_pass_saved_states(dtype):
    import torch

    import selective_state_space_35_amd as ssm

    base = workloads.MID if dtype == "bf16" else workloads.BLOCK
    w = base.with_shape(b=8, L=333, E=1536)
    x = to_device(workloads.make_scan_inputs(w, seed=21))
    h0 = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(21)).cuda()
    assert ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype)[0] == "single_pass"
    say(f"single pass saved states {dtype}")
    y, last, saved = ssm.ssm_scan_fwd_save(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                           x["delta_bias"], x["softplus"], initial_state=h0)
    yc, lastc, savedc = ssm.ssm_scan_fwd_save(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                              x["delta_bias"], x["softplus"], initial_state=h0,
                                              tuning={"path": "chunked"})
    torch.cuda.synchronize()
    worst = 0.0
    for k in range(saved.shape[1]):
        Lk = 64 * (k + 1)
        _, ref = oracle.scan(x["u"][:, :Lk], x["delta"][:, :Lk], x["A"], x["B"][:, :Lk], x["C"][:, :Lk], x["D"],
                             None if x["z"] is None else x["z"][:, :Lk], x["delta_bias"], x["softplus"], h0=h0)
        worst = max(worst, max_normalised_error(oracle.to_f64(saved[:, k]), ref))
    print(f"[parity] single pass saved states {dtype}: {worst:.2e}", flush=True)
    assert worst <= TOL[dtype]
    # both forms save the same states to the bound
    assert max_normalised_error(oracle.to_f64(saved), oracle.to_f64(savedc)) <= TOL[dtype]


def test_unaligned_tensors_fall_back():
    """Views that start 2 bytes into a word: the single pass refuses them, the automatic choice runs the chunked
    form, and both give the oracle's result."""
    import torch

    import selective_state_space_35_amd as ssm

    w = workloads.MID.with_shape(b=8, L=200, E=1536)
    x = to_device(workloads.make_scan_inputs(w, seed=31))
    shifted = {}
    for k in ("u", "delta", "z", "B", "C"):
        t = x[k]
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        shifted[k] = v
    xs = dict(x, **shifted)
    assert xs["u"].data_ptr() % 4 == 2
    say("single pass unaligned")
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_fwd(xs["u"], xs["delta"], xs["A"], xs["B"], xs["C"], xs["D"], xs["z"], xs["delta_bias"],
                         xs["softplus"], tuning=SINGLE)
    check_scan(xs, "bf16", "unaligned views, automatic form")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_both_forms_agree_on_the_reduced_workloads(dtype):
    """The single pass and the chunked form on one input, each against the oracle."""
    base = workloads.MID if dtype == "bf16" else workloads.BLOCK
    w = base.with_shape(b=8, L=700, E=1024)
    x = to_device(workloads.make_scan_inputs(w, seed=41))
    say(f"both forms {dtype}")
    check_scan(x, dtype, f"single pass {dtype}", tuning=SINGLE)
    check_scan(x, dtype, f"chunked {dtype}", tuning={"path": "chunked", "min_chunk": 16, "target_waves": 100000})
