"""Seeded random-shape sweeps of every entry point against the fp64 oracle.

Each case draws its sizes, dtype and flags from a fixed seed (printed before the
GPU call), so a failure names a reproducible configuration.  The forward scan
cases also force the chunked form with the sequence cut into small chunks (the
tuning argument of ssm_scan_fwd_tuned), so the chunk aggregate / carry path runs
on small inputs.
Bounds as in the other parity tests: 1e-4 (fp32) / 2e-2 (bf16) times (1 + |ref|).
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu

N01 = ("normal", 0.0, 1.0)


def scan_case(seed):
    rng = np.random.default_rng(1000 + seed)
    softplus = bool(rng.integers(2))
    w = workloads.ScanWorkload(
        f"sweep{seed}", b=int(rng.integers(1, 4)), L=int(rng.integers(1, 700)), E=int(rng.integers(1, 200)),
        N=int(rng.integers(1, 17)), dtype=str(rng.choice(["f32", "bf16"])), u=N01,
        delta=("normal", -1.0, 0.8) if softplus else ("normal", 0.5, 0.05),
        z=N01 if rng.integers(2) else None, B=N01, C=N01, D=N01 if rng.integers(2) else None,
        delta_bias=(("normal", 0.0, 0.3) if softplus else ("normal", 0.0, 0.05)) if rng.integers(2) else None,
        softplus=softplus)
    return w, bool(rng.integers(2)), int(rng.choice([8, 16, 40, 64]))


@pytest.mark.parametrize("seed", range(24))
def test_scan_forward_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    w, with_h0, min_chunk = scan_case(seed)
    tune = {"path": "chunked", "min_chunk": min_chunk, "target_waves": 100000}
    x = to_device(workloads.make_scan_inputs(w, seed=seed))
    h0 = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda() if with_h0 else None
    say(f"sweep scan seed={seed}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype} z={w.z is not None} D={w.D is not None} "
        f"bias={w.delta_bias is not None} softplus={w.softplus} h0={with_h0} min_chunk={min_chunk} "
        f"plan={ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype, tuning=tune)}")
    y, last = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                               x["softplus"], initial_state=h0, tuning=tune)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                  x["softplus"], h0=h0)
    assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL[w.dtype]
    assert max_normalised_error(oracle.to_f64(last), last_ref) <= TOL[w.dtype]


@pytest.mark.parametrize("seed", range(12))
def test_state_update_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(2000 + seed)
    w = workloads.DECODE.with_shape(b=int(rng.integers(1, 20)), E=int(rng.integers(1, 300)),
                                    N=int(rng.integers(1, 17)), steps=3, dtype=str(rng.choice(["f32", "bf16"])),
                                    z=N01 if rng.integers(2) else None, D=N01 if rng.integers(2) else None)
    x = to_device(workloads.make_decode_inputs(w, seed=seed))
    st = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda()
    ref = oracle.to_f64(st)
    say(f"sweep update seed={seed}: b{w.b} E{w.E} N{w.N} {w.dtype} z={w.z is not None} D={w.D is not None}")
    for k in range(w.steps):
        y = ssm.ssm_state_update(st, x["x"][k], x["delta"][k], x["A"], x["B"][k], x["C"][k], x["D"],
                                 None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"])
        ref, y_ref = oracle.state_update(ref, x["x"][k], x["delta"][k], x["A"], x["B"][k], x["C"][k], x["D"],
                                         None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"])
        torch.cuda.synchronize()
        assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL[w.dtype]
    assert max_normalised_error(oracle.to_f64(st), ref) <= TOL[w.dtype]


@pytest.mark.parametrize("seed", range(10))
def test_state_update_staged_sweep(seed):
    """E a multiple of 64 and N of 9..16: x, step, z, y (and for N = 16, B and C) move through LDS."""
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(2500 + seed)
    w = workloads.DECODE.with_shape(b=int(rng.integers(1, 20)), E=64 * int(rng.integers(1, 11)),
                                    N=int(rng.choice([16, 16, int(rng.integers(9, 17))])), steps=3,
                                    dtype=str(rng.choice(["f32", "bf16"])), z=N01 if rng.integers(2) else None,
                                    D=N01 if rng.integers(2) else None,
                                    delta_bias=("normal", 0.0, 0.3) if rng.integers(2) else None)
    x = to_device(workloads.make_decode_inputs(w, seed=seed))
    st = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda()
    ref = oracle.to_f64(st)
    say(f"sweep staged update seed={seed}: b{w.b} E{w.E} N{w.N} {w.dtype} z={w.z is not None} D={w.D is not None}")
    for k in range(w.steps):
        y = ssm.ssm_state_update(st, x["x"][k], x["delta"][k], x["A"], x["B"][k], x["C"][k], x["D"],
                                 None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"])
        ref, y_ref = oracle.state_update(ref, x["x"][k], x["delta"][k], x["A"], x["B"][k], x["C"][k], x["D"],
                                         None if x["z"] is None else x["z"][k], x["delta_bias"], x["softplus"])
        torch.cuda.synchronize()
        assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL[w.dtype]
    assert max_normalised_error(oracle.to_f64(st), ref) <= TOL[w.dtype]


@pytest.mark.parametrize("seed", range(8))
def test_chain_stretches_sweep(seed):
    """Few channels over many short chunks: the chunk chain cuts itself into stretches."""
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(2700 + seed)
    w = workloads.ScanWorkload(
        f"csweep{seed}", b=int(rng.integers(1, 3)), L=int(rng.integers(600, 3000)), E=int(rng.integers(1, 200)),
        N=int(rng.integers(1, 17)), dtype=str(rng.choice(["f32", "bf16"])), u=N01, delta=("normal", -1.0, 0.8),
        z=N01 if rng.integers(2) else None, B=N01, C=N01, D=N01, delta_bias=None, softplus=True)
    tune = {"path": "chunked", "min_chunk": int(rng.choice([8, 16])), "target_waves": 100000}
    x = to_device(workloads.make_scan_inputs(w, seed=seed))
    h0 = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda()
    say(f"sweep chain seed={seed}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype} "
        f"plan={ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype, tuning=tune)}")
    y, last = ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                               x["softplus"], initial_state=h0, tuning=tune)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                  x["softplus"], h0=h0)
    assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL[w.dtype]
    assert max_normalised_error(oracle.to_f64(last), last_ref) <= TOL[w.dtype]


@pytest.mark.parametrize("seed", range(12))
def test_backward_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(3000 + seed)
    w = workloads.ScanWorkload(
        f"bsweep{seed}", b=int(rng.integers(1, 3)), L=int(rng.integers(1, 300)), E=int(rng.integers(1, 150)),
        N=int(rng.integers(1, 17)), dtype=str(rng.choice(["f32", "bf16"])), u=N01, delta=("normal", -1.0, 0.8),
        z=N01 if rng.integers(2) else None, B=N01, C=N01, D=N01 if rng.integers(2) else None,
        delta_bias=("normal", 0.0, 0.3) if rng.integers(2) else None, softplus=True)
    x = to_device(workloads.make_scan_inputs(w, seed=seed))
    gen = torch.Generator().manual_seed(seed)
    dy = torch.randn(x["u"].shape, generator=gen).to(x["u"].dtype).cuda()
    h0 = torch.randn((w.b, w.E, w.N), generator=gen).cuda() if rng.integers(2) else None
    dlast = torch.randn((w.b, w.E, w.N), generator=gen).cuda() if rng.integers(2) else None
    say(f"sweep bwd seed={seed}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype} z={w.z is not None} D={w.D is not None} "
        f"bias={w.delta_bias is not None} h0={h0 is not None} dlast={dlast is not None}")
    g = ssm.ssm_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, x["D"], x["z"], x["delta_bias"], True,
                         initial_state=h0, d_last_state=dlast)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True, h0=h0,
                        dy=dy, dlast=dlast)
    for name, ref_name in (("du", "du"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA", "dA"), ("dB", "dB"),
                           ("dC", "dC"), ("dD", "dD"), ("d_delta_bias", "d_delta_bias"),
                           ("d_initial_state", "dh0")):
        if r[ref_name] is None:
            continue
        err = max_normalised_error(oracle.to_f64(g[name]), r[ref_name])
        assert err <= TOL[w.dtype], f"{name}: {err:.3e}"


@pytest.mark.parametrize("seed", range(8))
def test_saved_states_sweep(seed):
    """ssm_scan_fwd_save then ssm_scan_bwd_saved on random shapes, the forward cut into random chunks."""
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(6000 + seed)
    w = workloads.ScanWorkload(
        f"ssweep{seed}", b=int(rng.integers(1, 3)), L=int(rng.integers(1, 400)), E=int(rng.integers(1, 150)),
        N=int(rng.integers(1, 17)), dtype=str(rng.choice(["f32", "bf16"])), u=N01, delta=("normal", -1.0, 0.8),
        z=N01 if rng.integers(2) else None, B=N01, C=N01, D=N01 if rng.integers(2) else None,
        delta_bias=("normal", 0.0, 0.3) if rng.integers(2) else None, softplus=True)
    tune = {"path": "chunked", "min_chunk": int(rng.choice([8, 24, 40, 72, 136])), "target_waves": 100000}
    x = to_device(workloads.make_scan_inputs(w, seed=seed))
    gen = torch.Generator().manual_seed(seed)
    dy = torch.randn(x["u"].shape, generator=gen).to(x["u"].dtype).cuda()
    h0 = torch.randn((w.b, w.E, w.N), generator=gen).cuda() if rng.integers(2) else None
    dlast = torch.randn((w.b, w.E, w.N), generator=gen).cuda() if rng.integers(2) else None
    say(f"sweep saved seed={seed}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype} z={w.z is not None} D={w.D is not None} "
        f"bias={w.delta_bias is not None} h0={h0 is not None} dlast={dlast is not None} "
        f"plan={ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype, tuning=tune)}")
    y, last, saved = ssm.ssm_scan_fwd_save(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                           x["delta_bias"], True, initial_state=h0, tuning=tune)
    g = ssm.ssm_scan_bwd_saved(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, saved, x["D"], x["z"],
                               x["delta_bias"], True, initial_state=h0, d_last_state=dlast)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True,
                                  h0=h0)
    assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL[w.dtype]
    assert max_normalised_error(oracle.to_f64(last), last_ref) <= TOL[w.dtype]
    r = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], True, h0=h0,
                        dy=dy, dlast=dlast)
    for name, ref_name in (("du", "du"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA", "dA"), ("dB", "dB"),
                           ("dC", "dC"), ("dD", "dD"), ("d_delta_bias", "d_delta_bias"),
                           ("d_initial_state", "dh0")):
        if r[ref_name] is None:
            continue
        err = max_normalised_error(oracle.to_f64(g[name]), r[ref_name])
        assert err <= TOL[w.dtype], f"{name}: {err:.3e}"


@pytest.mark.parametrize("seed", range(12))
def test_conv_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(4000 + seed)
    w = workloads.ConvWorkload(f"csweep{seed}", b=int(rng.integers(1, 4)), L=int(rng.integers(1, 300)),
                               E=int(rng.choice([int(rng.integers(1, 300)), 8 * int(rng.integers(1, 40))])),
                               K=int(rng.integers(1, 9)), dtype=str(rng.choice(["f32", "bf16"])),
                               bias=bool(rng.integers(2)), state_in=bool(rng.integers(2)))
    x = to_device(workloads.make_conv_inputs(w, seed=seed))
    say(f"sweep conv seed={seed}: b{w.b} L{w.L} E{w.E} K{w.K} {w.dtype} bias={w.bias} state_in={w.state_in}")
    out, st = ssm.ssm_conv_fwd(x["v"], x["weight"], x["conv_bias"], x["state_in"])
    torch.cuda.synchronize()
    x_ref, st_ref = oracle.conv_fwd(x["v"], x["weight"], x["conv_bias"], x["state_in"])
    assert max_normalised_error(oracle.to_f64(out), x_ref) <= TOL[w.dtype]
    assert np.array_equal(oracle.to_f64(st), st_ref)


@pytest.mark.parametrize("seed", range(10))
def test_ssd_sweep(seed):
    import torch

    import selective_state_space_35_amd as ssm

    rng = np.random.default_rng(5000 + seed)
    w = workloads.SsdWorkload(f"ssweep{seed}", b=int(rng.integers(1, 3)), L=int(rng.integers(1, 400)),
                              H=int(rng.integers(1, 5)), N=16 * int(rng.integers(1, 9)), gate=bool(rng.integers(2)),
                              with_D=bool(rng.integers(2)), with_bias=bool(rng.integers(2)))
    x = to_device(workloads.make_ssd_inputs(w, seed=seed))
    h0 = torch.randn((w.b, w.E, w.N), generator=torch.Generator().manual_seed(seed)).cuda() if rng.integers(2) else None
    say(f"sweep ssd seed={seed}: b{w.b} L{w.L} H{w.H} N{w.N} z={w.gate} D={w.with_D} bias={w.with_bias} "
        f"h0={h0 is not None}")
    y, last = ssm.ssm_ssd_fwd(x["x"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                              x["softplus"], initial_state=h0)
    torch.cuda.synchronize()
    y_ref, last_ref = oracle.ssd(x["x"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                 x["softplus"], h0=h0)
    assert max_normalised_error(oracle.to_f64(y), y_ref) <= TOL["bf16"]
    assert max_normalised_error(oracle.to_f64(last), last_ref) <= TOL["bf16"]
