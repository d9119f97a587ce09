"""GPU parity of ssm_conv_fwd / ssm_conv_update against the fp64 oracle, through the C ABI.

Covers every kernel width K = 1..8, ragged channel counts (not a multiple of
the 64-lane wave) and ragged sequence lengths (not a multiple of the 64-step
chunk of the sequence kernel), both dtypes, with and without bias and
incoming state, sequences shorter than the kernel, the empty sequence,
chunked continuation, token-by-token streaming (== the sequence form), and
the full-size workloads: the convolution in front of the long scan
(b1 L65536 E5120 K4 bf16, oracle on sampled channels) and the generation
step (b256 E5120 K4 bf16, every element).

The convolution state is a copy of input samples, so it is compared
bitwise; x is compared to the elementwise bound of its dtype.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import sample_channels, say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu

BASE = workloads.ConvWorkload("conv_small", b=2, L=300, E=200, K=4, dtype="f32")


def make(w, seed=0, backend="numpy"):
    dev = "cpu" if backend == "numpy" else "cuda"
    return to_device(workloads.make_conv_inputs(w, seed=seed, device=dev, backend=backend))


def gpu_conv(x, state_in="from_inputs"):
    import torch

    import selective_state_space_35_amd as ssm

    sin = x["state_in"] if state_in == "from_inputs" else state_in
    out, st = ssm.ssm_conv_fwd(x["v"], x["weight"], x["conv_bias"], sin)
    torch.cuda.synchronize()
    return out, st


def check(x, kind, what, channels=None):
    out, st = gpu_conv(x)
    v, q, cb, sin = x["v"], x["weight"], x["conv_bias"], x["state_in"]
    if channels is not None:
        v = v.index_select(2, channels)
        q = q.index_select(0, channels)
        cb = None if cb is None else cb.index_select(0, channels)
        sin = None if sin is None else sin.index_select(1, channels)
        out = out.index_select(2, channels)
        st = st.index_select(1, channels)
    x_ref, st_ref = oracle.conv_fwd(v, q, cb, sin)
    err = max_normalised_error(oracle.to_f64(out), x_ref)
    print(f"[parity] {what}: max normalised error x {err:.3e} (bound {TOL[kind]:.0e})", flush=True)
    assert err <= TOL[kind], f"{what}: x error {err:.3e}"
    # the state holds input samples: bit-exact
    assert np.array_equal(oracle.to_f64(st), st_ref), f"{what}: state_out differs"
    return out, st


@pytest.mark.parametrize("K", range(1, 9))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_width_ragged(K, dtype):
    w = BASE.with_shape(K=K, dtype=dtype, state_in=(K % 2 == 0))
    say(f"conv K={K} {dtype} b{w.b} L{w.L} E{w.E} state_in={w.state_in}")
    check(make(w, seed=K), dtype, f"conv K={K} {dtype}")


@pytest.mark.parametrize("bias,state_in", [(False, False), (True, True), (False, True)])
def test_bias_and_state_flags(bias, state_in):
    w = BASE.with_shape(bias=bias, state_in=state_in, E=130, L=129)
    say(f"conv flags bias={bias} state_in={state_in}")
    check(make(w, seed=3), "f32", f"conv bias={bias} state_in={state_in}")


@pytest.mark.parametrize("E", [70, 128])  # 70: one channel per lane; 128: 16-byte vectors per lane
@pytest.mark.parametrize("L", [1, 2, 3, 5, 63, 64, 65, 128])
def test_short_and_boundary_lengths(L, E):
    w = BASE.with_shape(L=L, E=E, K=4, state_in=True)
    say(f"conv L={L} E={E}")
    check(make(w, seed=L), "f32", f"conv L={L} E={E}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E", [8, 1032])  # one vector; a partial second wave
def test_vector_path_edges(E, dtype):
    w = BASE.with_shape(L=70, E=E, K=3, dtype=dtype, state_in=True)
    say(f"conv vector path E={E} {dtype}")
    check(make(w, seed=E), dtype, f"conv vector E={E} {dtype}")


def test_empty_sequence_copies_state():
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=0, K=4, dtype="bf16", state_in=True)
    x = make(w, seed=1)
    say("conv L=0")
    out, st = gpu_conv(x)
    assert out.shape == (w.b, 0, w.E)
    assert torch.equal(st.cpu(), x["state_in"].cpu())
    out, st = gpu_conv(x, state_in=None)
    assert torch.count_nonzero(st).item() == 0
    # b == 0 and E == 0 are no-ops
    v = torch.zeros((0, 5, 8), device="cuda")
    xo, so = ssm.ssm_conv_fwd(v, torch.zeros((8, 4), device="cuda"))
    assert xo.shape == (0, 5, 8) and so.shape == (0, 8, 4)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_continuation_equals_whole(dtype):
    """conv over [0, L1) then [L1, L) with the state carried == conv over [0, L), including L1 < K."""
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=257, K=4, dtype=dtype, state_in=True)
    x = make(w, seed=11)
    say(f"conv continuation {dtype}")
    whole, st_whole = gpu_conv(x)
    for L1 in (1, 2, 64, 100, 256):
        a, st_a = ssm.ssm_conv_fwd(x["v"][:, :L1].contiguous(), x["weight"], x["conv_bias"], x["state_in"])
        b, st_b = ssm.ssm_conv_fwd(x["v"][:, L1:].contiguous(), x["weight"], x["conv_bias"], st_a)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([a, b], 1), whole), f"split at {L1}"
        assert torch.equal(st_b, st_whole), f"state after split at {L1}"


@pytest.mark.parametrize("K", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_updates_equal_sequence(K, dtype):
    """L calls of ssm_conv_update from state_in reproduce ssm_conv_fwd over the L tokens."""
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=20, E=130, K=K, dtype=dtype, state_in=True)
    x = make(w, seed=K + 20)
    say(f"conv tokens K={K} {dtype}")
    whole, st_whole = gpu_conv(x)
    st = x["state_in"].clone()
    outs = []
    for t in range(w.L):
        outs.append(ssm.ssm_conv_update(st, x["v"][:, t].contiguous(), x["weight"], x["conv_bias"]))
    torch.cuda.synchronize()
    tok = torch.stack(outs, 1)
    err = max_normalised_error(oracle.to_f64(tok), oracle.to_f64(whole))
    # both sides evaluate the same K-term sum in fp32, in the same order
    assert err <= TOL[dtype], err
    assert torch.equal(st, st_whole)
    # and the token form against the oracle's token form, step by step
    ref_st = oracle.to_f64(x["state_in"])
    st = x["state_in"].clone()
    for t in range(w.L):
        got = ssm.ssm_conv_update(st, x["v"][:, t].contiguous(), x["weight"], x["conv_bias"])
        ref_st, ref = oracle.conv_update(ref_st, x["v"][:, t], x["weight"], x["conv_bias"])
        torch.cuda.synchronize()
        assert max_normalised_error(oracle.to_f64(got), ref) <= TOL[dtype]
        assert np.array_equal(oracle.to_f64(st), ref_st)


def test_full_size_long_sampled():
    """The convolution in front of the long scan, at full size; oracle on sampled channels."""
    import torch

    w = workloads.CONV_LONG
    x = make(w, seed=0, backend="torch")
    ch = sample_channels(w.E, "cuda", k=32)
    say(f"conv full size {w.description}, {ch.numel()} channels checked")
    check(x, "bf16", "conv long (sampled channels)", channels=ch)


def test_full_size_decode_every_element():
    """One generation step of the convolution at b256 E5120 K4 bf16, every element vs the oracle."""
    import torch

    import selective_state_space_35_amd as ssm

    w = workloads.CONV_DECODE
    x = make(w, seed=5, backend="torch")
    st = x["state_in"].clone()
    say(f"conv decode {w.description}")
    for t in range(3):
        v_t = x["v"][:, 0] if t == 0 else torch.roll(x["v"][:, 0], t, dims=1).contiguous()
        ref_st, ref = oracle.conv_update(st, v_t, x["weight"], x["conv_bias"])
        got = ssm.ssm_conv_update(st, v_t, x["weight"], x["conv_bias"])
        torch.cuda.synchronize()
        err = max_normalised_error(oracle.to_f64(got), ref)
        print(f"[parity] conv decode step {t}: x error {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
        assert np.array_equal(oracle.to_f64(st), ref_st)


def test_unaligned_channel_offsets():
    """Row views starting at odd element offsets still match (scalar loads, no vector alignment assumed)."""
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=70, E=65, K=3, dtype="bf16", state_in=True)
    x = make(w, seed=9)
    say("conv unaligned base")
    buf = torch.empty(x["v"].numel() + 1, dtype=x["v"].dtype, device="cuda")
    v = buf[1:].view(x["v"].shape)
    v.copy_(x["v"])
    out, st = ssm.ssm_conv_fwd(v, x["weight"], x["conv_bias"], x["state_in"])
    ref, st_ref = gpu_conv(x)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(st, st_ref)


@pytest.mark.parametrize("K", [2, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_update_vector_and_element_paths_agree(K, dtype):
    """A state slice of a power-of-two size moves as one vector access when aligned; a state
    view offset by one element takes the per-element path.  Both give the same bits."""
    import torch

    import selective_state_space_35_amd as ssm

    w = BASE.with_shape(L=6, E=130, K=K, dtype=dtype, state_in=True)
    x = make(w, seed=K + 40)
    say(f"conv token vector vs element K={K} {dtype}")
    st_a = x["state_in"].clone()
    buf = torch.empty(st_a.numel() + 1, dtype=st_a.dtype, device="cuda")
    st_b = buf[1:].view(st_a.shape)
    st_b.copy_(st_a)
    assert st_a.data_ptr() % 16 == 0 and st_b.data_ptr() % (K * st_a.element_size()) != 0
    for t in range(w.L):
        v_t = x["v"][:, t].contiguous()
        ya = ssm.ssm_conv_update(st_a, v_t, x["weight"], x["conv_bias"])
        yb = ssm.ssm_conv_update(st_b, v_t, x["weight"], x["conv_bias"])
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"token {t}: outputs differ"
    assert torch.equal(st_a, st_b)
