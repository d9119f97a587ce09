"""ssm_scan_fwd_noalloc (the forward for callers that cannot allocate) against ssm_scan_fwd_from.

The entry point runs the plan ssm_scan_fwd_from runs, with the chunked form's
workspace in the library's fixed device buffer.  Through the C ABI (the binding
only marshals arguments):

* two calls in a row, the second on a smaller input, both in the cut chunked
  form (so the buffer is used and the second call finds the first one's data in
  it), each against ssm_scan_fwd_from on the same inputs and against the
  oracle on sampled channels;
* a single-pass and a one-chunk call, which take no workspace;
* a call whose workspace exceeds SSM_NOALLOC_SCRATCH_BYTES is refused with
  SSM_ERR_SCRATCH before anything is enqueued (its output keeps its contents).

Bounds as in the other parity tests: tol * (1 + |ref|) elementwise, tol = 1e-4
for fp32 I/O and 2e-2 for bf16 I/O.
"""
import pytest

import workloads
from tests.gpu_common import check_scan, sample_channels, say, to_device
from tests.parity import TOL, max_normalised_error

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20


def both(x, h0=None):
    """(noalloc outputs, ssm_scan_fwd_from outputs) on the same inputs."""
    import torch

    import selective_state_space_35_amd as ssm

    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], x["softplus"])
    y0, last0 = ssm.ssm_scan_fwd_noalloc(*args, initial_state=h0)
    y1, last1 = ssm.ssm_scan_fwd_from(*args, initial_state=h0)
    torch.cuda.synchronize()
    return (y0, last0), (y1, last1)


def compare(got, ref, kind, what):
    import oracle

    ey = max_normalised_error(oracle.to_f64(got[0]), oracle.to_f64(ref[0]))
    el = max_normalised_error(oracle.to_f64(got[1]), oracle.to_f64(ref[1]))
    print(f"[parity] {what}: noalloc vs ssm_scan_fwd_from y {ey:.2e} last {el:.2e}", flush=True)
    assert ey <= TOL[kind] and el <= TOL[kind]


def test_two_calls_in_a_row_second_smaller():
    import torch

    import selective_state_space_35_amd as ssm

    big = workloads.LONG.with_shape(b=1, L=8192, E=5120)
    small = workloads.BLOCK.with_shape(b=2, L=3000, E=640)
    for w in (big, small):
        path, chunk_len, n_chunks = ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype)
        assert path == "chunked" and n_chunks > 1, (w.name, path, n_chunks)
    say(f"noalloc call 1: b{big.b} L{big.L} E{big.E} N{big.N} {big.dtype}")
    xb = workloads.make_scan_inputs(big, seed=1, device="cuda", backend="torch")
    got, ref = both(xb)
    compare(got, ref, "bf16", "noalloc call 1")
    ch = sample_channels(big.E, "cuda", k=64, seed=1)
    check_scan(xb, "bf16", "noalloc call 1 vs oracle", channels=ch, y=got[0], last=got[1])
    del xb, got, ref

    say(f"noalloc call 2: b{small.b} L{small.L} E{small.E} N{small.N} {small.dtype}")
    xs = to_device(workloads.make_scan_inputs(small, seed=2))
    h0 = torch.randn((small.b, small.E, small.N), generator=torch.Generator().manual_seed(2)).cuda()
    got, ref = both(xs, h0)
    compare(got, ref, "f32", "noalloc call 2")
    import oracle

    y_ref, last_ref = oracle.scan(xs["u"], xs["delta"], xs["A"], xs["B"], xs["C"], xs["D"], xs["z"],
                                  xs["delta_bias"], xs["softplus"], h0=h0)
    assert max_normalised_error(oracle.to_f64(got[0]), y_ref) <= TOL["f32"]
    assert max_normalised_error(oracle.to_f64(got[1]), last_ref) <= TOL["f32"]


@pytest.mark.parametrize("name,w", [("single_pass", workloads.MID.with_shape(b=8, L=700, E=1536)),
                                    ("one_chunk", workloads.MID.with_shape(b=2, L=40, E=300))])
def test_forms_without_workspace(name, w):
    import selective_state_space_35_amd as ssm

    path, _, n_chunks = ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype)
    assert (path, n_chunks > 1) == (("single_pass", True) if name == "single_pass" else ("chunked", False))
    say(f"noalloc {name}: b{w.b} L{w.L} E{w.E} N{w.N} {w.dtype}")
    x = to_device(workloads.make_scan_inputs(w, seed=3))
    got, ref = both(x)
    compare(got, ref, "bf16", f"noalloc {name}")


def test_workspace_beyond_the_buffer_is_refused():
    import torch

    import selective_state_space_35_amd as ssm

    # b1 E64 L2^20 bf16: 16384 chunks of 64 steps; aggregates 71 MB + float rows 134 MB > 128 MiB
    b, L, E, N = 1, 1 << 20, 64, 16
    assert ssm.ssm_scan_plan(b, L, E, N, "bf16")[0] == "chunked"
    dev = "cuda"
    u = torch.zeros((b, L, E), dtype=torch.bfloat16, device=dev)
    bc = torch.zeros((b, L, N), dtype=torch.bfloat16, device=dev)
    A = -torch.ones((E, N), dtype=torch.float32, device=dev)
    y = torch.full((b, L, E), 3.0, dtype=torch.bfloat16, device=dev)
    say("noalloc refusal: b1 L1048576 E64 N16 bf16")
    with pytest.raises(ssm.SSMError, match="status -8"):
        ssm.ssm_scan_fwd_noalloc(u, u, A, bc, bc, y=y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
