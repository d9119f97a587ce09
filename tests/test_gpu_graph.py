"""The token path captured in a HIP graph (torch.cuda.CUDAGraph) replays bit for bit like eager calls.

A generation step of the block is launch-bound: per token, the convolution
token step and the state update are short kernels.  Both entry points launch
on the caller's stream, take no workspace and issue no memset, so a caller can
capture a run of tokens once and replay it.  This test captures T token steps
(ssm_conv_update, then ssm_state_update on the convolution's output), replays
the graph several times with eager work and synchronisations in between
(states reset by eager copies), and requires every replay to equal the eager
run exactly: outputs of every token and both final states.  The eager calls
are themselves checked against the fp64 oracle in test_gpu_update.py and
test_gpu_conv.py.
"""
import pytest

pytestmark = pytest.mark.gpu


def make_tokens(b, E, N, K, T, seed):
    import torch

    g = torch.Generator().manual_seed(seed)
    bf = torch.bfloat16
    t = {
        "v": torch.randn((T, b, E), generator=g).to(bf),
        "delta": (torch.randn((T, b, E), generator=g) - 1.0).to(bf),
        "B": torch.randn((T, b, N), generator=g).to(bf),
        "C": torch.randn((T, b, N), generator=g).to(bf),
        "z": torch.randn((T, b, E), generator=g).to(bf),
        "q": torch.randn((E, K), generator=g) * 0.5,
        "cb": torch.randn((E,), generator=g) * 0.1,
        "A": -torch.exp(torch.randn((E, N), generator=g) * 0.5),
        "D": torch.randn((E,), generator=g),
        "bias": torch.randn((E,), generator=g) * 0.3,
        "conv0": torch.randn((b, E, K), generator=g).to(bf),
        "ssm0": torch.randn((b, E, N), generator=g),
    }
    return {k: v.cuda().contiguous() for k, v in t.items()}


def token_loop(ssm, t, conv_state, ssm_state, xs, ys):
    for k in range(xs.shape[0]):
        ssm.ssm_conv_update(conv_state, t["v"][k], t["q"], t["cb"], x=xs[k])
        ssm.ssm_state_update(ssm_state, xs[k], t["delta"][k], t["A"], t["B"][k], t["C"][k], t["D"], t["z"][k],
                             t["bias"], True, y=ys[k])


@pytest.mark.parametrize("b,E,N,K,T", [(4, 200, 16, 4, 8), (16, 1024, 16, 4, 16)])
def test_token_steps_replay_exactly(b, E, N, K, T):
    import torch

    import selective_state_space_35_amd as ssm
    from tests.gpu_common import say

    say(f"graph capture of {T} token steps b{b} E{E} N{N} K{K}")
    t = make_tokens(b, E, N, K, T, seed=E)
    # eager reference
    conv_e, ssm_e = t["conv0"].clone(), t["ssm0"].clone()
    xs_e = torch.empty((T, b, E), dtype=torch.bfloat16, device="cuda")
    ys_e = torch.empty((T, b, E), dtype=torch.bfloat16, device="cuda")
    token_loop(ssm, t, conv_e, ssm_e, xs_e, ys_e)
    torch.cuda.synchronize()

    # static buffers for the graph; one warm-up on a side stream, as torch's capture expects
    conv_g, ssm_g = t["conv0"].clone(), t["ssm0"].clone()
    xs_g = torch.empty_like(xs_e)
    ys_g = torch.empty_like(ys_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        token_loop(ssm, t, conv_g, ssm_g, xs_g, ys_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token_loop(ssm, t, conv_g, ssm_g, xs_g, ys_g)
    torch.cuda.synchronize()

    for rep in range(3):
        conv_g.copy_(t["conv0"])
        ssm_g.copy_(t["ssm0"])
        xs_g.zero_()
        ys_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(xs_g, xs_e), f"replay {rep}: convolution outputs differ"
        assert torch.equal(ys_g, ys_e), f"replay {rep}: scan outputs differ"
        assert torch.equal(conv_g, conv_e), f"replay {rep}: convolution state differs"
        assert torch.equal(ssm_g, ssm_e), f"replay {rep}: scan state differs"
        _ = (ys_g.float().sum() + 1).item()  # eager work between replays
    print(f"[parity] graph of {T} token steps b{b} E{E}: 3 replays equal to eager", flush=True)


@pytest.mark.parametrize("name,b,L,E,N", [("chunked, cut into chunks", 1, 4096, 2560, 16),
                                          ("single pass", 8, 512, 1536, 16)])
def test_noalloc_scan_replays_exactly(name, b, L, E, N):
    """ssm_scan_fwd_noalloc allocates nothing and issues no memset, so it can be captured: the replays of a
    captured call equal the eager call bit for bit (the eager call is checked against ssm_scan_fwd_from and the
    oracle in test_zz_no_alloc.py)."""
    import torch

    import selective_state_space_35_amd as ssm
    import workloads
    from tests.gpu_common import say

    w = workloads.MID.with_shape(b=b, L=L, E=E, N=N)
    path, _, n_chunks = ssm.ssm_scan_plan(b, L, E, N, "bf16")
    assert (path == "chunked" and n_chunks > 1) if name.startswith("chunked") else path == "single_pass"
    say(f"graph capture of ssm_scan_fwd_noalloc ({name}) b{b} L{L} E{E} N{N}")
    x = workloads.make_scan_inputs(w, seed=L, device="cuda", backend="torch")
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], x["softplus"])
    y_e, last_e = ssm.ssm_scan_fwd_noalloc(*args)
    torch.cuda.synchronize()
    y_g, last_g = torch.empty_like(y_e), torch.empty_like(last_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ssm.ssm_scan_fwd_noalloc(*args, y=y_g, last_state=last_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ssm.ssm_scan_fwd_noalloc(*args, y=y_g, last_state=last_g)
    torch.cuda.synchronize()
    for rep in range(3):
        y_g.zero_()
        last_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs"
        assert torch.equal(last_g, last_e), f"replay {rep}: last state differs"
        ssm.ssm_scan_fwd_from(*args)  # eager work on the same buffer between replays
        _ = (y_g.float().sum() + 1).item()
    print(f"[parity] graph of ssm_scan_fwd_noalloc ({name}): 3 replays equal to eager", flush=True)
