"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

No GPU.  Every check here compares the oracle with something other than
itself: hand-unrolled brute force evaluated in 50-digit arithmetic, the
closed-form solution of the linear recurrence, the associative composition
evaluated as a prefix scan, a geometric-series closed form, a convolution
computed by numpy.convolve, library special functions, and invariants the
pages state (a vanishing step keeps the state, a large step resets it,
causality, full sequence == token steps).

Pages cited (title, site):
  [KK] "mamba, from scratch" (khushi keswani)
  [AB] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (abhik.ai)
  [NC] same title (nadeemcite research-papers summary)
  [MS] "mamba-from-scratch" README
"""
import mpmath
import numpy as np
import pytest
import scipy.special

import oracle

RNG = np.random.default_rng(1234)


def rand_problem(b, L, E, N, seed, softplus=True, gate=True, with_D=True, with_bias=False):
    rng = np.random.default_rng(seed)
    p = dict(
        u=rng.standard_normal((b, L, E)),
        delta=rng.normal(-1.0, 0.7, (b, L, E)),
        A=-np.exp(rng.normal(0.5, 0.6, (E, N))),
        B=rng.standard_normal((b, L, N)),
        C=rng.standard_normal((b, L, N)),
        D=rng.standard_normal(E) if with_D else None,
        z=rng.standard_normal((b, L, E)) if gate else None,
        delta_bias=rng.normal(0.0, 0.3, E) if with_bias else None,
        softplus=softplus,
    )
    return p


def run(p, **kw):
    return oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                       p["softplus"], **kw)


# ----------------------------------------------------------------------------
# p1: brute force
# ----------------------------------------------------------------------------
def test_p1_hand_unrolled_L5_in_50_digits():
    """[AB] row 2: h_t = a_t h_{t-1} + step*B*x, y_t = sum_n C h + D x.  L=5 unrolled by hand."""
    mpmath.mp.dps = 50
    p = rand_problem(1, 5, 3, 4, seed=11, softplus=True, gate=True, with_D=True, with_bias=True)
    y, last = run(p)
    mp = mpmath.mpf
    for e in range(3):
        for n in range(4):
            d = []
            for t in range(5):
                raw = mp(p["delta"][0, t, e]) + mp(p["delta_bias"][e])
                d.append(mpmath.log(1 + mpmath.exp(raw)))  # softplus, [KK] "from ssm to selective ssm"
            a = [mpmath.exp(d[t] * mp(p["A"][e, n])) for t in range(5)]
            w = [d[t] * mp(p["B"][0, t, n]) * mp(p["u"][0, t, e]) for t in range(5)]
            a1, a2, a3, a4, a5 = a
            w1, w2, w3, w4, w5 = w
            h = [
                w1,
                a2 * w1 + w2,
                a3 * a2 * w1 + a3 * w2 + w3,
                a4 * a3 * a2 * w1 + a4 * a3 * w2 + a4 * w3 + w4,
                a5 * a4 * a3 * a2 * w1 + a5 * a4 * a3 * w2 + a5 * a4 * w3 + a5 * w4 + w5,
            ]
            assert abs(float(h[4]) - last[0, e, n]) <= 1e-12 * abs(float(h[4]))
        # readout for every t, summing the unrolled states of all n
        for t in range(5):
            acc = mp(0)
            for n in range(4):
                d = [mpmath.log(1 + mpmath.exp(mp(p["delta"][0, s, e]) + mp(p["delta_bias"][e]))) for s in range(t + 1)]
                hs = mp(0)
                for s in range(t + 1):
                    prod = mp(1)
                    for r in range(s + 1, t + 1):
                        prod *= mpmath.exp(d[r] * mp(p["A"][e, n]))
                    hs += prod * d[s] * mp(p["B"][0, s, n]) * mp(p["u"][0, s, e])
                acc += mp(p["C"][0, t, n]) * hs
            yv = acc + mp(p["D"][e]) * mp(p["u"][0, t, e])
            zz = mp(p["z"][0, t, e])
            yv *= zz / (1 + mpmath.exp(-zz))
            assert abs(float(yv) - y[0, t, e]) <= 1e-12 * (1 + abs(float(yv)))


def test_p1_quadratic_closed_form_L64():
    """Closed-form solution of the linear recurrence: h_t = sum_{s<=t} exp(A * sum_{r=s+1..t} d_r) w_s.

    This uses sums of exponents instead of a running product, so it is an
    independent route to the same numbers ([MS]: the two views must agree).
    """
    p = rand_problem(2, 64, 5, 3, seed=5, softplus=True, gate=False, with_D=True)
    y, last, states = run(p, return_states=True)
    d = np.logaddexp(0.0, p["delta"])  # softplus via a library routine
    for bi in range(2):
        for e in range(5):
            cs = np.concatenate([[0.0], np.cumsum(d[bi, :, e])])  # cs[t+1] = sum_{r<=t} d_r
            for t in range(64):
                s = np.arange(t + 1)
                expo = cs[t + 1] - cs[s + 1]  # sum_{r=s+1..t} d_r
                w = d[bi, s, e][:, None] * p["B"][bi, s, :] * p["u"][bi, s, e][:, None]  # [s, N]
                h = np.sum(np.exp(expo[:, None] * p["A"][e][None, :]) * w, axis=0)
                np.testing.assert_allclose(states[bi, t, e], h, rtol=1e-11, atol=1e-13)
                yv = np.dot(p["C"][bi, t], h) + p["D"][e] * p["u"][bi, t, e]
                assert abs(yv - y[bi, t, e]) <= 1e-11 * (1 + abs(yv))


# ----------------------------------------------------------------------------
# p2: prefix composition == sequential
# ----------------------------------------------------------------------------
def compose(later, earlier):
    """(a2, w2) o (a1, w1) = (a2*a1, a2*w1 + w2): apply earlier first, then later.

    [KK] "the scan"; [AB] "Compose the updates instead of waiting for every state".
    """
    a2, w2 = later
    a1, w1 = earlier
    return a2 * a1, a2 * w1 + w2


def pairs_of(p):
    d = np.logaddexp(0.0, p["delta"]) if p["softplus"] else p["delta"]
    a = np.exp(d[..., None] * p["A"][None, None])  # [b, L, E, N]
    w = d[..., None] * p["B"][:, :, None, :] * p["u"][..., None]
    return a, w


def hillis_steele(a, w, op=compose):
    """Snapshot rounds: element t combines with element t - stride of the previous round."""
    L = a.shape[1]
    stride = 1
    while stride < L:
        na, nw = a.copy(), w.copy()
        ca, cw = op((a[:, stride:], w[:, stride:]), (a[:, :-stride], w[:, :-stride]))
        na[:, stride:], nw[:, stride:] = ca, cw
        a, w = na, nw
        stride *= 2
    return w  # with a zero initial state the prefix's write part is the state


def chunked_two_level(a, w, chunk):
    """Local sequential scans per chunk, then carries combined chunk by chunk (the GPU's decomposition)."""
    b, L = a.shape[:2]
    out = np.empty_like(w)
    carry = np.zeros_like(w[:, 0])
    for c0 in range(0, L, chunk):
        la, lw = a[:, c0].copy(), w[:, c0].copy()
        locals_ = [(la.copy(), lw.copy())]
        for t in range(c0 + 1, min(c0 + chunk, L)):
            la, lw = compose((a[:, t], w[:, t]), (la, lw))
            locals_.append((la.copy(), lw.copy()))
        for k, (pa, pw) in enumerate(locals_):
            out[:, c0 + k] = pa * carry + pw
        carry = out[:, min(c0 + chunk, L) - 1]
    return out


def test_p2_prefix_equals_sequential():
    """[AB] "Original paper ... runnable CPU code" row 3 and its self-check (fp64 atol = rtol = 1e-9)."""
    p = rand_problem(2, 37, 4, 3, seed=7)
    _, last, states = run(p, return_states=True)
    a, w = pairs_of(p)
    hs = hillis_steele(a, w)
    np.testing.assert_allclose(hs, states, rtol=1e-9, atol=1e-9)
    for chunk in (1, 4, 8, 37, 64):
        np.testing.assert_allclose(chunked_two_level(a, w, chunk), states, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(last, states[:, -1], rtol=0, atol=0)


def test_p2_negative_control_operand_order():
    """Composition is not commutative ([AB] "Compose the updates"): swapping operands must disagree."""
    p = rand_problem(1, 16, 3, 3, seed=8)
    _, _, states = run(p, return_states=True)
    a, w = pairs_of(p)
    wrong = hillis_steele(a, w, op=lambda later, earlier: compose(earlier, later))
    assert np.max(np.abs(wrong - states)) > 1e-3


# ----------------------------------------------------------------------------
# p3/p4: selection semantics ([NC] "Core Idea": small step keeps, large step resets)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("softplus", [False, True])
def test_p3_zero_step_keeps_state_bitwise(softplus):
    p = rand_problem(2, 32, 5, 4, seed=9, softplus=softplus, gate=True, with_D=True)
    # raw step 0 without softplus, or -800 with softplus (softplus(-800) underflows to exactly 0)
    p["delta"][:, 16:, :] = -800.0 if softplus else 0.0
    y, last, states = run(p, return_states=True)
    assert np.array_equal(last, states[:, 15])
    for t in range(16, 32):
        assert np.array_equal(states[:, t], states[:, 15])
    h = states[:, 15]  # [b, E, N]
    direct = p["D"][None, None, :] * p["u"][:, 16:]
    readout = np.einsum("btn,ben->bte", p["C"][:, 16:], h)
    gate = p["z"][:, 16:] * scipy.special.expit(p["z"][:, 16:])
    np.testing.assert_allclose(y[:, 16:], (readout + direct) * gate, rtol=1e-13, atol=1e-13)


def test_p4_large_step_resets_state():
    p = rand_problem(1, 20, 4, 5, seed=10, softplus=False, gate=False, with_D=False)
    p["A"] = -np.abs(p["A"]) - 1.0  # A <= -1, so exp(200 * A) <= e^-200
    t0 = 13
    p["delta"][:, t0, :] = 200.0
    _, _, states = run(p, return_states=True)
    expect = 200.0 * p["B"][0, t0][None, :] * p["u"][0, t0][:, None]  # [E, N]
    assert np.max(np.abs(states[0, t0] - expect) / np.abs(expect)) <= 1e-80


# ----------------------------------------------------------------------------
# p5/p6: fixed coefficients ([AB] "The input changes the coefficients": fixed
# coefficients give one global convolution kernel; [MS] recurrent == convolution)
# ----------------------------------------------------------------------------
def test_p5_geometric_series():
    L, E, N = 50, 3, 4
    rng = np.random.default_rng(12)
    d0, u0 = 0.3, 0.7
    Bn, Cn = rng.standard_normal(N), rng.standard_normal(N)
    A = -np.array([[1.0, 2.0, 3.5, 0.25]] * E) * np.array([[1.0], [1.3], [0.6]])
    Dv = rng.standard_normal(E)
    p = dict(u=np.full((1, L, E), u0), delta=np.full((1, L, E), d0), A=A,
             B=np.tile(Bn, (1, L, 1)), C=np.tile(Cn, (1, L, 1)), D=Dv, z=None, delta_bias=None, softplus=False)
    y, last, states = run(p, return_states=True)
    an = np.exp(d0 * A)  # [E, N]
    wn = d0 * Bn[None, :] * u0  # [E, N]
    for t in range(1, L + 1):
        h = wn * (1 - an ** t) / (1 - an)
        np.testing.assert_allclose(states[0, t - 1], h, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(y[0, t - 1], h @ Cn + Dv * u0, rtol=1e-12, atol=1e-13)


def test_p6_lti_convolution():
    L, E, N = 64, 4, 5
    rng = np.random.default_rng(13)
    d0 = 0.2
    Bn, Cn = rng.standard_normal(N), rng.standard_normal(N)
    A = -np.exp(rng.normal(0.3, 0.5, (E, N)))
    Dv = rng.standard_normal(E)
    u = rng.standard_normal((1, L, E))
    p = dict(u=u, delta=np.full((1, L, E), d0), A=A, B=np.tile(Bn, (1, L, 1)), C=np.tile(Cn, (1, L, 1)),
             D=Dv, z=None, delta_bias=None, softplus=False)
    y, _ = run(p)
    k = np.arange(L)
    for e in range(E):
        K = np.sum(Cn[None, :] * np.exp(d0 * A[e])[None, :] ** k[:, None] * d0 * Bn[None, :], axis=1)
        conv = np.convolve(u[0, :, e], K)[:L]
        np.testing.assert_allclose(y[0, :, e], conv + Dv[e] * u[0, :, e], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# p7/p8: full sequence == token steps, causality ([AB] self-check)
# ----------------------------------------------------------------------------
def test_p7_scan_equals_token_steps():
    p = rand_problem(3, 24, 6, 5, seed=14, softplus=True, gate=True, with_D=True, with_bias=True)
    y, last = run(p)
    s = np.zeros((3, 6, 5))
    for t in range(24):
        s, yt = oracle.state_update(s, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t], p["C"][:, t],
                                    p["D"], p["z"][:, t], p["delta_bias"], True)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s, last, rtol=1e-12, atol=1e-13)


def test_p8_causality_bitwise():
    p = rand_problem(2, 40, 4, 3, seed=15)
    y0, _ = run(p)
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    t0 = 23
    rng = np.random.default_rng(99)
    for key in ("u", "delta", "z", "B", "C"):
        q[key][:, t0:] += rng.standard_normal(q[key][:, t0:].shape)
    y1, _ = run(q)
    assert np.array_equal(y0[:, :t0], y1[:, :t0])
    assert not np.array_equal(y0[:, t0:], y1[:, t0:])


# ----------------------------------------------------------------------------
# p9/p10
# ----------------------------------------------------------------------------
def test_p9_retention_in_unit_interval():
    """Positive step and negative A give a retention in (0, 1] ([AB] "The input changes the coefficients")."""
    rng = np.random.default_rng(16)
    b, E, N = 4, 8, 6
    s0 = rng.standard_normal((b, E, N))
    A = -np.exp(rng.normal(0, 1, (E, N)))
    delta = rng.normal(-1, 2, (b, E))
    zeros_bn = np.zeros((b, N))
    s1, _ = oracle.state_update(s0, rng.standard_normal((b, E)), delta, A, zeros_bn, zeros_bn, softplus=True)
    ratio = s1 / s0
    assert np.all(ratio > 0) and np.all(ratio <= 1)


def test_p10_linear_in_u():
    p = rand_problem(2, 30, 4, 4, seed=17)
    rng = np.random.default_rng(18)
    u1, u2 = rng.standard_normal(p["u"].shape), rng.standard_normal(p["u"].shape)
    al, be = 0.7, -1.9
    ya, la = run(dict(p, u=u1))
    yb, lb = run(dict(p, u=u2))
    yc, lc = run(dict(p, u=al * u1 + be * u2))
    np.testing.assert_allclose(yc, al * ya + be * yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lc, al * la + be * lb, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# scalar helpers, bias placement, gate and direct path
# ----------------------------------------------------------------------------
def test_softplus_matches_library():
    xs = np.concatenate([np.linspace(-40, 40, 801), [-800.0, -745.0, -30.0, 0.0, 1e-300, 30.0, 700.0]])
    for x in xs:
        assert abs(oracle.softplus_value(x) - np.logaddexp(0.0, x)) <= 2e-16 * max(1.0, abs(x)) + 1e-300
    assert oracle.softplus_value(0.0) == np.log(2.0)


def test_silu_matches_library():
    zs = np.concatenate([np.linspace(-50, 50, 1001), [-800.0, 800.0]])
    for z in zs:
        ref = z * scipy.special.expit(z)
        assert abs(oracle.silu_value(z) - ref) <= 4e-16 * max(1.0, abs(ref))


def test_bias_is_added_before_softplus():
    """[NC] "Core Idea": the step is the softplus of (parameter + projection)."""
    p = rand_problem(2, 20, 5, 3, seed=19, with_bias=True)
    y1, l1 = run(p)
    y2, l2 = run(dict(p, delta=p["delta"] + p["delta_bias"][None, None, :], delta_bias=None))
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
    y3, _ = run(dict(p, delta_bias=None))
    assert not np.allclose(y1, y3)


def test_gate_and_direct_path_with_zero_readout():
    """With C = 0 the scan contributes nothing: y = D*u*silu(z) ([AB] rows 2 and 5)."""
    p = rand_problem(2, 16, 6, 4, seed=20)
    p["C"] = np.zeros_like(p["C"])
    y, _ = run(p)
    ref = p["D"][None, None, :] * p["u"] * p["z"] * scipy.special.expit(p["z"])
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)


def test_no_D_no_gate_is_plain_readout():
    p = rand_problem(1, 12, 3, 2, seed=21, gate=False, with_D=False)
    y, _, states = run(p, return_states=True)
    np.testing.assert_allclose(y, np.einsum("btn,bten->bte", p["C"], states), rtol=1e-14, atol=1e-15)


def test_initial_state_is_continued():
    """An incoming state is carried on ([AB] row 2: the loop continues an earlier prefix)."""
    p = rand_problem(2, 40, 3, 4, seed=22)
    y, last = run(p)
    q1 = {k: (v[:, :17] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    q2 = {k: (v[:, 17:] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    y1, l1 = run(q1)
    y2, l2 = run(q2, h0=l1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, last, rtol=1e-13, atol=1e-14)


def test_threads_do_not_change_results():
    p = rand_problem(3, 50, 7, 4, seed=23, with_bias=True)
    y1, l1 = run(p, threads=1)
    y8, l8 = run(p, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_degenerate_sizes():
    p = rand_problem(2, 0, 3, 4, seed=24)
    y, last = run(p)
    assert y.shape == (2, 0, 3) and np.array_equal(last, np.zeros((2, 3, 4)))
    p = rand_problem(0, 5, 3, 4, seed=25)
    y, last = run(p)
    assert y.shape == (0, 5, 3) and last.shape == (0, 3, 4)


def test_nan_propagates_along_its_channel_only():
    p = rand_problem(1, 20, 4, 3, seed=26)
    p["u"][0, 7, 2] = np.nan
    y, last = run(p)
    assert np.all(np.isnan(y[0, 7:, 2])) and not np.any(np.isnan(y[0, :7, 2]))
    assert not np.any(np.isnan(np.delete(y, 2, axis=2)))


# ----------------------------------------------------------------------------
# causal depthwise convolution + silu ([AB] row 4) and its token form ([AB] row 6)
# ----------------------------------------------------------------------------
def conv_problem(b, L, E, K, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((b, L, E)), rng.standard_normal((E, K)), rng.standard_normal(E)


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7])
def test_conv_matches_numpy_convolve(K):
    """x[t] = silu(cb + sum_k q[k] v[t-K+1+k]) with left zero padding == numpy.convolve with reversed taps."""
    v, q, cb = conv_problem(2, 29, 5, K, seed=30 + K)
    x, st = oracle.conv_fwd(v, q, cb)
    for bi in range(2):
        for c in range(5):
            pre = cb[c] + np.convolve(v[bi, :, c], q[c, ::-1])[:29]
            np.testing.assert_allclose(x[bi, :, c], pre * scipy.special.expit(pre), rtol=1e-13, atol=1e-14)
            # the returned state is the K most recent samples, oldest first (zeros before t = 0)
            tail = np.concatenate([np.zeros(K), v[bi, :, c]])[-K:]
            np.testing.assert_array_equal(st[bi, c], tail)


def test_conv_token_steps_equal_sequence():
    """Shifting the K-sample state and appending each token reproduces the sequence form ([AB] self-check)."""
    v, q, cb = conv_problem(3, 17, 6, 4, seed=40)
    x, st_out = oracle.conv_fwd(v, q, cb)
    st = np.zeros((3, 6, 4))
    for t in range(17):
        st, xt = oracle.conv_update(st, v[:, t], q, cb)
        np.testing.assert_allclose(xt, x[:, t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(st, st_out)


def test_conv_continuation_and_short_sequences():
    v, q, cb = conv_problem(2, 23, 4, 4, seed=41)
    x, st = oracle.conv_fwd(v, q, cb)
    for L1 in (1, 2, 3, 9, 22):  # includes a first part shorter than K
        x1, st1 = oracle.conv_fwd(v[:, :L1], q, cb)
        x2, st2 = oracle.conv_fwd(v[:, L1:], q, cb, state_in=st1)
        np.testing.assert_array_equal(np.concatenate([x1, x2], axis=1), x)
        np.testing.assert_array_equal(st2, st)


def test_conv_is_causal():
    v, q, cb = conv_problem(1, 30, 3, 4, seed=42)
    x0, _ = oracle.conv_fwd(v, q, cb)
    v2 = v.copy()
    v2[:, 13:] += 1.0
    x1, _ = oracle.conv_fwd(v2, q, cb)
    assert np.array_equal(x0[:, :13], x1[:, :13]) and not np.array_equal(x0[:, 13:], x1[:, 13:])


# ----------------------------------------------------------------------------
# backward: the gradient of the scan against central finite differences of the
# (pinned) forward oracle.  The pages train the block end to end and recompute
# states in the backward pass ([NC] "Core Idea"); the gradient itself is fixed
# by the forward definition, so differentiating the forward numerically pins it.
# ----------------------------------------------------------------------------
GRAD_INPUTS = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")
GRAD_NAMES = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
              "delta_bias": "d_delta_bias", "h0": "dh0"}


def bwd_problem(seed, softplus=True, gate=True, with_D=True, with_bias=True, with_h0=True, with_dlast=True,
                b=2, L=7, E=3, N=4):
    p = rand_problem(b, L, E, N, seed, softplus=softplus, gate=gate, with_D=with_D, with_bias=with_bias)
    rng = np.random.default_rng(seed + 1000)
    if not softplus:  # a positive step keeps every retention below one
        p["delta"] = rng.uniform(0.05, 0.8, (b, L, E))
    p["h0"] = rng.standard_normal((b, E, N)) if with_h0 else None
    p["dy"] = rng.standard_normal((b, L, E))
    p["dlast"] = rng.standard_normal((b, E, N)) if with_dlast else None
    return p


def loss_of(p):
    y, last = oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                          p["softplus"], h0=p["h0"], threads=1)
    total = float(np.sum(p["dy"] * y))
    if p["dlast"] is not None:
        total += float(np.sum(p["dlast"] * last))
    return total


def grads_of(p):
    return oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                           p["softplus"], h0=p["h0"], dy=p["dy"], dlast=p["dlast"], threads=2)


def finite_difference(p, name, eps=1e-6):
    base = p[name]
    g = np.empty_like(base)
    for idx in np.ndindex(base.shape):
        old = base[idx]
        h = eps * max(1.0, abs(old))
        base[idx] = old + h
        fp = loss_of(p)
        base[idx] = old - h
        fm = loss_of(p)
        base[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("softplus,gate,with_D,with_bias,with_h0,with_dlast", [
    (True, True, True, True, True, True),
    (False, False, False, False, False, False),
    (True, False, True, False, True, False),
    (False, True, False, True, False, True),
])
def test_bwd_matches_finite_differences(softplus, gate, with_D, with_bias, with_h0, with_dlast):
    p = bwd_problem(seed=51, softplus=softplus, gate=gate, with_D=with_D, with_bias=with_bias, with_h0=with_h0,
                    with_dlast=with_dlast)
    g = grads_of(p)
    for name in GRAD_INPUTS:
        if p[name] is None:
            assert name in ("h0",) or g[GRAD_NAMES[name]] is None
            continue
        fd = finite_difference(p, name)
        err = np.max(np.abs(g[GRAD_NAMES[name]] - fd) / (1.0 + np.abs(fd)))
        assert err < 1e-6, f"{GRAD_NAMES[name]}: max error {err:.2e} against finite differences"


def test_bwd_zero_initial_state_gradient_is_defined():
    """Without h0 the gradient with respect to the (zero) initial state is still reported."""
    p = bwd_problem(seed=52, with_h0=False)
    g = grads_of(p)
    p["h0"] = np.zeros((2, 3, 4))
    fd = finite_difference(p, "h0")
    assert np.max(np.abs(g["dh0"] - fd) / (1.0 + np.abs(fd))) < 1e-6


def test_bwd_threads_do_not_change_results():
    p = bwd_problem(seed=53, b=3, L=40, E=9, N=5)
    g1 = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
                         h0=p["h0"], dy=p["dy"], dlast=p["dlast"], threads=1)
    g4 = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
                         h0=p["h0"], dy=p["dy"], dlast=p["dlast"], threads=4)
    for k, v in g1.items():
        if v is None:
            continue
        if k in ("du", "ddelta", "dz", "dh0"):  # per-chain results do not depend on the split
            assert np.array_equal(v, g4[k]), k
        else:  # sums over chains: same terms, another addition order
            np.testing.assert_allclose(v, g4[k], rtol=1e-12, atol=1e-12)


def test_bwd_split_sequence_chains_through_the_state():
    """Gradients of a sequence cut in two, with the state and its gradient passed across the cut,
    equal those of the whole sequence (the backward of the continuation used for chunked training)."""
    p = bwd_problem(seed=54, L=12)
    g = grads_of(p)
    L1 = 5
    part = lambda k, sl: None if p[k] is None else p[k][:, sl]
    first = {k: (part(k, slice(0, L1)) if k in ("u", "delta", "z", "B", "C", "dy") else p[k]) for k in p}
    second = {k: (part(k, slice(L1, None)) if k in ("u", "delta", "z", "B", "C", "dy") else p[k]) for k in p}
    _, mid = oracle.scan(first["u"], first["delta"], p["A"], first["B"], first["C"], p["D"], first["z"],
                         p["delta_bias"], p["softplus"], h0=p["h0"])
    second["h0"] = mid
    g2 = grads_of(second)
    first["dlast"] = g2["dh0"]
    g1 = grads_of(first)
    np.testing.assert_allclose(np.concatenate([g1["du"], g2["du"]], 1), g["du"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([g1["dB"], g2["dB"]], 1), g["dB"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g1["dA"] + g2["dA"], g["dA"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g1["dh0"], g["dh0"], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# scalar transition per head (structured state-space duality).  With a_t the same
# for every state of a head, the scan is a lower-triangular mixing matrix applied
# to the inputs: y_t = sum_{s<=t} (C_t . B_s) exp(A (S_t - S_s)) d_s x_s
# + (C_t . h0) exp(A S_t) + D x_t, with S_t the running sum of steps ([AB] "Key
# takeaways": a restricted state update becomes a structured mixing matrix;
# [MS] Mamba-2 / SSD, the chunked attention view).  The dense matrix is built here
# directly from that closed form and compared with the recurrence.
# ----------------------------------------------------------------------------
def ssd_problem(seed, b=2, L=23, H=3, P=4, N=5, gate=True, with_h0=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((b, L, H * P)), delta=rng.normal(-1.0, 0.8, (b, L, H)),
                A=-np.exp(rng.normal(0.3, 0.5, H)), B=rng.standard_normal((b, L, N)),
                C=rng.standard_normal((b, L, N)), D=rng.standard_normal(H),
                z=rng.standard_normal((b, L, H * P)) if gate else None,
                delta_bias=rng.normal(0.0, 0.3, H), h0=rng.standard_normal((b, H * P, N)) if with_h0 else None)


def ssd_dense(p, softplus=True):
    x, B, C, A, D = p["x"], p["B"], p["C"], p["A"], p["D"]
    b, L, E = x.shape
    H = p["delta"].shape[2]
    P = E // H
    raw = p["delta"] + p["delta_bias"]
    d = np.logaddexp(0.0, raw) if softplus else raw            # [b, L, H]
    S = np.cumsum(d, axis=1)                                     # running sum of steps
    y = np.zeros((b, L, E))
    for bi in range(b):
        G = C[bi] @ B[bi].T                                      # [L, L]: C_t . B_s
        for h in range(H):
            decay = np.exp(A[h] * (S[bi, :, h][:, None] - S[bi, :, h][None, :]))
            M = np.tril(G * decay) * d[bi, :, h][None, :]
            xs = x[bi, :, h * P:(h + 1) * P]
            yh = M @ xs + D[h] * xs
            if p["h0"] is not None:
                h0 = p["h0"][bi, h * P:(h + 1) * P, :]           # [P, N]
                yh += np.exp(A[h] * S[bi, :, h])[:, None] * (C[bi] @ h0.T)
            y[bi, :, h * P:(h + 1) * P] = yh
    if p["z"] is not None:
        y = y * p["z"] / (1.0 + np.exp(-p["z"]))
    return y


@pytest.mark.parametrize("gate,with_h0,softplus", [(True, True, True), (False, False, True), (True, False, False)])
def test_ssd_recurrence_equals_structured_matrix(gate, with_h0, softplus):
    p = ssd_problem(61, gate=gate, with_h0=with_h0)
    if not softplus:
        p["delta"] = np.abs(p["delta"]) * 0.3 + 0.05
        p["delta_bias"] = np.zeros_like(p["delta_bias"])
    y, _ = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], softplus, h0=p["h0"])
    np.testing.assert_allclose(y, ssd_dense(p, softplus), rtol=1e-10, atol=1e-10)


def test_ssd_last_state_closed_form():
    """last_state[e, n] = sum_s exp(A (S_L - S_s)) d_s B_s[n] x_s[e] + exp(A S_L) h0[e, n]."""
    p = ssd_problem(62)
    _, last = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True, h0=p["h0"])
    b, L, E = p["x"].shape
    H = p["delta"].shape[2]
    P = E // H
    d = np.logaddexp(0.0, p["delta"] + p["delta_bias"])
    S = np.cumsum(d, axis=1)
    for bi in range(b):
        for h in range(H):
            w = np.exp(p["A"][h] * (S[bi, -1, h] - S[bi, :, h])) * d[bi, :, h]     # [L]
            xs = p["x"][bi, :, h * P:(h + 1) * P]                                    # [L, P]
            ref = (xs * w[:, None]).T @ p["B"][bi] + np.exp(p["A"][h] * S[bi, -1, h]) * p["h0"][bi, h * P:(h + 1) * P]
            np.testing.assert_allclose(last[bi, h * P:(h + 1) * P], ref, rtol=1e-10, atol=1e-10)
