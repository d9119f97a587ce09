"""Plain double-precision CPU oracle of the S6 selective scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library and the GPU library never calls it.

The arithmetic lives in ``ssm_oracle.c`` (sequential definition, fp64, one
thread per group of independent (batch, channel) chains).  This module only
widens inputs to float64 exactly (bfloat16 and float32 values are exactly
representable in float64), calls the C routine and returns numpy arrays.

Definitions followed (page title, site, section):
  * recurrence, readout and direct path -- "Mamba: Linear-Time Sequence
    Modeling with Selective State Spaces" (abhik.ai), "Original paper,
    equations and runnable CPU code", row 2 "Retain, write and read each
    channel's state";
  * softplus step and A = -exp(A_log) -- "mamba, from scratch" (khushi
    keswani), "from ssm to selective ssm";
  * silu(z) gate -- abhik.ai page, row 5 "Put the selective operator inside
    the complete mixer";
  * single-token update -- abhik.ai page, row 6 "Carry both buffers to the
    next token";
  * causal depthwise convolution + silu before the scan -- abhik.ai page,
    row 4 "Add causal local context before selecting coefficients", and its
    single-token form in row 6;
  * the scan with a scalar transition per head (structured state-space
    duality, computed by the GPU in chunks of matrix products) -- abhik.ai
    page, "Key takeaways" and "Related reading" (Mamba-2: a restricted state
    update turned into a structured mixing matrix and a chunked algorithm);
    "mamba-from-scratch" README (Mamba-2 / SSD: chunked parallel scan);
  * backward of the scan (gradients of every input by the chain rule of the
    definition; the pages train the block end to end and recompute states in
    the backward pass) -- nadeemcite summary, "Core Idea"; abhik.ai page,
    "Compose the updates instead of waiting for every state".

Parity status: every function here is pinned by closed forms, invariants and
brute force in ``tests/test_oracle_pins.py`` (the backward by central finite
differences of the pinned forward); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libssm_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def _load(path=None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    if path is None:
        path = _LIB_PATH
        if not os.path.exists(path):
            from . import build as _build

            _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_scan.restype = ctypes.c_int
    lib.oracle_scan.argtypes = [_dp] * 8 + [ctypes.c_int, _dp, _dp, _dp, _dp] + [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.oracle_state_update.restype = ctypes.c_int
    lib.oracle_state_update.argtypes = [_dp] * 9 + [ctypes.c_int, _dp] + [ctypes.c_int64] * 3 + [ctypes.c_int]
    lib.oracle_conv_fwd.restype = ctypes.c_int
    lib.oracle_conv_fwd.argtypes = [_dp] * 6 + [ctypes.c_int64] * 4
    lib.oracle_conv_update.restype = ctypes.c_int
    lib.oracle_conv_update.argtypes = [_dp] * 5 + [ctypes.c_int64] * 3
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [_dp] * 8 + [ctypes.c_int] + [_dp] * 12 + [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.oracle_softplus_value.restype = ctypes.c_double
    lib.oracle_softplus_value.argtypes = [ctypes.c_double]
    lib.oracle_silu_value.restype = ctypes.c_double
    lib.oracle_silu_value.argtypes = [ctypes.c_double]
    _lib = lib
    return lib


def use_library(path=None):
    """Point this module at another build of the oracle (mutation tests); None restores the default."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def default_threads() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS if set (the share of the host a job is given), else
    every core this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def to_f64(x):
    """Widen a numpy array or a (CPU or GPU) torch tensor to a contiguous float64 numpy array.

    bfloat16 and float32 values widen exactly, so the oracle sees exactly the
    numbers the GPU sees.
    """
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch

        t = x.detach()
        if t.dtype == torch.bfloat16 or t.dtype == torch.float16:
            t = t.float()
        x = t.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None,
         return_states=False, threads=None):
    """Sequential fp64 selective scan.

    Shapes: u, delta, z [b, L, E]; A [E, N]; B, C [b, L, N]; D, delta_bias [E];
    h0 [b, E, N] (None means a zero initial state).
    Returns (y [b, L, E], last_state [b, E, N]) and, with return_states=True,
    also every state [b, L, E, N].
    """
    lib = _load()
    u, delta, A, B, C = (to_f64(v) for v in (u, delta, A, B, C))
    D, z, delta_bias, h0 = (to_f64(v) for v in (D, z, delta_bias, h0))
    b, L, E = u.shape
    N = A.shape[1]
    if delta.shape != (b, L, E) or A.shape != (E, N) or B.shape != (b, L, N) or C.shape != (b, L, N):
        raise ValueError("oracle.scan: inconsistent shapes")
    if z is not None and z.shape != (b, L, E):
        raise ValueError("oracle.scan: z shape")
    for v in (D, delta_bias):
        if v is not None and v.shape != (E,):
            raise ValueError("oracle.scan: D / delta_bias shape")
    if h0 is not None and h0.shape != (b, E, N):
        raise ValueError("oracle.scan: h0 shape")
    y = np.empty((b, L, E), dtype=np.float64)
    last = np.empty((b, E, N), dtype=np.float64)
    states = np.empty((b, L, E, N), dtype=np.float64) if return_states else None
    rc = lib.oracle_scan(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                         int(bool(softplus)), _ptr(h0), _ptr(y), _ptr(last), _ptr(states),
                         b, L, E, N, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_scan failed with {rc}")
    if return_states:
        return y, last, states
    return y, last


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None, dy=None, dlast=None,
             threads=None):
    """Gradients of loss = sum(dy * y) + sum(dlast * last_state) for the scan above.

    Returns a dict with du, ddelta [b, L, E]; dA [E, N]; dB, dC [b, L, N]; dh0 [b, E, N];
    and dD [E], dz [b, L, E], d_delta_bias [E] when D, z, delta_bias are given (else None).
    """
    lib = _load()
    u, delta, A, B, C, dy = (to_f64(v) for v in (u, delta, A, B, C, dy))
    D, z, delta_bias, h0, dlast = (to_f64(v) for v in (D, z, delta_bias, h0, dlast))
    b, L, E = u.shape
    N = A.shape[1]
    if (delta.shape != (b, L, E) or dy.shape != (b, L, E) or A.shape != (E, N) or B.shape != (b, L, N)
            or C.shape != (b, L, N)):
        raise ValueError("oracle.scan_bwd: inconsistent shapes")
    for v, shp in ((z, (b, L, E)), (D, (E,)), (delta_bias, (E,)), (h0, (b, E, N)), (dlast, (b, E, N))):
        if v is not None and v.shape != shp:
            raise ValueError("oracle.scan_bwd: optional input shape")
    out = {"du": np.empty((b, L, E)), "ddelta": np.empty((b, L, E)), "dA": np.empty((E, N)),
           "dB": np.empty((b, L, N)), "dC": np.empty((b, L, N)), "dh0": np.empty((b, E, N)),
           "dD": np.empty(E) if D is not None else None, "dz": np.empty((b, L, E)) if z is not None else None,
           "d_delta_bias": np.empty(E) if delta_bias is not None else None}
    rc = lib.oracle_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                             int(bool(softplus)), _ptr(h0), _ptr(dy), _ptr(dlast), _ptr(out["du"]),
                             _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                             _ptr(out["dz"]), _ptr(out["d_delta_bias"]), _ptr(out["dh0"]), b, L, E, N,
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_scan_bwd failed with {rc}")
    return out


def ssd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None, threads=None):
    """The scan with the transition restricted to a scalar per head (structured state-space duality).

    x, z [b, L, H*P] (channel e = h*P + p); delta [b, L, H]; A, D, delta_bias [H];
    B, C [b, L, N]; h0 [b, H*P, N].  Every channel of head h uses the head's step,
    A, D and bias, identical over the N states: the scan above on broadcast inputs.
    Returns (y [b, L, H*P], last_state [b, H*P, N]).
    """
    x, delta, A = to_f64(x), to_f64(delta), to_f64(A)
    b, L, E = x.shape
    H = delta.shape[2]
    N = to_f64(B).shape[2]
    if E % H or A.shape != (H,):
        raise ValueError("oracle.ssd: channels must split evenly into heads")
    P = E // H
    rep = lambda v: None if v is None else np.repeat(to_f64(v), P, axis=-1)
    A_full = np.repeat(A, P)[:, None] * np.ones((1, N))
    return scan(x, rep(delta), A_full, B, C, rep(D), z, rep(delta_bias), softplus, h0=h0, threads=threads)


def state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, threads=None):
    """One recurrent step.  state [b, E, N] (not modified); x, delta, z [b, E]; B, C [b, N].

    Returns (new_state [b, E, N], y [b, E]).
    """
    lib = _load()
    s = to_f64(state).copy()
    x, delta, A, B, C = (to_f64(v) for v in (x, delta, A, B, C))
    D, z, delta_bias = (to_f64(v) for v in (D, z, delta_bias))
    b, E, N = s.shape
    if x.shape != (b, E) or delta.shape != (b, E) or A.shape != (E, N) or B.shape != (b, N) or C.shape != (b, N):
        raise ValueError("oracle.state_update: inconsistent shapes")
    y = np.empty((b, E), dtype=np.float64)
    rc = lib.oracle_state_update(_ptr(s), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), int(bool(softplus)), _ptr(y), b, E, N,
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_state_update failed with {rc}")
    return s, y


def conv_fwd(v, q, cb=None, state_in=None):
    """Causal depthwise convolution + silu: v [b, L, E], q [E, K], cb [E], state_in [b, E, K].

    Returns (x [b, L, E], state_out [b, E, K]) where state_out holds the K most
    recent samples (oldest first) -- the convolution state a decoder continues from.
    """
    lib = _load()
    v, q, cb, state_in = (to_f64(a) for a in (v, q, cb, state_in))
    b, L, E = v.shape
    K = q.shape[1]
    if q.shape != (E, K) or (cb is not None and cb.shape != (E,)) or (
            state_in is not None and state_in.shape != (b, E, K)):
        raise ValueError("oracle.conv_fwd: inconsistent shapes")
    x = np.empty((b, L, E), dtype=np.float64)
    st = np.empty((b, E, K), dtype=np.float64)
    rc = lib.oracle_conv_fwd(_ptr(v), _ptr(q), _ptr(cb), _ptr(state_in), _ptr(x), _ptr(st), b, L, E, K)
    if rc != 0:
        raise RuntimeError(f"oracle_conv_fwd failed with {rc}")
    return x, st


def conv_update(state, v, q, cb=None):
    """One token: returns (new state [b, E, K], x [b, E]); ``state`` is not modified."""
    lib = _load()
    st = to_f64(state).copy()
    v, q, cb = (to_f64(a) for a in (v, q, cb))
    b, E, K = st.shape
    if v.shape != (b, E) or q.shape != (E, K):
        raise ValueError("oracle.conv_update: inconsistent shapes")
    x = np.empty((b, E), dtype=np.float64)
    rc = lib.oracle_conv_update(_ptr(st), _ptr(v), _ptr(q), _ptr(cb), _ptr(x), b, E, K)
    if rc != 0:
        raise RuntimeError(f"oracle_conv_update failed with {rc}")
    return st, x


def softplus_value(x: float) -> float:
    return _load().oracle_softplus_value(float(x))


def silu_value(z: float) -> float:
    return _load().oracle_silu_value(float(z))
