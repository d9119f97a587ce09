"""MI355X (gfx950) selective scan of Mamba-1 (S6): Python binding of ``libssm.so``.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/ssm.h``; this module checks
shapes, dtypes and devices, allocates outputs with PyTorch (device memory
and streams are PyTorch's job here), and calls the library on the current
PyTorch stream of the tensors' device.  There is no CPU fallback: if the
library is missing or the tensors are not on a GPU, the call raises.

Functions (same names as the C entry points):

* ``ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
  softplus=False, y=None, last_state=None, return_last_state=True,
  initial_state=None, saved_states=None, tuning=None)`` -> ``(y, last_state)``;
  ``tuning`` (a dict with keys ``path`` in "auto" / "chunked" /
  "single_pass", ``min_chunk``, ``target_waves``) selects the C entry point
  ``ssm_scan_fwd_tuned``
* ``ssm_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None,
  softplus=False, initial_state=None, y=None, last_state=None)`` ->
  ``(y, last_state)``: the same scan with the library's fixed workspace buffer
  (no device allocation in the library)
* ``ssm_scan_plan(b, L, E, N, dtype="bf16", tuning=None)`` ->
  ``(path, chunk_len, n_chunks)``: how the forward runs at that size
* ``ssm_state_update(state, x, delta, A, B, C, D=None, z=None,
  delta_bias=None, softplus=False, y=None)`` -> ``y`` (``state`` is updated
  in place)
* ``ssm_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
  softplus=False, initial_state=None, d_last_state=None)`` -> dict of
  gradients (du, ddelta, dA, dB, dC, dD, dz, d_delta_bias, d_initial_state)
* ``ssm_ssd_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None,
  softplus=False, initial_state=None, y=None, last_state=None,
  return_last_state=True)`` -> ``(y, last_state)``: the scan with a scalar
  transition per head (x [b, L, H*64], delta [b, L, H], A, D, delta_bias [H]),
  bf16 only
* ``ssm_conv_fwd(v, weight, conv_bias=None, state_in=None, x=None,
  state_out=None, return_state=True)`` -> ``(x, state_out)``: causal depthwise
  convolution + SiLU over the sequence
* ``ssm_conv_update(conv_state, v, weight, conv_bias=None, x=None)`` -> ``x``
  (``conv_state`` is shifted and appended to in place)

Shapes: u, delta, z, y [b, L, E]; A [E, N] (float32); B, C [b, L, N];
D, delta_bias [E] (float32); state / last_state [b, E, N] (float32).
Convolution: v, x [b, L, E]; weight [E, K] float32 (1 <= K <= 8); conv_bias
[E] float32; convolution state [b, E, K] in the streamed dtype, oldest sample
first.  Streamed tensors are all float32 or all bfloat16.
"""
import contextlib
import ctypes
import os

__all__ = [
    "ssm_scan_fwd", "ssm_scan_fwd_from", "ssm_scan_fwd_noalloc", "ssm_scan_bwd", "ssm_ssd_fwd", "ssm_state_update", "ssm_conv_fwd", "ssm_conv_update", "ssm_scan_plan", "ssm_profile_enable", "ssm_profile_read",
    "ssm_status_string", "library_path", "SSMError", "ScanTuning", "SCAN_PATHS",
    "SSM_F32", "SSM_BF16", "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssm.so")
_lib = None

SSM_F32 = 0
SSM_BF16 = 1

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


# ssm_scan_path values
SCAN_PATHS = {"auto": 0, "chunked": 1, "single_pass": 2}
_PATH_NAMES = {v: k for k, v in SCAN_PATHS.items()}


class ScanTuning(ctypes.Structure):
    """``ssm_scan_tuning``: path (ssm_scan_path), min_chunk, target_waves; zero fields mean the library's choice."""
    _fields_ = [("path", ctypes.c_int32), ("min_chunk", ctypes.c_int32), ("target_waves", ctypes.c_int32)]


def _tuning(tuning):
    """A ScanTuning from None, a ScanTuning or a dict {path, min_chunk, target_waves}."""
    if tuning is None or isinstance(tuning, ScanTuning):
        return tuning
    unknown = set(tuning) - {"path", "min_chunk", "target_waves"}
    if unknown:
        raise ValueError(f"unknown tuning keys {sorted(unknown)}")
    path = tuning.get("path", "auto")
    return ScanTuning(SCAN_PATHS[path] if isinstance(path, str) else int(path), int(tuning.get("min_chunk", 0)),
                      int(tuning.get("target_waves", 0)))


class SSMError(RuntimeError):
    """A call into libssm.so returned a non-zero ssm_status."""

    def __init__(self, fn, status, detail=""):
        self.status = status
        msg = f"{fn} failed: {ssm_status_string(status)} (status {status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssm.so (built in-tree by ``python -m selective_state_space_35_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -m selective_state_space_35_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ssm_scan_fwd.restype = _int
    lib.ssm_scan_fwd.argtypes = [_vp] * 8 + [_int, _vp, _vp] + [_i64] * 4 + [_int, _vp]
    lib.ssm_scan_fwd_from.restype = _int
    lib.ssm_scan_fwd_from.argtypes = [_vp] * 8 + [_int, _vp, _vp, _vp] + [_i64] * 4 + [_int, _vp]
    lib.ssm_scan_fwd_save.restype = _int
    lib.ssm_scan_fwd_save.argtypes = [_vp] * 8 + [_int, _vp, _vp, _vp, _vp] + [_i64] * 4 + [_int, _vp]
    lib.ssm_scan_fwd_noalloc.restype = _int
    lib.ssm_scan_fwd_noalloc.argtypes = [_vp] * 8 + [_int, _vp, _vp, _vp] + [_i64] * 4 + [_int, _vp]
    lib.ssm_scan_fwd_tuned.restype = _int
    lib.ssm_scan_fwd_tuned.argtypes = ([_vp] * 8 + [_int, _vp, _vp, _vp, _vp, ctypes.POINTER(ScanTuning)] +
                                       [_i64] * 4 + [_int, _vp])
    lib.ssm_state_update.restype = _int
    lib.ssm_state_update.argtypes = [_vp] * 9 + [_int, _vp] + [_i64] * 3 + [_int, _vp]
    lib.ssm_scan_bwd.restype = _int
    lib.ssm_scan_bwd.argtypes = [_vp] * 8 + [_int] + [_vp] * 12 + [_i64] * 4 + [_int, _vp]
    lib.ssm_scan_bwd_saved.restype = _int
    lib.ssm_scan_bwd_saved.argtypes = [_vp] * 8 + [_int] + [_vp] * 13 + [_i64] * 4 + [_int, _vp]
    lib.ssm_ssd_fwd.restype = _int
    lib.ssm_ssd_fwd.argtypes = [_vp] * 8 + [_int] + [_vp] * 3 + [_i64] * 5 + [_int, _vp]
    lib.ssm_conv_fwd.restype = _int
    lib.ssm_conv_fwd.argtypes = [_vp] * 6 + [_i64] * 4 + [_int, _vp]
    lib.ssm_conv_update.restype = _int
    lib.ssm_conv_update.argtypes = [_vp] * 5 + [_i64] * 3 + [_int, _vp]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [_int]
    lib.ssm_last_hip_error.restype = ctypes.c_char_p
    lib.ssm_last_hip_error.argtypes = []
    lib.ssm_version.restype = _int
    lib.ssm_version.argtypes = []
    lib.ssm_profile_enable.restype = _int
    lib.ssm_profile_enable.argtypes = [_int]
    lib.ssm_profile_read.restype = _int
    lib.ssm_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64), _int]
    lib.ssm_profile_kind_name.restype = ctypes.c_char_p
    lib.ssm_profile_kind_name.argtypes = [_int]
    lib.ssm_scan_plan.restype = _int
    lib.ssm_scan_plan.argtypes = [_i64, _i64, _i64, _i64, _int, ctypes.POINTER(ScanTuning), ctypes.POINTER(_int),
                                  ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
    _lib = lib
    return lib


def ssm_status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


def ssm_scan_plan(b, L, E, N, dtype="bf16", tuning=None):
    """(path, chunk_len, n_chunks) of a forward scan of this size (host-only query).

    path is "chunked" or "single_pass"; see ssm_scan_plan in include/ssm.h.
    """
    code = {"f32": SSM_F32, "bf16": SSM_BF16}.get(dtype, dtype)
    t = _tuning(tuning)
    path, cl, nc = _int(0), _i64(0), _i64(0)
    status = load_library().ssm_scan_plan(int(b), int(L), int(E), int(N), int(code),
                                          ctypes.byref(t) if t is not None else None, ctypes.byref(path),
                                          ctypes.byref(cl), ctypes.byref(nc))
    _raise_on("ssm_scan_plan", status)
    return _PATH_NAMES[path.value], cl.value, nc.value


PROFILE_KINDS = 17


def ssm_profile_enable(on=True):
    """Bracket every library kernel with HIP events on its stream (benchmark timing)."""
    load_library().ssm_profile_enable(int(bool(on)))


def ssm_profile_read():
    """Wait for the recorded events; return {kind name: (total ms, launches)} and clear the record."""
    lib = load_library()
    ms = (ctypes.c_double * PROFILE_KINDS)()
    cnt = (_i64 * PROFILE_KINDS)()
    _raise_on("ssm_profile_read", lib.ssm_profile_read(ms, cnt, PROFILE_KINDS))
    return {lib.ssm_profile_kind_name(k).decode(): (ms[k], cnt[k]) for k in range(PROFILE_KINDS)}


def _ptr(t):
    return None if t is None else t.data_ptr()  # an int: ctypes passes it as the void* argument


def _dtype_code(torch, dt):
    if dt == torch.float32:
        return SSM_F32
    if dt == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"streamed tensors must be float32 or bfloat16, got {dt}")


def _check(torch, name, t, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    try:  # the common case in one pass; anything off falls through to the checks that name it
        if t.dtype is dtype and t.shape == shape and t.get_device() == device.index and t.is_contiguous():
            return
    except (AttributeError, TypeError):
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_of(torch, device):
    """The current PyTorch stream of ``device`` as a raw handle."""
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index)
    return torch.cuda.current_stream(device).cuda_stream


_NULL_CTX = contextlib.nullcontext()


def _on(torch, device):
    """A context with ``device`` current: a no-op when it already is (switching costs microseconds)."""
    get = getattr(torch._C, "_cuda_getDevice", None)
    current = get() if get is not None else torch.cuda.current_device()
    return _NULL_CTX if current == device.index else torch.cuda.device(device)


def _raise_on(fn, status):
    if status != 0:
        detail = load_library().ssm_last_hip_error().decode() if status == -6 else ""
        raise SSMError(fn, status, detail)


SAVE_INTERVAL = 64  # SSM_SAVE_INTERVAL of include/ssm.h


def saved_states_shape(b, L, E, N):
    """Shape of the states ``ssm_scan_fwd_save`` keeps: one [E, N] slice per 64 steps but the last."""
    return (b, max((L + SAVE_INTERVAL - 1) // SAVE_INTERVAL - 1, 0), E, N)


def _scan_outputs(torch, u, delta, A, B, C, D, z, delta_bias, y, last_state, return_last_state, initial_state,
                  saved_states):
    """Checks the forward's tensors; returns (b, L, E, N, dtype code, device, y, last_state)."""
    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u must be a [b, L, E] tensor")
    device = u.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    b, L, E = u.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be an [E, N] tensor")
    N = A.shape[1]
    io = u.dtype
    code = _dtype_code(torch, io)
    _check(torch, "delta", delta, (b, L, E), io, device)
    _check(torch, "A", A, (E, N), torch.float32, device)
    _check(torch, "B", B, (b, L, N), io, device)
    _check(torch, "C", C, (b, L, N), io, device)
    _check(torch, "D", D, (E,), torch.float32, device, optional=True)
    _check(torch, "z", z, (b, L, E), io, device, optional=True)
    _check(torch, "delta_bias", delta_bias, (E,), torch.float32, device, optional=True)
    _check(torch, "u", u, (b, L, E), io, device)
    if y is None:
        y = torch.empty((b, L, E), dtype=io, device=device)
    else:
        _check(torch, "y", y, (b, L, E), io, device)
    if last_state is None and return_last_state:
        last_state = torch.empty((b, E, N), dtype=torch.float32, device=device)
    elif last_state is not None:
        _check(torch, "last_state", last_state, (b, E, N), torch.float32, device)
    _check(torch, "initial_state", initial_state, (b, E, N), torch.float32, device, optional=True)
    if initial_state is not None and last_state is not None and initial_state.data_ptr() == last_state.data_ptr():
        raise ValueError("initial_state must not be the last_state buffer")
    if saved_states is not None:
        _check(torch, "saved_states", saved_states, saved_states_shape(b, L, E, N), torch.float32, device)
    return b, L, E, N, code, device, y, last_state


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, y=None,
                 last_state=None, return_last_state=True, initial_state=None, saved_states=None, tuning=None):
    """Selective scan forward on the GPU.  Returns ``(y, last_state)`` (last_state None if not requested).

    ``initial_state`` [b, E, N] float32 continues the recurrence from that state
    (the C entry point ``ssm_scan_fwd_from``); None starts from zero.  A given
    ``saved_states`` buffer (``saved_states_shape``, float32) receives the state
    every 64 steps (the C entry point ``ssm_scan_fwd_save``).  ``tuning`` (dict
    or ScanTuning) fixes the form and split (the C entry point ``ssm_scan_fwd_tuned``).
    """
    import torch

    lib = load_library()
    b, L, E, N, code, device, y, last_state = _scan_outputs(torch, u, delta, A, B, C, D, z, delta_bias, y, last_state,
                                                            return_last_state, initial_state, saved_states)
    t = _tuning(tuning)
    if t is not None:
        with _on(torch, device):
            status = lib.ssm_scan_fwd_tuned(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                            _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(y),
                                            _ptr(last_state), _ptr(saved_states), ctypes.byref(t), b, L, E, N, code,
                                            _stream_of(torch, device))
        _raise_on("ssm_scan_fwd_tuned", status)
        return y, last_state
    if saved_states is not None:
        with _on(torch, device):
            status = lib.ssm_scan_fwd_save(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                           _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(y),
                                           _ptr(last_state), _ptr(saved_states), b, L, E, N, code,
                                           _stream_of(torch, device))
        _raise_on("ssm_scan_fwd_save", status)
        return y, last_state
    with _on(torch, device):
        if initial_state is None:
            status = lib.ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(delta_bias), int(bool(softplus)), _ptr(y), _ptr(last_state),
                                      b, L, E, N, code, _stream_of(torch, device))
        else:
            status = lib.ssm_scan_fwd_from(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                           _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(y),
                                           _ptr(last_state), b, L, E, N, code, _stream_of(torch, device))
    _raise_on("ssm_scan_fwd" if initial_state is None else "ssm_scan_fwd_from", status)
    return y, last_state


def ssm_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, initial_state=None,
                         y=None, last_state=None, return_last_state=True):
    """``ssm_scan_fwd_from`` whose library side allocates no device memory (the C entry point
    ``ssm_scan_fwd_noalloc``): a workspace comes from the library's fixed buffer.  The outputs y and
    last_state are the caller's; pass them to keep this call free of allocations on the PyTorch side too."""
    import torch

    lib = load_library()
    b, L, E, N, code, device, y, last_state = _scan_outputs(torch, u, delta, A, B, C, D, z, delta_bias, y, last_state,
                                                            return_last_state, initial_state, None)
    with _on(torch, device):
        status = lib.ssm_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                          _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(y),
                                          _ptr(last_state), b, L, E, N, code, _stream_of(torch, device))
    _raise_on("ssm_scan_fwd_noalloc", status)
    return y, last_state


def ssm_scan_fwd_from(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, initial_state=None,
                      y=None, last_state=None, return_last_state=True):
    """``ssm_scan_fwd`` continuing from ``initial_state`` (same name as the C entry point)."""
    return ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, softplus, y=y, last_state=last_state,
                        return_last_state=return_last_state, initial_state=initial_state)


def ssm_scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, initial_state=None,
                      y=None, last_state=None, saved_states=None, tuning=None):
    """``ssm_scan_fwd_from`` that also keeps the state every 64 steps for ``ssm_scan_bwd_saved``.

    Returns ``(y, last_state, saved_states)``; saved_states [b, ceil(L / 64) - 1, E, N] float32 holds
    the state entering steps 64, 128, ...
    """
    import torch

    b, L, E = u.shape
    N = A.shape[1]
    if saved_states is None:
        saved_states = torch.empty(saved_states_shape(b, L, E, N), dtype=torch.float32, device=u.device)
    y, last_state = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, softplus, y=y, last_state=last_state,
                                 initial_state=initial_state, saved_states=saved_states, tuning=tuning)
    return y, last_state, saved_states


def ssm_scan_bwd_saved(u, delta, A, B, C, dy, saved_states, D=None, z=None, delta_bias=None, softplus=False,
                       initial_state=None, d_last_state=None):
    """``ssm_scan_bwd`` with the states entering its chunks from ``ssm_scan_fwd_save``."""
    return ssm_scan_bwd(u, delta, A, B, C, dy, D, z, delta_bias, softplus, initial_state=initial_state,
                        d_last_state=d_last_state, saved_states=saved_states)


def ssm_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=False, initial_state=None,
                 d_last_state=None, saved_states=None):
    """Gradients of sum(dy * y) + sum(d_last_state * last_state) for ``ssm_scan_fwd_from``'s arguments.

    Returns a dict: du, ddelta (and dz when z is given) [b, L, E] in the streamed dtype;
    dA [E, N], dB and dC [b, L, N], d_initial_state [b, E, N], dD and d_delta_bias [E]
    (None when D / delta_bias are None), all float32.  ``saved_states`` from
    ``ssm_scan_fwd_save`` on the same inputs replaces the recomputed chunk states
    (the C entry point ``ssm_scan_bwd_saved``).
    """
    import torch

    lib = load_library()
    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u must be a [b, L, E] tensor")
    device = u.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    b, L, E = u.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be an [E, N] tensor")
    N = A.shape[1]
    io = u.dtype
    code = _dtype_code(torch, io)
    f32 = torch.float32
    _check(torch, "u", u, (b, L, E), io, device)
    _check(torch, "delta", delta, (b, L, E), io, device)
    _check(torch, "A", A, (E, N), f32, device)
    _check(torch, "B", B, (b, L, N), io, device)
    _check(torch, "C", C, (b, L, N), io, device)
    _check(torch, "dy", dy, (b, L, E), io, device)
    _check(torch, "D", D, (E,), f32, device, optional=True)
    _check(torch, "z", z, (b, L, E), io, device, optional=True)
    _check(torch, "delta_bias", delta_bias, (E,), f32, device, optional=True)
    _check(torch, "initial_state", initial_state, (b, E, N), f32, device, optional=True)
    _check(torch, "d_last_state", d_last_state, (b, E, N), f32, device, optional=True)
    g = {
        "du": torch.empty((b, L, E), dtype=io, device=device),
        "ddelta": torch.empty((b, L, E), dtype=io, device=device),
        "dz": torch.empty((b, L, E), dtype=io, device=device) if z is not None else None,
        "dA": torch.empty((E, N), dtype=f32, device=device),
        "dB": torch.empty((b, L, N), dtype=f32, device=device),
        "dC": torch.empty((b, L, N), dtype=f32, device=device),
        "dD": torch.empty((E,), dtype=f32, device=device) if D is not None else None,
        "d_delta_bias": torch.empty((E,), dtype=f32, device=device) if delta_bias is not None else None,
        "d_initial_state": torch.empty((b, E, N), dtype=f32, device=device),
    }
    if saved_states is not None:
        _check(torch, "saved_states", saved_states, saved_states_shape(b, L, E, N), f32, device)
        with _on(torch, device):
            status = lib.ssm_scan_bwd_saved(
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                int(bool(softplus)), _ptr(initial_state), _ptr(saved_states), _ptr(dy), _ptr(d_last_state),
                _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                _ptr(g["dz"]), _ptr(g["d_delta_bias"]), _ptr(g["d_initial_state"]), b, L, E, N, code,
                _stream_of(torch, device))
        _raise_on("ssm_scan_bwd_saved", status)
        return g
    with _on(torch, device):
        status = lib.ssm_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                  int(bool(softplus)), _ptr(initial_state), _ptr(dy), _ptr(d_last_state), _ptr(g["du"]),
                                  _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                                  _ptr(g["dz"]), _ptr(g["d_delta_bias"]), _ptr(g["d_initial_state"]), b, L, E, N, code,
                                  _stream_of(torch, device))
    _raise_on("ssm_scan_bwd", status)
    return g


def ssm_ssd_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, initial_state=None, y=None,
                last_state=None, return_last_state=True):
    """The scan with a scalar transition per head on the GPU (bf16).  Returns ``(y, last_state)``."""
    import torch

    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [b, L, H*P] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    if not isinstance(delta, torch.Tensor) or delta.dim() != 3:
        raise ValueError("delta must be a [b, L, H] tensor")
    b, L, E = x.shape
    H = delta.shape[2]
    if H == 0 or E % H:
        raise ValueError("the channels of x must split evenly into the heads of delta")
    P = E // H
    N = B.shape[2] if isinstance(B, torch.Tensor) and B.dim() == 3 else -1
    io = x.dtype
    code = _dtype_code(torch, io)
    f32 = torch.float32
    _check(torch, "x", x, (b, L, E), io, device)
    _check(torch, "delta", delta, (b, L, H), io, device)
    _check(torch, "A", A, (H,), f32, device)
    _check(torch, "B", B, (b, L, N), io, device)
    _check(torch, "C", C, (b, L, N), io, device)
    _check(torch, "D", D, (H,), f32, device, optional=True)
    _check(torch, "z", z, (b, L, E), io, device, optional=True)
    _check(torch, "delta_bias", delta_bias, (H,), f32, device, optional=True)
    _check(torch, "initial_state", initial_state, (b, E, N), f32, device, optional=True)
    if y is None:
        y = torch.empty((b, L, E), dtype=io, device=device)
    else:
        _check(torch, "y", y, (b, L, E), io, device)
    if last_state is None and return_last_state:
        last_state = torch.empty((b, E, N), dtype=f32, device=device)
    elif last_state is not None:
        _check(torch, "last_state", last_state, (b, E, N), f32, device)
    with _on(torch, device):
        status = lib.ssm_ssd_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                 int(bool(softplus)), _ptr(initial_state), _ptr(y), _ptr(last_state), b, L, H, P, N,
                                 code, _stream_of(torch, device))
    _raise_on("ssm_ssd_fwd", status)
    return y, last_state


def ssm_state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, y=None):
    """One recurrent step on the GPU; ``state`` [b, E, N] float32 is updated in place.  Returns y [b, E]."""
    import torch

    lib = load_library()
    if not isinstance(state, torch.Tensor) or state.dim() != 3:
        raise ValueError("state must be a [b, E, N] tensor")
    device = state.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    b, E, N = state.shape
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    io = x.dtype
    code = _dtype_code(torch, io)
    _check(torch, "state", state, (b, E, N), torch.float32, device)
    _check(torch, "x", x, (b, E), io, device)
    _check(torch, "delta", delta, (b, E), io, device)
    _check(torch, "A", A, (E, N), torch.float32, device)
    _check(torch, "B", B, (b, N), io, device)
    _check(torch, "C", C, (b, N), io, device)
    _check(torch, "D", D, (E,), torch.float32, device, optional=True)
    _check(torch, "z", z, (b, E), io, device, optional=True)
    _check(torch, "delta_bias", delta_bias, (E,), torch.float32, device, optional=True)
    if y is None:
        y = torch.empty((b, E), dtype=io, device=device)
    else:
        _check(torch, "y", y, (b, E), io, device)
    with _on(torch, device):
        status = lib.ssm_state_update(_ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(delta_bias), int(bool(softplus)), _ptr(y), b, E, N, code,
                                      _stream_of(torch, device))
    _raise_on("ssm_state_update", status)
    return y


def ssm_conv_fwd(v, weight, conv_bias=None, state_in=None, x=None, state_out=None, return_state=True):
    """Causal depthwise convolution + SiLU over [b, L, E] on the GPU.  Returns ``(x, state_out)``.

    ``state_in`` [b, E, K] holds the K samples before the sequence (oldest first);
    None pads with zeros.  ``state_out`` receives the K most recent samples.
    """
    import torch

    lib = load_library()
    if not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("v must be a [b, L, E] tensor")
    device = v.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    b, L, E = v.shape
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be an [E, K] tensor")
    K = weight.shape[1]
    io = v.dtype
    code = _dtype_code(torch, io)
    _check(torch, "v", v, (b, L, E), io, device)
    _check(torch, "weight", weight, (E, K), torch.float32, device)
    _check(torch, "conv_bias", conv_bias, (E,), torch.float32, device, optional=True)
    _check(torch, "state_in", state_in, (b, E, K), io, device, optional=True)
    if x is None:
        x = torch.empty((b, L, E), dtype=io, device=device)
    else:
        _check(torch, "x", x, (b, L, E), io, device)
    if state_out is None and return_state:
        state_out = torch.empty((b, E, K), dtype=io, device=device)
    elif state_out is not None:
        _check(torch, "state_out", state_out, (b, E, K), io, device)
    if state_in is not None and state_out is not None and state_in.data_ptr() == state_out.data_ptr():
        raise ValueError("state_in must not be the state_out buffer")
    with _on(torch, device):
        status = lib.ssm_conv_fwd(_ptr(v), _ptr(weight), _ptr(conv_bias), _ptr(state_in), _ptr(x), _ptr(state_out),
                                  b, L, E, K, code, _stream_of(torch, device))
    _raise_on("ssm_conv_fwd", status)
    return x, state_out


def ssm_conv_update(conv_state, v, weight, conv_bias=None, x=None):
    """One token of the convolution; ``conv_state`` [b, E, K] is updated in place.  Returns x [b, E]."""
    import torch

    lib = load_library()
    if not isinstance(conv_state, torch.Tensor) or conv_state.dim() != 3:
        raise ValueError("conv_state must be a [b, E, K] tensor")
    device = conv_state.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")
    b, E, K = conv_state.shape
    io = conv_state.dtype
    code = _dtype_code(torch, io)
    _check(torch, "conv_state", conv_state, (b, E, K), io, device)
    _check(torch, "v", v, (b, E), io, device)
    _check(torch, "weight", weight, (E, K), torch.float32, device)
    _check(torch, "conv_bias", conv_bias, (E,), torch.float32, device, optional=True)
    if x is None:
        x = torch.empty((b, E), dtype=io, device=device)
    else:
        _check(torch, "x", x, (b, E), io, device)
    with _on(torch, device):
        status = lib.ssm_conv_update(_ptr(conv_state), _ptr(v), _ptr(weight), _ptr(conv_bias), _ptr(x), b, E, K, code,
                                     _stream_of(torch, device))
    _raise_on("ssm_conv_update", status)
    return x
