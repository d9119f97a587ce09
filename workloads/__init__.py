"""Seeded synthetic inputs for the selective scan and the state update.

This module only draws random numbers with the shapes, dtypes and value
distributions of the workloads.  It holds none of the method's arithmetic
(no softplus, no exponentials of the step, no recurrence); the only
computation on values is the input recipe ``A = -exp(A_log)`` with
``A_log[e, n] = log(n + 1)`` (the S4D-Real diagonal the workloads are
defined with), evaluated in float32 so both sides receive the same fp32
array.

Both the GPU tests and the oracle tests take their inputs from here, so the
two sides always see the same arrays.  Two backends:

* ``numpy`` -- ``numpy.random.default_rng(seed)`` (PCG64) draws in float64,
  rounded to float32 and then, for bf16 workloads, to bfloat16
  (round-to-nearest-even, by torch).  Used for every size the oracle checks
  in full.
* ``torch`` -- ``torch.Generator`` on the target device, for the full-size
  long-sequence and decode workloads whose numpy draw would take minutes.
  Deterministic for a given torch build and device.

Draw order is fixed: u, delta_raw, z, B, C, D, delta_bias.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# value recipes: ("normal", mean, std) | ("const", value) | ("mixture", p, (m1, s1), (m0, s0))
# ----------------------------------------------------------------------------
N01 = ("normal", 0.0, 1.0)


@dataclass(frozen=True)
class ScanWorkload:
    name: str
    b: int
    L: int
    E: int
    N: int
    dtype: str  # "f32" or "bf16": dtype of u, delta, z, B, C and y
    u: tuple = N01
    delta: tuple = N01  # raw step, softplus applied by the operator when softplus=True
    z: Optional[tuple] = None
    B: tuple = N01
    C: tuple = N01
    D: Optional[tuple] = None
    delta_bias: Optional[tuple] = None
    softplus: bool = True
    description: str = ""

    @property
    def elements(self) -> int:
        return self.b * self.L * self.E

    def with_shape(self, **kw) -> "ScanWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return ScanWorkload(**d)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    b: int
    E: int
    N: int
    steps: int
    dtype: str
    x: tuple = N01
    delta: tuple = ("normal", -2.0, 1.0)
    z: Optional[tuple] = N01
    B: tuple = N01
    C: tuple = N01
    D: Optional[tuple] = N01
    delta_bias: Optional[tuple] = None
    softplus: bool = True
    description: str = ""

    def with_shape(self, **kw) -> "DecodeWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return DecodeWorkload(**d)


# The five workloads: a tiny scan, a classifier-block scan, a mid-size LM-layer
# scan, the long-sequence scan and the generation-time state update.
TINY = ScanWorkload(
    "tiny", b=1, L=64, E=16, N=4, dtype="f32",
    u=N01, delta=("normal", -1.0, 0.5), z=None, B=N01, C=N01, D=N01, delta_bias=None,
    description="tiny S6 scan: b1 L64 E16 N4 fp32, no gate",
)
BLOCK = ScanWorkload(
    "block", b=32, L=512, E=512, N=16, dtype="f32",
    u=N01, delta=N01, z=N01, B=N01, C=N01, D=("const", 1.0), delta_bias=("normal", -2.0, 0.5),
    description="4-layer d_model=256 classifier block scan: b32 L512 E512 N16 fp32, gate on",
)
MID = ScanWorkload(
    "mid", b=8, L=2048, E=1536, N=16, dtype="bf16",
    u=N01, delta=("normal", -3.0, 1.0), z=N01, B=("normal", 0.0, 0.25), C=("normal", 0.0, 0.25), D=N01,
    description="mid-size LM-layer scan: b8 L2048 E1536 N16 bf16 I/O, fp32 state",
)
LONG = ScanWorkload(
    "long", b=1, L=65536, E=5120, N=16, dtype="bf16",
    u=N01, delta=("mixture", 0.05, (2.0, 0.5), (-4.0, 1.0)), z=N01,
    B=("normal", 0.0, 0.25), C=("normal", 0.0, 0.25), D=N01,
    description="long-sequence scan: b1 L65536 E5120 N16 bf16 I/O, fp32 state, 5% reset steps",
)
# one GPU's share of the long scan when its channels are split over 8 GPUs (channels
# are independent chains, so the share is the same kernel at E = 5120 / 8)
LONG_E640 = LONG.with_shape(
    name="long_e640", E=640,
    description="one GPU's share of the long scan split 8 ways over channels: b1 L65536 E640 N16 bf16 I/O",
)
DECODE = DecodeWorkload(
    "decode", b=256, E=5120, N=16, steps=128, dtype="bf16",
    description="generation state update: b256 E5120 N16, 128 successive single-token updates",
)

SCAN_WORKLOADS = {w.name: w for w in (TINY, BLOCK, MID, LONG)}


@dataclass(frozen=True)
class ConvWorkload:
    """Causal depthwise convolution before the scan: v [b, L, E], weight [E, K]."""
    name: str
    b: int
    L: int
    E: int
    K: int
    dtype: str
    bias: bool = True
    state_in: bool = False
    description: str = ""

    def with_shape(self, **kw) -> "ConvWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return ConvWorkload(**d)


# the convolution in front of the long-sequence scan and of the generation step
CONV_LONG = ConvWorkload("conv_long", b=1, L=65536, E=5120, K=4, dtype="bf16",
                         description="convolution before the long scan: b1 L65536 E5120 K4 bf16")
CONV_DECODE = ConvWorkload("conv_decode", b=256, L=1, E=5120, K=4, dtype="bf16", state_in=True,
                           description="generation-time convolution state update: b256 E5120 K4 bf16")


@dataclass(frozen=True)
class SsdWorkload:
    """The scan with a scalar transition per head: x [b, L, H*P], delta [b, L, H], B, C [b, L, N]."""
    name: str
    b: int
    L: int
    H: int
    N: int
    P: int = 64
    dtype: str = "bf16"
    gate: bool = True
    with_D: bool = True
    with_bias: bool = False
    softplus: bool = True
    description: str = ""

    @property
    def E(self) -> int:
        return self.H * self.P

    def with_shape(self, **kw) -> "SsdWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return SsdWorkload(**d)


# a long sequence through a layer of 80 heads of 64 channels (5120 channels, as the long scan) with 64 states
SSD_LONG = SsdWorkload("ssd_long", b=1, L=65536, H=80, N=64,
                       description="scalar-per-head scan: b1 L65536 H80 P64 (E5120) N64 bf16, gate, D")
SSD_MID = SsdWorkload("ssd_mid", b=4, L=2048, H=24, N=64,
                      description="scalar-per-head scan: b4 L2048 H24 P64 (E1536) N64 bf16, gate, D")


def ssd_a(H: int) -> np.ndarray:
    """A[h] = -exp(A_log[h]) with A_log[h] = log(1 + 15 h / max(H - 1, 1)): decay rates spread over 1..16, float32."""
    a_log = np.log(1.0 + 15.0 * np.arange(H, dtype=np.float64) / max(H - 1, 1)).astype(np.float32)
    return (-np.exp(a_log)).astype(np.float32)


def a_matrix(E: int, N: int) -> np.ndarray:
    """A[e, n] = -exp(A_log[e, n]) with A_log[e, n] = log(n + 1), in float32, shape [E, N]."""
    a_log = np.log(np.arange(1, N + 1, dtype=np.float64)).astype(np.float32)
    a = -np.exp(a_log)  # float32 exp
    return np.ascontiguousarray(np.broadcast_to(a, (E, N)).astype(np.float32))


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------
class _NumpyDraw:
    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)

    def normal(self, shape, mean, std):
        return (mean + std * self.rng.standard_normal(shape)).astype(np.float32)

    def uniform(self, shape):
        return self.rng.random(shape)

    def const(self, shape, value):
        return np.full(shape, value, dtype=np.float32)

    def finish(self, arr, torch_dtype, device):
        import torch

        return torch.from_numpy(np.ascontiguousarray(arr)).to(device=device).to(torch_dtype)


class _TorchDraw:
    def __init__(self, seed, device):
        import torch

        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(int(seed))

    def normal(self, shape, mean, std):
        import torch

        t = torch.randn(shape, generator=self.gen, device=self.device, dtype=torch.float32)
        return t.mul_(std).add_(mean)

    def uniform(self, shape):
        import torch

        return torch.rand(shape, generator=self.gen, device=self.device, dtype=torch.float32)

    def const(self, shape, value):
        import torch

        return torch.full(shape, float(value), device=self.device, dtype=torch.float32)

    def finish(self, arr, torch_dtype, device):
        return arr.to(device=device).to(torch_dtype).contiguous()


def _draw(drawer, recipe, shape):
    kind = recipe[0]
    if kind == "normal":
        return drawer.normal(shape, recipe[1], recipe[2])
    if kind == "const":
        return drawer.const(shape, recipe[1])
    if kind == "mixture":
        p, (m1, s1), (m0, s0) = recipe[1], recipe[2], recipe[3]
        pick = drawer.uniform(shape) < p
        a1 = drawer.normal(shape, m1, s1)
        a0 = drawer.normal(shape, m0, s0)
        if isinstance(drawer, _NumpyDraw):
            return np.where(pick, a1, a0).astype(np.float32)
        import torch

        return torch.where(pick, a1, a0)
    raise ValueError(recipe)


def _torch_dtype(name):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_scan_inputs(w: ScanWorkload, seed: int = 0, device="cpu", backend: str = "numpy") -> dict:
    """Inputs of one scan call as torch tensors on ``device``.

    Keys: u, delta, z, A, B, C, D, delta_bias (None where the workload has none)
    and softplus (bool).
    """
    import torch

    drawer = _NumpyDraw(seed) if backend == "numpy" else _TorchDraw(seed, device)
    io = _torch_dtype(w.dtype)
    shp_x = (w.b, w.L, w.E)
    shp_bc = (w.b, w.L, w.N)
    out = {}
    out["u"] = drawer.finish(_draw(drawer, w.u, shp_x), io, device)
    out["delta"] = drawer.finish(_draw(drawer, w.delta, shp_x), io, device)
    out["z"] = drawer.finish(_draw(drawer, w.z, shp_x), io, device) if w.z else None
    out["B"] = drawer.finish(_draw(drawer, w.B, shp_bc), io, device)
    out["C"] = drawer.finish(_draw(drawer, w.C, shp_bc), io, device)
    out["D"] = drawer.finish(_draw(drawer, w.D, (w.E,)), torch.float32, device) if w.D else None
    out["delta_bias"] = (drawer.finish(_draw(drawer, w.delta_bias, (w.E,)), torch.float32, device)
                         if w.delta_bias else None)
    out["A"] = torch.from_numpy(a_matrix(w.E, w.N)).to(device)
    out["softplus"] = w.softplus
    return out


def make_decode_inputs(w: DecodeWorkload, seed: int = 0, device="cpu", backend: str = "numpy") -> dict:
    """Inputs of ``w.steps`` successive state updates, stacked on a leading step axis.

    Keys: x, delta, z [steps, b, E]; B, C [steps, b, N]; A [E, N]; D, delta_bias [E];
    state0 [b, E, N] (zeros, float32); softplus.
    """
    import torch

    drawer = _NumpyDraw(seed) if backend == "numpy" else _TorchDraw(seed, device)
    io = _torch_dtype(w.dtype)
    shp_x = (w.steps, w.b, w.E)
    shp_bc = (w.steps, w.b, w.N)
    out = {}
    out["x"] = drawer.finish(_draw(drawer, w.x, shp_x), io, device)
    out["delta"] = drawer.finish(_draw(drawer, w.delta, shp_x), io, device)
    out["z"] = drawer.finish(_draw(drawer, w.z, shp_x), io, device) if w.z else None
    out["B"] = drawer.finish(_draw(drawer, w.B, shp_bc), io, device)
    out["C"] = drawer.finish(_draw(drawer, w.C, shp_bc), io, device)
    out["D"] = drawer.finish(_draw(drawer, w.D, (w.E,)), torch.float32, device) if w.D else None
    out["delta_bias"] = (drawer.finish(_draw(drawer, w.delta_bias, (w.E,)), torch.float32, device)
                         if w.delta_bias else None)
    out["A"] = torch.from_numpy(a_matrix(w.E, w.N)).to(device)
    out["state0"] = torch.zeros((w.b, w.E, w.N), dtype=torch.float32, device=device)
    out["softplus"] = w.softplus
    return out


def make_conv_inputs(w: ConvWorkload, seed: int = 0, device="cpu", backend: str = "numpy") -> dict:
    """Inputs of one convolution call.

    Keys: v [b, L, E] (N(0,1)); weight [E, K] float32, N(0, 1/K) like a fan-in
    scaled initialisation; conv_bias [E] float32 N(0, 0.1^2) or None; state_in
    [b, E, K] (N(0,1), the streamed dtype) or None.  Draw order: v, weight,
    conv_bias, state_in.
    """
    import torch

    drawer = _NumpyDraw(seed) if backend == "numpy" else _TorchDraw(seed, device)
    io = _torch_dtype(w.dtype)
    out = {}
    out["v"] = drawer.finish(drawer.normal((w.b, w.L, w.E), 0.0, 1.0), io, device)
    out["weight"] = drawer.finish(drawer.normal((w.E, w.K), 0.0, 1.0 / np.sqrt(w.K)), torch.float32, device)
    out["conv_bias"] = drawer.finish(drawer.normal((w.E,), 0.0, 0.1), torch.float32, device) if w.bias else None
    out["state_in"] = (drawer.finish(drawer.normal((w.b, w.E, w.K), 0.0, 1.0), io, device)
                       if w.state_in else None)
    return out


def make_ssd_inputs(w: SsdWorkload, seed: int = 0, device="cpu", backend: str = "numpy") -> dict:
    """Inputs of one scalar-per-head scan call.

    Keys: x [b, L, H*P] N(0,1); delta [b, L, H] raw step N(-3, 1) (softplus applied by
    the operator); B, C [b, L, N] N(0, 0.25^2); A [H] from ssd_a; D [H] N(0,1) or None;
    z [b, L, H*P] N(0,1) or None; delta_bias [H] N(0, 0.3^2) or None; softplus.
    Draw order: x, delta, z, B, C, D, delta_bias.
    """
    import torch

    drawer = _NumpyDraw(seed) if backend == "numpy" else _TorchDraw(seed, device)
    io = _torch_dtype(w.dtype)
    out = {}
    out["x"] = drawer.finish(drawer.normal((w.b, w.L, w.E), 0.0, 1.0), io, device)
    out["delta"] = drawer.finish(drawer.normal((w.b, w.L, w.H), -3.0, 1.0), io, device)
    out["z"] = drawer.finish(drawer.normal((w.b, w.L, w.E), 0.0, 1.0), io, device) if w.gate else None
    out["B"] = drawer.finish(drawer.normal((w.b, w.L, w.N), 0.0, 0.25), io, device)
    out["C"] = drawer.finish(drawer.normal((w.b, w.L, w.N), 0.0, 0.25), io, device)
    out["D"] = drawer.finish(drawer.normal((w.H,), 0.0, 1.0), torch.float32, device) if w.with_D else None
    out["delta_bias"] = (drawer.finish(drawer.normal((w.H,), 0.0, 0.3), torch.float32, device)
                         if w.with_bias else None)
    out["A"] = torch.from_numpy(ssd_a(w.H)).to(device)
    out["softplus"] = w.softplus
    return out
