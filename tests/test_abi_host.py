"""Host-side checks of the C ABI: no GPU needed.

* libssm.so loads and exports every function include/ssm.h declares;
* status strings;
* argument validation returns the documented ssm_status before anything is
  enqueued (every call here is invalid or a no-op, so no HIP work happens);
* the Python binding refuses CPU tensors (there is no CPU fallback) and
  raises when the library is missing.
"""
import ctypes
import os
import re

import pytest

import selective_state_space_35_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

OK, ERR_NULL, ERR_DIM, ERR_DTYPE, ERR_N, ERR_ALIGN, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
FAKE = 0x10000  # a non-null, 64 KiB-aligned address that is never dereferenced by these calls


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"SSM_API\s+[\w\s\*]+?\b(ssm_\w+)\s*\(", src)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.library_path()):
        pytest.skip("libssm.so not built")
    return ssm.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_state_update", "ssm_status_string", "ssm_last_hip_error",
            "ssm_version"} <= set(names)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in ssm.h but not exported"
    out = os.popen(f"nm -D --defined-only {ssm.library_path()}").read()
    exported = set(re.findall(r" T (\w+)", out))
    assert set(declared_functions()) <= exported
    # nothing else leaks out of the library's C namespace
    assert {s for s in exported if s.startswith("ssm_")} == set(declared_functions())


def test_status_strings(lib):
    for code in (OK, ERR_NULL, ERR_DIM, ERR_DTYPE, ERR_N, ERR_ALIGN, ERR_HIP):
        s = ssm.ssm_status_string(code)
        assert s and s != "unknown status"
    assert ssm.ssm_status_string(12345) == "unknown status"
    assert lib.ssm_version() >= 10000


def scan(lib, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1, y=FAKE,
         last=None, b=1, L=8, E=64, N=16, dtype=0):
    return lib.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, softplus, y, last, b, L, E, N, dtype, None)


def update(lib, state=FAKE, x=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1,
           y=FAKE, b=1, E=64, N=16, dtype=0):
    return lib.ssm_state_update(state, x, delta, A, B, C, D, z, bias, softplus, y, b, E, N, dtype, None)


def test_scan_validation(lib):
    assert scan(lib, dtype=2) == ERR_DTYPE
    assert scan(lib, dtype=-1) == ERR_DTYPE
    assert scan(lib, b=-1) == ERR_DIM
    assert scan(lib, L=-5) == ERR_DIM
    assert scan(lib, E=-64) == ERR_DIM
    assert scan(lib, N=0) == ERR_N
    assert scan(lib, N=17) == ERR_N
    assert scan(lib, u=None) == ERR_NULL
    assert scan(lib, delta=None) == ERR_NULL
    assert scan(lib, A=None) == ERR_NULL
    assert scan(lib, B=None) == ERR_NULL
    assert scan(lib, C=None) == ERR_NULL
    assert scan(lib, y=None) == ERR_NULL
    assert scan(lib, u=FAKE + 2, dtype=0) == ERR_ALIGN      # fp32 needs 4-byte alignment
    assert scan(lib, u=FAKE + 1, dtype=1) == ERR_ALIGN      # bf16 needs 2-byte alignment
    assert scan(lib, A=FAKE + 2) == ERR_ALIGN
    assert scan(lib, last=FAKE + 1) == ERR_ALIGN
    assert scan(lib, z=FAKE + 1, dtype=1) == ERR_ALIGN
    assert scan(lib, b=1 << 40, L=1 << 20, E=1 << 10) == ERR_DIM  # b*L*E*4 overflows int64


def test_scan_noop_sizes_return_ok_without_work(lib):
    # b == 0 or E == 0: nothing to do, pointers are not even looked at
    assert scan(lib, b=0, u=None, delta=None, A=None, B=None, C=None, y=None) == OK
    assert scan(lib, E=0, u=None, delta=None, A=None, B=None, C=None, y=None) == OK


def test_scan_from_validation(lib):
    f = lambda h0, **kw: lib.ssm_scan_fwd_from(kw.get("u", FAKE), FAKE, FAKE, FAKE, FAKE, None, None, None, 1, h0,
                                               kw.get("y", FAKE), None, kw.get("b", 1), 8, 64, 16, 0, None)
    assert f(FAKE + 2) == ERR_ALIGN
    assert f(FAKE, u=None) == ERR_NULL
    assert f(FAKE, y=None) == ERR_NULL
    assert f(FAKE, b=-1) == ERR_DIM
    assert f(None, b=0) == OK


def test_scan_noalloc_validation(lib):
    f = lambda **kw: lib.ssm_scan_fwd_noalloc(kw.get("u", FAKE), FAKE, FAKE, FAKE, FAKE, None, None, None, 1,
                                              kw.get("h0", None), kw.get("y", FAKE), None, kw.get("b", 1), 8, 64,
                                              kw.get("N", 16), kw.get("dtype", 0), None)
    assert f(dtype=5) == ERR_DTYPE
    assert f(N=17) == ERR_N
    assert f(u=None) == ERR_NULL
    assert f(y=None) == ERR_NULL
    assert f(h0=FAKE + 2) == ERR_ALIGN
    assert f(b=-1) == ERR_DIM
    assert f(b=0, u=None, y=None) == OK
    assert "SSM_NOALLOC_SCRATCH_BYTES" in ssm.ssm_status_string(-8)


def test_update_validation(lib):
    assert update(lib, dtype=7) == ERR_DTYPE
    assert update(lib, b=-2) == ERR_DIM
    assert update(lib, N=0) == ERR_N
    assert update(lib, N=32) == ERR_N
    for k in ("state", "x", "delta", "A", "B", "C", "y"):
        assert update(lib, **{k: None}) == ERR_NULL, k
    assert update(lib, state=FAKE + 2) == ERR_ALIGN
    assert update(lib, x=FAKE + 1, dtype=1) == ERR_ALIGN
    assert update(lib, b=0, state=None) == OK


def conv(lib, v=FAKE, q=FAKE, cb=None, sin=None, x=FAKE, sout=None, b=1, L=8, E=64, K=4, dtype=0):
    return lib.ssm_conv_fwd(v, q, cb, sin, x, sout, b, L, E, K, dtype, None)


def conv_update(lib, state=FAKE, v=FAKE, q=FAKE, cb=None, x=FAKE, b=1, E=64, K=4, dtype=0):
    return lib.ssm_conv_update(state, v, q, cb, x, b, E, K, dtype, None)


def test_conv_validation(lib):
    assert conv(lib, dtype=3) == ERR_DTYPE
    assert conv(lib, K=0) == ERR_DIM
    assert conv(lib, K=9) == ERR_DIM
    assert conv(lib, L=-1) == ERR_DIM
    assert conv(lib, b=-1) == ERR_DIM
    assert conv(lib, v=None) == ERR_NULL
    assert conv(lib, x=None) == ERR_NULL
    assert conv(lib, q=None) == ERR_NULL
    assert conv(lib, v=FAKE + 2) == ERR_ALIGN
    assert conv(lib, x=FAKE + 1, dtype=1) == ERR_ALIGN
    assert conv(lib, q=FAKE + 2) == ERR_ALIGN
    assert conv(lib, cb=FAKE + 1) == ERR_ALIGN
    assert conv(lib, sin=FAKE + 1, dtype=1) == ERR_ALIGN
    assert conv(lib, sout=FAKE + 2) == ERR_ALIGN
    assert conv(lib, E=1 << 30) == ERR_DIM  # 64 rows of this width overflow 32-bit offsets
    assert conv(lib, b=0, v=None, q=None, x=None) == OK
    assert conv(lib, E=0, v=None, q=None, x=None) == OK


def test_conv_update_validation(lib):
    assert conv_update(lib, dtype=-1) == ERR_DTYPE
    assert conv_update(lib, K=0) == ERR_DIM
    assert conv_update(lib, K=9) == ERR_DIM
    assert conv_update(lib, E=-1) == ERR_DIM
    for k in ("state", "v", "q", "x"):
        assert conv_update(lib, **{k: None}) == ERR_NULL, k
    assert conv_update(lib, state=FAKE + 1, dtype=1) == ERR_ALIGN
    assert conv_update(lib, v=FAKE + 2) == ERR_ALIGN
    assert conv_update(lib, cb=FAKE + 2) == ERR_ALIGN
    assert conv_update(lib, b=0, state=None) == OK


def bwd(lib, **kw):
    args = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1, h0=None, dy=FAKE,
                dlast=None, du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dz=None, dbias=None, dh0=None,
                b=1, L=8, E=64, N=16, dtype=0)
    args.update(kw)
    a = args
    return lib.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["softplus"],
                            a["h0"], a["dy"], a["dlast"], a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"],
                            a["dz"], a["dbias"], a["dh0"], a["b"], a["L"], a["E"], a["N"], a["dtype"], None)


def test_bwd_validation(lib):
    assert bwd(lib, dtype=5) == ERR_DTYPE
    assert bwd(lib, N=0) == ERR_N
    assert bwd(lib, N=17) == ERR_N
    assert bwd(lib, L=-1) == ERR_DIM
    for k in ("u", "delta", "A", "B", "C", "dy", "du", "ddelta", "dA", "dB", "dC"):
        assert bwd(lib, **{k: None}) == ERR_NULL, k
    assert bwd(lib, z=FAKE) == ERR_NULL  # a gate needs its gradient buffer
    assert bwd(lib, du=FAKE + 2) == ERR_ALIGN
    assert bwd(lib, dz=FAKE + 1, z=FAKE, dtype=1) == ERR_ALIGN
    assert bwd(lib, dA=FAKE + 2) == ERR_ALIGN
    assert bwd(lib, dh0=FAKE + 1) == ERR_ALIGN
    assert bwd(lib, E=1 << 26) == ERR_DIM  # 64 rows of this width overflow 32-bit offsets
    assert bwd(lib, b=0, E=0, u=None, delta=None, A=None, B=None, C=None, dy=None, du=None, ddelta=None, dA=None,
               dB=None, dC=None) == OK


def fwd_save(lib, saved=FAKE, u=FAKE, b=1, L=200, E=64, N=16, dtype=0):
    return lib.ssm_scan_fwd_save(u, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, FAKE, None, saved, b, L, E, N,
                                 dtype, None)


def bwd_saved(lib, saved=FAKE, **kw):
    args = dict(u=FAKE, b=1, L=200, E=64, N=16, dtype=0, dy=FAKE)
    args.update(kw)
    a = args
    return lib.ssm_scan_bwd_saved(a["u"], FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, saved, a["dy"], None, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, None, None, None, None, a["b"], a["L"], a["E"], a["N"],
                                  a["dtype"], None)


def test_saved_state_entry_points_validation(lib):
    # the saved states are required as soon as the sequence is longer than one interval of 64
    assert fwd_save(lib, saved=None, L=65) == ERR_NULL
    assert bwd_saved(lib, saved=None, L=65) == ERR_NULL
    assert fwd_save(lib, saved=FAKE + 2) == ERR_ALIGN
    assert bwd_saved(lib, saved=FAKE + 2) == ERR_ALIGN
    # otherwise the checks of ssm_scan_fwd_from / ssm_scan_bwd apply
    assert fwd_save(lib, dtype=3) == ERR_DTYPE
    assert fwd_save(lib, N=0) == ERR_N
    assert fwd_save(lib, u=None) == ERR_NULL
    assert fwd_save(lib, b=-1) == ERR_DIM
    assert bwd_saved(lib, dtype=3) == ERR_DTYPE
    assert bwd_saved(lib, u=None) == ERR_NULL
    assert bwd_saved(lib, dy=None) == ERR_NULL
    assert bwd_saved(lib, E=1 << 26) == ERR_DIM
    # nothing to do: no saved states are needed, pointers are not looked at
    assert fwd_save(lib, saved=None, b=0, u=None) == OK
    assert fwd_save(lib, saved=None, E=0, u=None) == OK
    assert ssm.saved_states_shape(3, 64, 5, 4) == (3, 0, 5, 4)
    assert ssm.saved_states_shape(3, 65, 5, 4) == (3, 1, 5, 4)
    assert ssm.saved_states_shape(2, 65536, 5120, 16) == (2, 1023, 5120, 16)
    assert ssm.saved_states_shape(1, 0, 5, 4) == (1, 0, 5, 4)


def ssd(lib, x=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, h0=None, y=FAKE, last=None,
        b=1, L=8, H=2, P=64, N=16, dtype=1):
    return lib.ssm_ssd_fwd(x, delta, A, B, C, D, z, bias, 1, h0, y, last, b, L, H, P, N, dtype, None)


def test_ssd_validation(lib):
    assert ssd(lib, dtype=0) == ERR_DTYPE      # bf16 only
    assert ssd(lib, dtype=4) == ERR_DTYPE
    assert ssd(lib, P=32) == ERR_DIM
    assert ssd(lib, L=-1) == ERR_DIM
    for n in (0, 8, 24, 144):
        assert ssd(lib, N=n) == ERR_N, n
    for k in ("x", "delta", "A", "B", "C", "y"):
        assert ssd(lib, **{k: None}) == ERR_NULL, k
    assert ssd(lib, x=FAKE + 8) == ERR_ALIGN    # 16-byte rows
    assert ssd(lib, B=FAKE + 2) == ERR_ALIGN
    assert ssd(lib, delta=FAKE + 1) == ERR_ALIGN
    assert ssd(lib, last=FAKE + 2) == ERR_ALIGN
    assert ssd(lib, b=0, x=None, delta=None, A=None, B=None, C=None, y=None) == OK
    # a chunk's 129 rows of H * 64 bf16 channels must stay within 32-bit byte offsets
    assert ssd(lib, H=130056, L=1) == ERR_DIM
    assert ssd(lib, H=130055, L=1, x=None) == ERR_NULL  # the size is accepted; the null x is not


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    if not os.path.exists(ssm.library_path()):
        pytest.skip("libssm.so not built")
    b, L, E, N = 1, 4, 8, 4
    u = torch.zeros(b, L, E)
    A = -torch.ones(E, N)
    BC = torch.zeros(b, L, N)
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_scan_fwd(u, u, A, BC, BC)
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_state_update(torch.zeros(b, E, N), torch.zeros(b, E), torch.zeros(b, E), A,
                             torch.zeros(b, N), torch.zeros(b, N))
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_scan_bwd(u, u, A, BC, BC, u)
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_conv_fwd(u, torch.zeros(E, 4))
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_conv_update(torch.zeros(b, E, 4), torch.zeros(b, E), torch.zeros(E, 4))


def test_binding_raises_when_library_missing(monkeypatch):
    monkeypatch.setattr(ssm, "_lib", None)
    monkeypatch.setattr(ssm, "_LIB_PATH", "/nonexistent/libssm.so")
    with pytest.raises(ImportError, match="build the HIP library"):
        ssm.load_library()


def test_scan_plan_query(lib):
    # a tiny problem is one chunk; big batch x channel counts need no split
    assert ssm.ssm_scan_plan(1, 64, 16, 4, "f32") == ("chunked", 64, 1)
    assert ssm.ssm_scan_plan(256, 4096, 8192, 16, "bf16")[2] == 1
    chunked = {"path": "chunked"}
    for (b, L, E, N, dt) in [(32, 512, 512, 16, "f32"), (8, 2048, 1536, 16, "bf16"), (1, 65536, 5120, 16, "bf16"),
                             (3, 1003, 70, 5, "bf16"), (1, 1 << 20, 64, 16, "f32")]:
        path, cl, nc = ssm.ssm_scan_plan(b, L, E, N, dt, tuning=chunked)
        assert path == "chunked" and cl >= 1 and nc >= 1
        assert (nc - 1) * cl < L <= nc * cl, (b, L, E, cl, nc)  # chunks tile the sequence exactly
        assert cl * E * (4 if dt == "f32" else 2) < 2 ** 31  # 32-bit buffer offsets inside a chunk
    # the long sequence: 256 chunks x 80 channel blocks = 20480 waves, the target that
    # measured best; its single pass would chain 11 chunk maps per block, so the chunked
    # form runs
    assert ssm.ssm_scan_plan(1, 65536, 5120, 16, "bf16") == ("chunked", 256, 256)
    # the chunked form of the mid workload takes 64-step chunks (6144 waves); the block
    # workload (2048 waves at 64 steps) 32-step chunks
    assert ssm.ssm_scan_plan(8, 2048, 1536, 16, "bf16", tuning=chunked) == ("chunked", 64, 32)
    assert ssm.ssm_scan_plan(32, 512, 512, 16, "f32", tuning=chunked) == ("chunked", 32, 16)
    # by default both run the single pass (4 and 3 chunk maps per block), in 8-step chunks
    assert ssm.ssm_scan_plan(8, 2048, 1536, 16, "bf16") == ("single_pass", 8, 256)
    assert ssm.ssm_scan_plan(32, 512, 512, 16, "f32") == ("single_pass", 8, 64)
    # the tuning fields are honoured
    forced = {"path": "chunked", "target_waves": 100000, "min_chunk": 8}
    assert ssm.ssm_scan_plan(3, 1003, 70, 16, "bf16", tuning=forced) == ("chunked", 8, 126)
    assert ssm.ssm_scan_plan(3, 1003, 70, 16, "bf16", tuning=dict(forced, min_chunk=1000)) == ("chunked", 1000, 2)
    assert ssm.ssm_scan_plan(1, 65536, 5120, 16, "bf16", tuning={"path": "single_pass"}) == ("single_pass", 8, 8192)
    # a single pass that cannot run (too few channels per CU; rows that are not whole
    # 8-byte units) or an out-of-range field is refused
    for bad in [dict(b=1, L=4096, E=64, N=16, dtype="f32", tuning={"path": "single_pass"}),
                dict(b=8, L=4096, E=1538, N=16, dtype="bf16", tuning={"path": "single_pass"}),
                dict(b=8, L=4096, E=1536, N=16, dtype="bf16", tuning={"path": 7}),
                dict(b=8, L=4096, E=1536, N=16, dtype="bf16", tuning={"min_chunk": -1})]:
        with pytest.raises(ssm.SSMError, match="SSM_ERR_PLAN|-7|tuning"):
            ssm.ssm_scan_plan(**bad)
    # a row too wide for 32-bit offsets is rejected
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_plan(1, 4, 1 << 31, 16, "f32")


def test_profile_read_with_nothing_recorded(lib):
    out = ssm.ssm_profile_read()
    assert set(out) == {"widen_rows", "chunk_aggregate", "chunk_carry", "scan_main", "fill_state", "state_update",
                        "conv", "conv_update", "bwd_rows", "bwd_aggregate", "bwd_carry", "bwd_main", "bwd_reduce", "ssd_state", "ssd_carry", "ssd_scan",
                        "scan_fused"}
    assert all(v == (0.0, 0) for v in out.values())
