"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle (``oracle/ssm_oracle.c``), built with gcc and
  ``-fsanitize=address,undefined``, runs every one of its functions on small
  inputs (``tests/sanitize/oracle_driver.c``): optional arguments present and
  absent, several thread counts, L = 0 and one-element sizes.
* The library's host code (argument checks, plans, status and profiling
  queries), built with hipcc with the sanitizers on the host side only
  (``-Xarch_host``; the kernels are compiled as usual and never launched here),
  is driven through the C ABI by ``tests/sanitize/api_driver.c``: every entry
  point's refusals, plans over sizes up to 2^48 and past it, and valid calls
  that stop at the first HIP call on a host without a GPU.

Any sanitizer report aborts the driver with a non-zero status.  Leak detection
is off for the library driver because the HIP runtime it loads keeps its own
allocations until exit.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_35_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread",
                   os.path.join(ROOT, "oracle", "ssm_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe,
                   "-lm"])
    assert rc == 0, out
    rc, out = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert rc == 0 and "oracle driver: ok" in out, out


@pytest.mark.timeout(900)
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and ROCm clang")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from selective_state_space_35_amd import build as lib_build

    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    common = [f for f in lib_build.COMMON if f != "-O3"] + ["-O1", "-g"]
    objs = [str(tmp_path / s.replace(".hip", ".o")) for s in lib_build.SOURCES]

    def compile_one(i):
        return run([HIPCC, *common, *san, "-c", os.path.join(CSRC, lib_build.SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(8, len(objs))) as ex:
        for rc, out in ex.map(compile_one, range(len(objs))):
            assert rc == 0, out
    lib = str(tmp_path / "libssm_asan.so")
    rc, out = run([HIPCC, f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC", *san, "-o", lib, *objs])
    assert rc == 0, out
    exe = str(tmp_path / "api_driver")
    rc, out = run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "api_driver.c"), f"-L{tmp_path}",
                   "-lssm_asan", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    rc, out = run([exe], env=env)
    assert rc == 0 and "api driver: ok" in out, out
