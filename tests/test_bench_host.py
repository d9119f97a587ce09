"""Host-side checks of bench.py (no GPU).

* The command line keeps to one GPU: ``--gpus 2``, or a launcher's WORLD_SIZE
  above 1, ends with exit status 2 and a message, before anything touches a GPU;
  without a GPU the bench stops with exit status 1 instead of timing anything
  else (there is no CPU path to fall back to).
* The algorithmic byte and VALU-slot models that the bench divides by kernel
  time, against figures worked out here by hand from the tensor sizes of the
  long-sequence scan (b1 L65536 E5120 N16 bf16, gate, D, no step bias) and of
  the generation-time state update (b256 E5120 N16 bf16, gate, D, step bias).
* A traffic figure measured on another kernel source is dropped (null), and one
  taken on the current source is passed through.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

BENCH = os.path.join(ROOT, "bench.py")


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_launcher_world_size_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr
    assert r.stdout == ""


def test_no_gpu_stops_the_bench():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the bench would run")
    r = run_bench(["--steps", "1", "--warmup", "0", "--no-cpu-baseline"])
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def test_scan_bytes_of_the_long_workload():
    elems = 1 * 65536 * 5120
    streams = 4 * elems * 2                 # u, delta, z read and y written, bf16
    rows = 2 * 65536 * 16 * 2               # B and C, bf16
    params = 5120 * 16 * 4 + 2 * 5120 * 4   # A, and D and the step bias (counted by the model either way)
    last = 5120 * 16 * 4                    # last_state, fp32
    assert bench.scan_bytes(1, 65536, 5120, 16, 2, gate=True) == streams + rows + params + last == 2_689_245_184
    # without the gate one stream fewer, without last_state no state write
    assert bench.scan_bytes(1, 65536, 5120, 16, 2, gate=False, last_state=False) == 3 * elems * 2 + rows + params


def test_scan_slots_of_the_long_workload():
    # a transcendental takes one issue slot like any VALU instruction
    assert bench.TRANS_SLOTS == 1
    # per (t, e, n): step times A, exp2, d u times B, the state update, the readout -> 5
    # per (t, e): d u (1), softplus 2 exp/log + 4, D u (1), silu gate 2 transcendentals + 4,
    #             bf16 widening of u, delta, z and rounding of y (4)
    per_elem = 5 * 16 + 1 + 6 + 1 + 6 + 4
    assert per_elem == 98
    got = bench.scan_slots(1, 65536, 5120, 16, softplus=True, gate=True, has_d=True, has_bias=False, bf16=True)
    assert got == 98 * 65536 * 5120
    # fp32 I/O drops the widening and rounding; a step bias adds one slot per (t, e)
    got = bench.scan_slots(1, 64, 16, 4, softplus=True, gate=False, has_d=True, has_bias=True, bf16=False)
    assert got == 64 * 16 * (5 * 4 + 1 + 1 + 6 + 1)
    # the peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (non-packed fp32)
    assert bench.VALU_SLOT_PEAK == 256 * 4 * 16 * 2.4e9


def test_update_bytes_of_the_decode_workload():
    b, E, N = 256, 5120, 16
    state = 2 * b * E * N * 4        # read and written, fp32
    tokens = 4 * b * E * 2           # x, delta, z in and y out, bf16
    rows = 2 * b * N * 2             # B and C, bf16
    params = E * N * 4 + 2 * E * 4   # A, D, step bias
    assert bench.update_bytes(b, E, N, 2) == state + tokens + rows + params == 178_642_944


def test_profiles_need_the_current_kernel_source(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_scan_long.json")
    with open(path) as f:
        doc = json.load(f)
    monkeypatch.setattr(bench, "source_hash", lambda: doc["source_hash"])
    got, note = bench.load_profile("traffic_scan_long")
    assert got == doc and note == ""
    assert got["kernels"]["scan_main_kernel"]["hbm_bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    got, note = bench.load_profile("traffic_scan_long")
    assert got is None and "changed" in note
    got, note = bench.load_profile("traffic_no_such_workload")
    assert got is None and "no summary" in note


def test_source_hash_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "selective_state_space_35_amd", "csrc")
    names = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    assert {"ssm_kernels.hip", "ssm_fused.hip", "ssm_chain.h", "ssm_device.h"} <= names
    assert len(bench.source_hash()) == 16


def test_kernel_names_of_the_profiles():
    assert bench._split("void ssm::(anonymous namespace)::scan_fused_kernel<unsigned short, 4, true, true, false>"
                        "(unsigned short const*, float)") == (
        "scan_fused_kernel", "scan_fused_kernel<unsigned short, 4, true, true, false>")
    assert bench._short("void ssm::chain_kernel<1, 32, false, false, false>(ssm::ChainArgs)") == "chain_kernel"
    assert bench._short("void at::native::elementwise_kernel<128, 2, direct_copy_kernel_cuda>(int)") == "copy"


def test_profile_summaries_keep_every_library_kernel():
    """Every __global__ kernel of the library is one the profile summaries keep (none is dropped as foreign)."""
    import re

    csrc = os.path.join(ROOT, "selective_state_space_35_amd", "csrc")
    found = set()
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".h")):
            text = open(os.path.join(csrc, f)).read()
            found |= set(re.findall(r"__global__.{0,200}?\bvoid\s+(\w+)\s*\(", text, flags=re.S))
    assert "bwd_chunk_maps_kernel" in found and "scan_main_kernel" in found
    assert found <= set(bench.LIB_KERNELS), found - set(bench.LIB_KERNELS)
