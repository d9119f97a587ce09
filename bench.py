#!/usr/bin/env python3
"""Benchmark of the MI355X selective scan (Mamba-1 / S6 forward) on one GPU.

One step = one ``ssm_scan_fwd`` call over the long-sequence workload
(b=1, L=65536, E=5120, N=16, bf16 inputs/outputs, fp32 state, softplus step,
silu gate, D skip), with inputs already resident in HBM.  That call runs the
whole hot path: discretisation, recurrence, readout, gate and the last-state
write.  The single-token state update is measured as well (128 successive
updates of the generation workload b=256, E=5120, N=16) and reported in its
own JSON object, and so are the causal convolution that precedes the scan
(b1 L65536 E5120 K4 bf16, and its token step at b256 E5120 K4), the scan's
backward on the long workload, and the scan with a scalar transition per head
(b1 L65536 H80 P64 N64 bf16, chunked MFMA form).

Prints ONE JSON line on stdout:
  value        b*L*E elements per second over the timed steps
  roofline     ALU roofline of the dominant kernel (the main pass of the chunked form, or the single-pass
               kernel): algorithmic VALU issue slots of one pass (one non-packed fp32 lane-op per slot, a
               transcendental included) over its duration, measured with HIP events on the launch stream
               over the timed region, against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13 slot/s;
               `hbm` holds the HBM view of the same kernel and of the whole call (algorithmic bytes over
               time vs 8 TB/s); traffic (L2-to-fabric bytes per launch) and VALU busy per kernel come from
               the committed rocprofv3 summaries in profiles/ when they were taken on the current kernel
               sources, else null
  cpu_baseline the fp64 oracle on a bounded channel sample of the same inputs
               (channels are independent chains), timed on the host cores
  configs      the tiny (b1 L64 E16 N4 fp32), block (b32 L512 E512 N16 fp32) and
               mid (b8 L2048 E1536 N16 bf16) scans and the long scan's one-GPU
               share under 8-way channel sharding (E640), each call timed on its
               own: median and min, elem/s, algorithmic GB/s against 8 TB/s and
               against a measured 1 GiB copy, ALU-issue fraction; the oracle's
               rate on 1 and on all host threads, and parity of the timed outputs

Other modes: --alu-calibration (issue rates of single instruction kinds), --copy-calibration (a 1 GiB copy
for the byte counters), --summarize RUN_ROOT (no GPU: profiles/ summaries from rocprofv3 output).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--workload long]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
# VALU issue peak in lane-slots/s: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13.  A wave64 VALU
# instruction holds a SIMD for 4 cycles; one slot is one non-packed fp32 lane-op (78.6 TFLOP/s of FMA;
# the library is built with packed FP32 disabled, so 157.3 TFLOP/s, the packed rate, is out of reach).
VALU_SLOT_PEAK = 256 * 4 * 16 * 2.4e9
# Slots a v_exp_f32 (and the other fp32 transcendentals) takes: one, like any VALU instruction.  In the scan
# kernels' mix (a fifth of the instructions transcendental) the long scan's main pass issues 5.30e8 wave64
# VALU instructions in 976 us, 4.52 cycles each at 2.4 GHz: 88% of one instruction per 4 cycles per SIMD
# (profiles/sq_scan_long.txt); two slots per transcendental would put that kernel at 103% of the peak.  The
# standalone calibration kinds (profiles/alu_issue_rates.txt) bound the cost from above: an exp alone takes
# 9.4 cycles, and beside 4 dependent-free FMAs it added 8.1.
TRANS_SLOTS = 1
# profile kinds of ssm_profile_read() -> the kernel symbol they time
KIND_SYMBOL = {"chunk_aggregate": "scan_chunk_agg_kernel", "chunk_carry": "chain_kernel", "scan_main": "scan_main_kernel",
               "scan_fused": "scan_fused_kernel", "widen_rows": "widen_rows_kernel", "state_update": "state_update_kernel",
               "bwd_main": "bwd_main_kernel", "ssd_scan": "ssd_scan_kernel", "ssd_state": "ssd_state_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_bytes(b, L, E, N, s, gate=True, last_state=True):
    """Algorithmic HBM bytes of one scan: u, delta (, z) in and y out at s bytes each; B and C rows;
    A, D (and bias); the fp32 last state."""
    streams_in = 3 if gate else 2
    by = b * L * E * (streams_in + 1) * s + 2 * b * L * N * s + E * (N + 2) * 4
    if last_state:
        by += b * E * N * 4
    return by


def scan_slots(b, L, E, N, softplus=True, gate=True, has_d=True, has_bias=False, bf16=True):
    """Algorithmic fp32 VALU lane-slots of one scan pass (the minimal single pass).

    Per (t, e, n): d*A2 (1), exp2 (TRANS_SLOTS), du*B (1), a*h + w (1), C*h + acc (1)     -> 4 + TRANS_SLOTS
    Per (t, e):    delta + bias (1); softplus: 2 transcendentals + 4 VALU; d*u (1); D*u (1);
                   silu gate: 2 transcendentals + 3 VALU, and the product; bf16 widening of each
                   streamed input and rounding of y (1 each)
    """
    per_te = 1  # d * u
    per_te += 1 if has_bias else 0
    per_te += 2 * TRANS_SLOTS + 4 if softplus else 0
    per_te += 1 if has_d else 0
    per_te += 2 * TRANS_SLOTS + 4 if gate else 0
    per_te += (3 if gate else 2) + 1 if bf16 else 0
    return b * L * E * ((4 + TRANS_SLOTS) * N + per_te)


def update_bytes(b, E, N, s, gate=True):
    """Algorithmic bytes of one state update: fp32 state read + write, x, delta (, z) in, y out, B, C, A, D."""
    return 8 * b * E * N + b * E * ((3 if gate else 2) + 1) * s + 2 * b * N * s + E * (N + 2) * 4


def bwd_bytes(b, L, E, N, s, gate=True):
    """Algorithmic bytes of one backward call: u, delta (, z), dy and B, C read; du, ddelta (, dz) written
    in the I/O dtype; dB, dC [b, L, N] and dA, dD, dbias written in float32; A, D, bias read."""
    streams = (4 if gate else 3) + (3 if gate else 2)
    return b * L * E * streams * s + 2 * b * L * N * s + 2 * b * L * N * 4 + 2 * E * (N + 2) * 4


def ssd_bytes(b, L, H, P, N, s, gate=True):
    """Algorithmic bytes of one scalar-per-head scan: x (, z) in and y out; delta; B, C; A, D; the last state."""
    E = H * P
    return b * L * E * ((2 if gate else 1) + 1) * s + b * L * H * s + 2 * b * L * N * s + 2 * H * 4 + b * E * N * 4


def ssd_flops(b, L, H, P, N, Q=128):
    """Matrix-product flops of the chunked form: C B^T (causal half), L o (C B^T) X (causal half), C S_in, B^T (w o X)."""
    chunks = (L + Q - 1) // Q
    per = Q * Q * N + Q * Q * P + 2 * Q * N * P  # multiply-adds per (chunk, head), causal halves counted
    return 2 * b * H * chunks * per


def conv_bytes(b, L, E, K, s, bias=True):
    """Algorithmic bytes of one causal convolution: v in, x out, the weights (and bias), the K-sample state out."""
    return 2 * b * L * E * s + E * K * 4 + (E * 4 if bias else 0) + b * E * K * s


def conv_update_bytes(b, E, K, s, bias=True):
    """Algorithmic bytes of one convolution token step: state read + write, v in, x out, weights (and bias)."""
    return 2 * b * E * K * s + 2 * b * E * s + E * K * 4 + (E * 4 if bias else 0)


HASH_EXCLUDES = ("ssm_api.hip",)  # the C ABI's argument checks: no kernel, no launch shape


def source_hash():
    """sha256[:16] of every library source that builds a kernel or plans a launch (all of csrc/ but the argument
    checks): a profile taken on other sources is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_35_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")) and f not in HASH_EXCLUDES:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def load_profile(name):
    """A committed profile summary (profiles/<name>.json) and whether it was taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(path):
        return None, "no summary in profiles/"
    with open(path) as f:
        doc = json.load(f)
    if doc.get("source_hash") != source_hash():
        return None, "kernel sources changed since the counters were taken"
    return doc, ""


def cpu_facts():
    """The host as the CPU baseline sees it: model strings from /proc/cpuinfo, nproc, the cores this
    process may run on, and OMP_NUM_THREADS (the share of the host a job is given, where set)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break  # the first processor's block is enough
                    continue
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("vendor_id", "model name", "cpu family", "model", "stepping", "cpu MHz", "cache size",
                         "siblings", "cpu cores"):
                    fields[k] = v
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpuinfo": fields, "nproc": os.cpu_count(), "affinity_cores": affinity,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def copy_bandwidth(torch, dev, stream, nbytes=1 << 30, reps=10):
    """GB/s of a plain device-to-device copy (bytes read + bytes written over its time)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    del src
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, dst


def scan_configs(ssm, workloads, torch, dev, stream, seed, cpu=True):
    """Each scan configuration timed call by call, with the oracle beside it.

    The block and mid configurations are small enough to stay in the 256 MB
    Infinity Cache between calls, so a 1 GiB buffer is written before every
    timed call (outside its event pair).  A 1 GiB read does not do it: it
    leaves a state of 84 MB in the cache (the decode leg's evicted_by_read
    figure equals its resident one).  The written lines are dirty, so part of
    their write-back to HBM runs inside the timed call.  The tiny one is
    launch-bound.  The
    long workload's share at E = 640 is what one GPU of 8 runs when the
    channels are split over them.  With ``cpu``, the fp64 oracle runs on the
    same inputs, on 1 thread and on the host's threads, and checks the
    timed outputs elementwise.
    """
    import numpy as np

    copy_gbps, flush = copy_bandwidth(torch, dev, stream)
    out = {"copy_GBps": round(copy_gbps, 1),
           "copy_note": "1 GiB device-to-device copy: bytes read + written over its time",
           "timing": "event pair around each call on the launch stream; median and min over the calls"}
    if cpu:
        import oracle

        threads = oracle.default_threads()
    for wc, reps, flushed, t1 in ((workloads.TINY, 200, False, True), (workloads.BLOCK, 100, True, True),
                                  (workloads.MID, 100, True, True), (workloads.LONG_E640, 20, False, False)):
        xc = workloads.make_scan_inputs(wc, seed=seed, device=dev, backend="torch" if wc.L * wc.E > 1 << 24 else "numpy")
        yc = torch.empty_like(xc["u"])
        lc = torch.empty((wc.b, wc.E, wc.N), dtype=torch.float32, device=dev)

        def call():
            ssm.ssm_scan_fwd(xc["u"], xc["delta"], xc["A"], xc["B"], xc["C"], xc["D"], xc["z"],
                             xc["delta_bias"], xc["softplus"], y=yc, last_state=lc)

        for _ in range(5):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for k in range(reps):
            if flushed:
                flush.fill_(k & 0x7F)
            ev[k][0].record(stream)
            call()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        us = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
        med, mn = us[len(us) // 2], us[0]
        s = 2 if wc.dtype == "bf16" else 4
        nb = scan_bytes(wc.b, wc.L, wc.E, wc.N, s, gate=wc.z is not None)
        sl = scan_slots(wc.b, wc.L, wc.E, wc.N, softplus=wc.softplus, gate=wc.z is not None,
                        has_d=wc.D is not None, has_bias=wc.delta_bias is not None, bf16=(wc.dtype == "bf16"))
        el = wc.b * wc.L * wc.E
        gbps = nb / (med * 1e-6) / 1e9
        rec = {"workload": wc.description, "calls": reps,
               "cache_flushed": "1 GiB written before each call" if flushed else False,
               "us_median": round(med, 2), "us_min": round(mn, 2), "elem_per_s": el / (med * 1e-6),
               "algorithmic_bytes": nb, "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
               "copy_frac": round(gbps / copy_gbps, 4),
               "alu_frac": round(sl / (med * 1e-6) / VALU_SLOT_PEAK, 4),
               "plan": dict(zip(("path", "chunk_len", "n_chunks"),
                                ssm.ssm_scan_plan(wc.b, wc.L, wc.E, wc.N, wc.dtype)))}
        if cpu:
            a64 = [oracle.to_f64(xc[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
            rates = {}
            for th in ((1, threads) if t1 else (threads,)):
                c0 = time.perf_counter()
                y_ref, last_ref = oracle.scan(*a64, softplus=xc["softplus"], threads=th)
                rates[f"threads_{th}"] = el / (time.perf_counter() - c0)
            rec["cpu_oracle_elem_per_s"] = rates
            err = lambda g, r: float(np.max(np.abs(g - r) / (1 + np.abs(r)))) if r.size else 0.0
            bound = 2e-2 if wc.dtype == "bf16" else 1e-4
            rec["parity"] = {"y": err(oracle.to_f64(yc), y_ref), "last_state": err(oracle.to_f64(lc), last_ref),
                             "bound": bound}
        out[wc.name] = rec
        del xc, yc, lc
    del flush
    if cpu:  # the decode workload on the host: a sample of its token steps (the GPU side is state_update)
        wd = workloads.DECODE.with_shape(steps=8)
        xd = workloads.make_decode_inputs(wd, seed=seed, device=dev, backend="torch")
        xd = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in xd.items()}
        rates = {}
        for th in (1, threads):
            st = oracle.to_f64(xd["state0"])
            c0 = time.perf_counter()
            for k in range(wd.steps):
                st, _ = oracle.state_update(st, xd["x"][k], xd["delta"][k], xd["A"], xd["B"][k], xd["C"][k], xd["D"],
                                            xd["z"][k], xd["delta_bias"], xd["softplus"], threads=th)
            rates[f"threads_{th}"] = round(1e6 * (time.perf_counter() - c0) / wd.steps, 1)
        out["decode"] = {"workload": workloads.DECODE.description, "cpu_oracle_us_per_call": rates,
                         "sample": f"the first {wd.steps} of {workloads.DECODE.steps} token steps"}
    return out


def measure_decode(ssm, torch, workloads, dev, stream, seed):
    """128 successive state updates of the decode workload, and the token step (eager and from a HIP graph)."""
    wd = workloads.DECODE
    xd = workloads.make_decode_inputs(wd, seed=seed, device=dev, backend="torch")
    st = xd["state0"].clone()
    yd = torch.empty(wd.b, wd.E, dtype=torch.bfloat16, device=dev)

    def decode_pass():
        for k in range(wd.steps):
            ssm.ssm_state_update(st, xd["x"][k], xd["delta"][k], xd["A"], xd["B"][k], xd["C"][k], xd["D"],
                                 xd["z"][k], xd["delta_bias"], xd["softplus"], y=yd)

    decode_pass()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ssm.ssm_profile_enable(True)
    e0.record(stream)
    for _ in range(reps):
        st.zero_()
        decode_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    upd = ssm.ssm_profile_read()["state_update"]
    per_call_us = 1e3 * upd[0] / upd[1]
    ub = update_bytes(wd.b, wd.E, wd.N, 2)
    update = {"workload": wd.description, "us_per_call": round(per_call_us, 3),
              "calls": upd[1], "wall_ms_per_128": round(e0.elapsed_time(e1) / reps, 4),
              "GBps": round(ub / (per_call_us * 1e-6) / 1e9, 1),
              "bytes_per_call": ub,
              "note": "the 84 MB fp32 state fits in the 256 MB Infinity Cache, so carried-state traffic "
                      "can be served from it; GB/s is algorithmic bytes over kernel time"}
    # where the carried state comes from: the same calls with a 1 GiB buffer written between them (outside
    # each call's event pair), which evicts the state from the Infinity Cache, so every call reads it from HBM
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_words = flush.view(torch.int64)
    res, evi, evr = [], [], []
    for k in range(wd.steps):
        for how, acc in ((None, res), ("write", evi), ("read", evr)):
            if how == "write":
                flush.fill_(k & 0x7F)
            elif how == "read":
                flush_words.max()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            ssm.ssm_state_update(st, xd["x"][k], xd["delta"][k], xd["A"], xd["B"][k], xd["C"][k], xd["D"],
                                 xd["z"][k], xd["delta_bias"], xd["softplus"], y=yd)
            a1.record(stream)
            acc.append((a0, a1))
    torch.cuda.synchronize()
    med = lambda ev: sorted(1e3 * a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
    r_us, e_us, er_us = med(res), med(evi), med(evr)
    update["state_source"] = {
        "resident_us_median": round(r_us, 3), "evicted_us_median": round(e_us, 3),
        "evicted_by_read_us_median": round(er_us, 3),
        "resident_GBps": round(ub / (r_us * 1e-6) / 1e9, 1), "evicted_GBps": round(ub / (e_us * 1e-6) / 1e9, 1),
        "evicted_hbm_frac": round(ub / (e_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "note": "each call timed alone with an event pair: right after the previous call (state in the Infinity "
                "Cache) and after a 1 GiB write that evicts it (state from HBM); the evicted rate is the HBM "
                "figure, the difference is what the cache serves. evicted_by_read: the same after a 1 GiB read "
                "instead, which does not evict the state (a read flush is not used anywhere)"}
    del flush, flush_words

    # one generation step of the block's kernels per token: the convolution token step, then the state
    # update on its output; eager launches against the same T tokens captured once in a HIP graph
    def token_step(bt, T=32):
        g2 = torch.Generator(device=dev).manual_seed(seed + 5)
        v_tok = torch.randn((T, bt, wd.E), generator=g2, device=dev).to(torch.bfloat16)
        dl = torch.randn((T, bt, wd.E), generator=g2, device=dev).to(torch.bfloat16)
        Bt = torch.randn((T, bt, wd.N), generator=g2, device=dev).to(torch.bfloat16)
        Ct = torch.randn((T, bt, wd.N), generator=g2, device=dev).to(torch.bfloat16)
        zt = torch.randn((T, bt, wd.E), generator=g2, device=dev).to(torch.bfloat16)
        q = torch.randn((wd.E, 4), generator=g2, device=dev) * 0.5
        cb = torch.randn((wd.E,), generator=g2, device=dev) * 0.1
        cst = torch.zeros((bt, wd.E, 4), dtype=torch.bfloat16, device=dev)
        sst = torch.zeros((bt, wd.E, wd.N), dtype=torch.float32, device=dev)
        xs = torch.empty((T, bt, wd.E), dtype=torch.bfloat16, device=dev)
        ys = torch.empty((T, bt, wd.E), dtype=torch.bfloat16, device=dev)

        def tokens():
            for k in range(T):
                ssm.ssm_conv_update(cst, v_tok[k], q, cb, x=xs[k])
                ssm.ssm_state_update(sst, xs[k], dl[k], xd["A"], Bt[k], Ct[k], xd["D"], zt[k],
                                     xd["delta_bias"], xd["softplus"], y=ys[k])

        tokens()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            tokens()
        t1.record(stream)
        torch.cuda.synchronize()
        eager_us = 1e3 * t0.elapsed_time(t1) / (reps * T)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            tokens()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            tokens()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        graph_us = 1e3 * t0.elapsed_time(t1) / (reps * T)
        del graph
        return {"eager_us_per_token": round(eager_us, 2), "graph_us_per_token": round(graph_us, 2)}

    update["token_step"] = {
        "workload": f"per token: ssm_conv_update (K4) then ssm_state_update, E{wd.E} N{wd.N} bf16, 32 tokens",
        "b256": token_step(wd.b), "b1": token_step(1),
        "note": "both entry points launch on the caller's stream with no workspace and no memset, so the "
                "token loop can be captured in a HIP graph (torch.cuda.CUDAGraph) and replayed; at b1 the "
                "step is launch-bound"}
    log(f"[bench] token step {update['token_step']}")
    del xd, st, yd
    return update


def measure_backward(ssm, torch, dev, stream, x, w, steps, seed):
    """ssm_scan_bwd on the long workload, and the training form (forward with saved states, backward from them)."""
    s = 2 if w.dtype == "bf16" else 4
    elems = w.b * w.L * w.E
    gen = torch.Generator(device=dev).manual_seed(seed + 11)
    dy = torch.randn(x["u"].shape, generator=gen, device=dev).to(x["u"].dtype)

    def bwd_step():
        return ssm.ssm_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, x["D"], x["z"],
                                x["delta_bias"], x["softplus"])

    for _ in range(2):
        g = bwd_step()
    del g
    torch.cuda.synchronize()
    ssm.ssm_profile_read()
    ssm.ssm_profile_enable(True)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, steps // 5)
    b0.record(stream)
    for _ in range(reps):
        g = bwd_step()
    b1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    del g
    prof = ssm.ssm_profile_read()
    bwd_ms = b0.elapsed_time(b1) / reps
    bb = bwd_bytes(w.b, w.L, w.E, w.N, s, gate=w.z is not None)
    bwd = {"workload": "backward of the long-sequence scan (same inputs, dy ~ N(0,1) bf16)",
           "ms_per_call": round(bwd_ms, 4), "elem_per_s": elems / (bwd_ms * 1e-3),
           "algorithmic_bytes": bb, "GBps": round(bb / (bwd_ms * 1e-3) / 1e9, 1),
           "kernels": {k: {"avg_us": round(1e3 * v[0] / v[1], 2), "launches": v[1]}
                       for k, v in prof.items() if v[1]},
           "note": "includes the workspace allocation and the chunk maps it recomputes (bwd_aggregate: the "
                   "forward and reverse maps of every chunk in one walk; chunk_carry and bwd_carry: their chains)"}
    log(f"[bench] backward {bwd}")

    # training form: the forward keeps the state every 64 steps, the backward starts its chunks from them
    saved = torch.empty(ssm.saved_states_shape(w.b, w.L, w.E, w.N), dtype=torch.float32, device=dev)
    ys = torch.empty_like(x["u"])

    def fwd_save():
        ssm.ssm_scan_fwd_save(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                              x["softplus"], y=ys, saved_states=saved)

    def bwd_saved():
        return ssm.ssm_scan_bwd_saved(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, saved, x["D"], x["z"],
                                      x["delta_bias"], x["softplus"])

    fwd_save()
    g = bwd_saved()
    del g
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(reps):
        fwd_save()
    f1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_read()
    ssm.ssm_profile_enable(True)
    b0.record(stream)
    for _ in range(reps):
        g = bwd_saved()
    b1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    del g
    prof = ssm.ssm_profile_read()
    fs_ms, bs_ms = f0.elapsed_time(f1) / reps, b0.elapsed_time(b1) / reps
    bwd["from_saved_states"] = {
        "forward_with_save_ms": round(fs_ms, 4), "backward_ms": round(bs_ms, 4),
        "saved_bytes": saved.numel() * 4,
        "kernels": {k: {"avg_us": round(1e3 * v[0] / v[1], 2), "launches": v[1]} for k, v in prof.items() if v[1]},
        "note": "ssm_scan_fwd_save keeps the state every 64 steps (1/64 of the states); ssm_scan_bwd_saved "
                "starts its 64-step chunks from them instead of rerunning the forward chunk-state passes"}
    log(f"[bench] backward from saved states {bwd['from_saved_states']}")
    del dy, saved, ys
    return bwd


def measure_ssd(ssm, torch, workloads, dev, stream, seed, cpu=True):
    """ssm_ssd_fwd on the scalar-per-head workload, with its per-kernel split; with ``cpu``, the fp64 oracle
    checks the timed outputs on a sample of heads."""
    ws = workloads.SSD_LONG
    xs = workloads.make_ssd_inputs(ws, seed=seed, device=dev, backend="torch")
    ys = torch.empty_like(xs["x"])
    ls = torch.empty((ws.b, ws.E, ws.N), dtype=torch.float32, device=dev)

    def ssd_step():
        ssm.ssm_ssd_fwd(xs["x"], xs["delta"], xs["A"], xs["B"], xs["C"], xs["D"], xs["z"], xs["delta_bias"],
                        xs["softplus"], y=ys, last_state=ls)

    for _ in range(3):
        ssd_step()
    torch.cuda.synchronize()
    ssm.ssm_profile_read()
    ssm.ssm_profile_enable(True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(20):
        ssd_step()
    s1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    prof = ssm.ssm_profile_read()
    ssd_ms = s0.elapsed_time(s1) / 20
    sb = ssd_bytes(ws.b, ws.L, ws.H, ws.P, ws.N, 2, gate=ws.gate)
    sf = ssd_flops(ws.b, ws.L, ws.H, ws.P, ws.N)
    ssd = {"workload": ws.description, "ms_per_call": round(ssd_ms, 4),
           "elem_per_s": ws.b * ws.L * ws.E / (ssd_ms * 1e-3), "algorithmic_bytes": sb,
           "GBps": round(sb / (ssd_ms * 1e-3) / 1e9, 1), "matrix_TFLOPs": round(sf / (ssd_ms * 1e-3) / 1e12, 2),
           "kernels": {k: {"avg_us": round(1e3 * v[0] / v[1], 2), "launches": v[1]}
                       for k, v in prof.items() if v[1]}}
    if cpu:  # heads are independent: the oracle on a head sample is exactly that sample of the oracle
        import numpy as np

        import oracle

        rng = np.random.default_rng(seed + 3)
        heads = sorted({0, ws.H - 1, *rng.choice(ws.H, size=2, replace=False).tolist()})
        hs = torch.tensor(heads, device=dev)
        ch = (hs[:, None] * ws.P + torch.arange(ws.P, device=dev)[None, :]).reshape(-1)
        sel = lambda t, idx, dim: None if t is None else t.index_select(dim, idx)
        c0 = time.perf_counter()
        y_ref, l_ref = oracle.ssd(sel(xs["x"], ch, 2), sel(xs["delta"], hs, 2), sel(xs["A"], hs, 0), xs["B"],
                                  xs["C"], sel(xs["D"], hs, 0), sel(xs["z"], ch, 2), sel(xs["delta_bias"], hs, 0),
                                  xs["softplus"])
        err = lambda g, r: float(np.max(np.abs(g - r) / (1 + np.abs(r))))
        ssd["parity"] = {"y_max_normalised_error": err(oracle.to_f64(ys.index_select(2, ch)), y_ref),
                         "last_state_max_normalised_error": err(oracle.to_f64(ls.index_select(1, ch)), l_ref),
                         "bound": 2e-2, "heads_checked": heads, "oracle_seconds": round(time.perf_counter() - c0, 2)}
    log(f"[bench] ssd {ssd}")
    del xs, ys, ls
    return ssd


def measure_conv(ssm, torch, workloads, dev, seed):
    """ssm_conv_fwd on the long workload and ssm_conv_update on the decode workload."""
    wc = workloads.CONV_LONG
    xc = workloads.make_conv_inputs(wc, seed=seed, device=dev, backend="torch")
    xo = torch.empty_like(xc["v"])
    so = torch.empty((wc.b, wc.E, wc.K), dtype=xc["v"].dtype, device=dev)
    for _ in range(3):
        ssm.ssm_conv_fwd(xc["v"], xc["weight"], xc["conv_bias"], None, x=xo, state_out=so)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(True)
    for _ in range(20):
        ssm.ssm_conv_fwd(xc["v"], xc["weight"], xc["conv_bias"], None, x=xo, state_out=so)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    cf = ssm.ssm_profile_read()["conv"]
    cf_us = 1e3 * cf[0] / cf[1]
    cb_ = conv_bytes(wc.b, wc.L, wc.E, wc.K, 2)
    del xc, xo, so
    wu = workloads.CONV_DECODE
    xu = workloads.make_conv_inputs(wu, seed=seed, device=dev, backend="torch")
    cst = xu["state_in"].clone()
    v_t = xu["v"][:, 0].contiguous()
    xt = torch.empty_like(v_t)
    for _ in range(3):
        ssm.ssm_conv_update(cst, v_t, xu["weight"], xu["conv_bias"], x=xt)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(True)
    for _ in range(128):
        ssm.ssm_conv_update(cst, v_t, xu["weight"], xu["conv_bias"], x=xt)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    cu = ssm.ssm_profile_read()["conv_update"]
    cu_us = 1e3 * cu[0] / cu[1]
    ub_ = conv_update_bytes(wu.b, wu.E, wu.K, 2)
    conv = {"sequence": {"workload": wc.description, "us_per_call": round(cf_us, 2), "calls": cf[1],
                         "bytes_per_call": cb_, "GBps": round(cb_ / (cf_us * 1e-6) / 1e9, 1),
                         "frac": round(cb_ / (cf_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
            "token": {"workload": wu.description, "us_per_call": round(cu_us, 3), "calls": cu[1],
                      "bytes_per_call": ub_, "GBps": round(ub_ / (cu_us * 1e-6) / 1e9, 1)}}
    log(f"[bench] conv {conv}")
    del xu, cst, v_t, xt
    return conv


def measure_cpu_baseline(torch, dev, x, w, y, last, cpu_seconds):
    """The fp64 oracle on a bounded channel sample of the long workload's inputs, timed on the host
    cores, and the parity of the GPU outputs on those channels."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    rng = np.random.default_rng(1)

    def sample(nch):
        ch = torch.from_numpy(np.sort(rng.choice(w.E, size=nch, replace=False))).to(dev)
        sel = lambda t: None if t is None else t.index_select(2, ch)
        args_ = (sel(x["u"]), sel(x["delta"]), x["A"].index_select(0, ch), x["B"], x["C"],
                 None if x["D"] is None else x["D"].index_select(0, ch), sel(x["z"]),
                 None if x["delta_bias"] is None else x["delta_bias"].index_select(0, ch))
        return ch, [oracle.to_f64(a) for a in args_]

    # calibrate on a small sample, then size the measured sample to about --cpu-seconds
    ch, a = sample(threads)
    c0 = time.perf_counter()
    oracle.scan(*a, softplus=x["softplus"], threads=threads)
    rate = threads * w.L / (time.perf_counter() - c0)  # channel-steps per second
    nch = int(max(threads, min(w.E, cpu_seconds * rate / w.L)))
    nch = max(threads, (nch // threads) * threads)
    ch, a = sample(nch)
    c0 = time.perf_counter()
    y_ref, last_ref = oracle.scan(*a, softplus=x["softplus"], threads=threads)
    cpu_s = time.perf_counter() - c0
    cpu = {"value": w.b * w.L * nch / cpu_s, "unit": "elem/s", "cores": threads, "kind": "oracle",
           "host": cpu_facts(), "seconds": round(cpu_s, 2),
           "threads_note": "threads = OMP_NUM_THREADS where set (the host share given to the job), else every core "
                           "the process may run on",
           "sample": f"{nch} of {w.E} channels (independent chains), full L={w.L}, b={w.b}; "
                     "fp64 sequential oracle, same inputs"}
    yg = oracle.to_f64(y.index_select(2, ch))
    lg = oracle.to_f64(last.index_select(1, ch))
    err = lambda g, r: float(np.max(np.abs(g - r) / (1 + np.abs(r))))
    parity = {"y_max_normalised_error": err(yg, y_ref), "last_state_max_normalised_error": err(lg, last_ref),
              "bound": 2e-2, "channels_checked": nch}
    log(f"[bench] cpu baseline {cpu['value']:.3e} elem/s on {threads} threads; parity {parity}")
    return cpu, parity


# ---------------------------------------------------------------------------------------------------
# summaries of rocprofv3 output (run on any host, after the GPU run): profiles/*.txt and *.json
# ---------------------------------------------------------------------------------------------------
def _split(name):
    """(symbol, symbol with template arguments) of a demangled kernel name: no namespace, no parameters."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    q = n[:cut]
    lt = q.find("<")
    sym = (q if lt < 0 else q[:lt]).split("::")[-1].strip()
    return sym, sym + (q[lt:] if lt >= 0 else "")


def _short(name):
    """Kernel symbol ("copy" for torch's copy kernels)."""
    sym = _split(name)[0]
    if sym not in LIB_KERNELS and "copy" in name:
        return "copy"
    return sym


def _template(name):
    return _split(name)[1]


def _csv_rows(d, suffix):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counters(d, only=None):
    """{(symbol, grid, wg): {counter: mean value per dispatch}} from a rocprofv3 --pmc run."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        sym = _short(r["Kernel_Name"])
        if only and sym not in only:
            continue
        key = (sym, int(r["Grid_Size"]), int(r["Workgroup_Size"]))
        per = acc.setdefault(key, {})
        per.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in per.items()} for k, per in acc.items()}


LIB_KERNELS = ("scan_main_kernel", "scan_chunk_agg_kernel", "chain_kernel", "scan_fused_kernel", "widen_rows_kernel",
               "fill_state_kernel", "state_update_kernel", "bwd_main_kernel", "bwd_chunk_maps_kernel",
               "bwd_chunk_agg_kernel", "bwd_rows_kernel", "bwd_reduce_bc_kernel", "bwd_reduce_chan_kernel",
               "bwd_fill_kernel", "ssd_state_kernel", "ssd_scan_kernel", "ssd_fill_kernel", "conv_fwd_kernel",
               "conv_fwd_vec_kernel", "conv_update_kernel", "conv_state_copy_kernel")


def summarize(run_root, prefix, title, commands, profiled_hash=None):
    """Write profiles/<prefix>_kernel_stats.txt, traffic_<prefix>.{txt,json} and sq_<prefix>.{txt,json} from the
    rocprofv3 runs under run_root: trace/ (--kernel-trace --stats), fetch/ and write/ (FETCH_SIZE, WRITE_SIZE),
    raw/ (TCC request counters), sq/ (SQ counters and VALUBusy), and copy_fetch/, copy_write/, copy_raw/ (the
    same counters on `bench.py --copy-calibration`).  Missing runs are skipped."""
    out_dir = os.path.join(ROOT, "profiles")
    sh = profiled_hash or source_hash()
    head = [f"# {title}", "# commands (from the repository root, on one MI355X; each --pmc set in a run of its own):"]
    head += [f"#   {c}" for c in commands]
    head += [f"# kernel source hash (bench.source_hash(): sha256[:16] of selective_state_space_35_amd/csrc/*.hip, *.h "
             f"but ssm_api.hip): {sh}", "#"]
    sub = lambda n: os.path.join(run_root, n)
    # kernel trace: per launch shape
    if os.path.isdir(sub("trace")):
        import statistics

        groups = {}
        for r in _csv_rows(sub("trace"), "kernel_trace.csv"):
            sym = _short(r["Kernel_Name"])
            if sym not in LIB_KERNELS:
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            groups.setdefault((_template(r["Kernel_Name"]), grid, wg, int(r["LDS_Block_Size"]),
                               int(r["VGPR_Count"])), []).append(us)
        lines = head + ["# per launch shape (grid and workgroup in threads, LDS in bytes); med_us is the steady "
                        "state, avg_us includes the first calls while the clocks ramp up",
                        f"# {'kernel':<78} {'grid':>9} {'wg':>5} {'lds':>7} {'vgpr':>4} {'calls':>5} {'avg_us':>9} "
                        f"{'med_us':>9} {'min_us':>9} {'max_us':>9}"]
        for (name, grid, wg, lds, vg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"  {name[:78]:<78} {grid:>9} {wg:>5} {lds:>7} {vg:>4} {len(v):>5} "
                         f"{sum(v) / len(v):>9.2f} {statistics.median(v):>9.2f} {min(v):>9.2f} {max(v):>9.2f}")
        with open(os.path.join(out_dir, f"{prefix}_kernel_stats.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # traffic
    if os.path.isdir(sub("fetch")) and os.path.isdir(sub("write")) and os.path.isdir(sub("copy_fetch")):
        fe, wr = _counters(sub("fetch"), LIB_KERNELS), _counters(sub("write"), LIB_KERNELS)
        cf, cw = _counters(sub("copy_fetch"), ("copy",)), _counters(sub("copy_write"), ("copy",))
        big = lambda d, c: max((v for k, v in d.items() if k[0] == "copy"), key=lambda v: v.get(c, 0))
        nbytes = 1 << 30
        rf = nbytes / (big(cf, "FETCH_SIZE")["FETCH_SIZE"] * 1024)
        wf = nbytes / (big(cw, "WRITE_SIZE")["WRITE_SIZE"] * 1024)
        doc = {"source_hash": sh, "title": title, "commands": commands,
               "copy_calibration": {"bytes": nbytes, "fetch_size_kib": big(cf, "FETCH_SIZE")["FETCH_SIZE"],
                                    "write_size_kib": big(cw, "WRITE_SIZE")["WRITE_SIZE"], "read_factor": rf,
                                    "write_factor": wf},
               "kernels": {}}
        if os.path.isdir(sub("copy_raw")):
            raw = big(_counters(sub("copy_raw"), ("copy",)), "TCC_EA0_RDREQ_sum")
            doc["copy_calibration"]["raw"] = raw
        raw_k = _counters(sub("raw"), LIB_KERNELS) if os.path.isdir(sub("raw")) else {}
        lines = head + [f"# copy calibration (1 GiB read + 1 GiB written): FETCH_SIZE "
                        f"{doc['copy_calibration']['fetch_size_kib']:.0f} KiB -> read factor {rf:.3f}; WRITE_SIZE "
                        f"{doc['copy_calibration']['write_size_kib']:.0f} KiB -> write factor {wf:.3f}"]
        if "raw" in doc["copy_calibration"]:
            r = doc["copy_calibration"]["raw"]
            lines.append(f"# copy raw TCC requests: TCC_EA0_RDREQ_sum {r.get('TCC_EA0_RDREQ_sum', 0):.0f}, "
                         f"TCC_EA0_RDREQ_32B_sum {r.get('TCC_EA0_RDREQ_32B_sum', 0):.0f}, TCC_BUBBLE_sum "
                         f"{r.get('TCC_BUBBLE_sum', 0):.0f} (1 GiB / 128 B = {nbytes // 128})")
        lines.append(f"# {'kernel':<24} {'grid':>9} {'wg':>5} {'FETCH_KiB':>12} {'WRITE_KiB':>12} {'read_GB':>9} "
                     f"{'write_GB':>9} {'RDREQ':>12} {'RDREQ_32B':>10} {'BUBBLE':>10}")
        for key in sorted(fe, key=lambda k: -fe[k].get("FETCH_SIZE", 0)):
            if key not in wr:
                continue
            rd = fe[key]["FETCH_SIZE"] * 1024 * rf
            wt = wr[key]["WRITE_SIZE"] * 1024 * wf
            rk = raw_k.get(key, {})
            rec = {"grid": key[1], "workgroup": key[2], "fetch_size_kib": fe[key]["FETCH_SIZE"],
                   "write_size_kib": wr[key]["WRITE_SIZE"], "read_bytes_per_launch": rd,
                   "write_bytes_per_launch": wt, "hbm_bytes_per_launch": rd + wt, "raw": rk}
            name = key[0] if key[0] not in doc["kernels"] else f"{key[0]}@{key[1]}"
            doc["kernels"][name] = rec
            lines.append(f"  {key[0]:<24} {key[1]:>9} {key[2]:>5} {fe[key]['FETCH_SIZE']:>12.0f} "
                         f"{wr[key]['WRITE_SIZE']:>12.0f} {rd / 1e9:>9.4f} {wt / 1e9:>9.4f} "
                         f"{rk.get('TCC_EA0_RDREQ_sum', float('nan')):>12.0f} "
                         f"{rk.get('TCC_EA0_RDREQ_32B_sum', float('nan')):>10.0f} "
                         f"{rk.get('TCC_BUBBLE_sum', float('nan')):>10.0f}")
        with open(os.path.join(out_dir, f"traffic_{prefix}.json"), "w") as f:
            json.dump(doc, f, indent=1)
        with open(os.path.join(out_dir, f"traffic_{prefix}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # issue rates of the calibration kernels
    if os.path.exists(sub("alu.json")):
        with open(sub("alu.json")) as f:
            alu = json.loads(f.read().strip().splitlines()[-1])
        lines = [f"# issue rates of single VALU instruction kinds on one MI355X ({alu['simds']} SIMDs, "
                 f"{alu['clock_GHz_assumed']} GHz assumed)",
                 "# command (from the repository root):", "#   python3 bench.py --alu-calibration",
                 "# kernels: selective_state_space_35_amd/calib/ssm_calib.hip, built by build_calib() with the "
                 "library's flags:", f"#   {alu['flags']}",
                 "# each kind runs 8 independent chains per lane over 256 CUs x waves_per_simd x 4 waves",
                 f"# {'kind':<46} {'waves/SIMD':>10} {'ms':>8} {'VALU lane-op/s':>15} {'trans lane-op/s':>15} "
                 f"{'cyc/inst':>9} {'cyc/group':>9}"]
        for k in alu["kinds"]:
            lines.append(f"  {k['what']:<46} {k['waves_per_simd']:>10} {k['ms']:>8.3f} "
                         f"{k['valu_lane_ops_per_s']:>15.4g} {k['trans_lane_ops_per_s']:>15.4g} "
                         f"{k['cycles_per_wave_inst']:>9.3f} {k.get('cycles_per_group', float('nan')):>9.3f}")
        fma = [k for k in alu["kinds"] if k["kind"] == 0 and k["waves_per_simd"] == 8][0]["cycles_per_wave_inst"]
        mix4 = [k for k in alu["kinds"] if k["kind"] == 2 and k["waves_per_simd"] == 8][0]["cycles_per_group"]
        mix2 = [k for k in alu["kinds"] if k["kind"] == 3][0]["cycles_per_group"]
        lines += ["#", f"# reading: an fp32 FMA issues in {fma:.2f} cycles per wave64 instruction (4 at the "
                  f"nominal 16 lanes/clock/SIMD: {4 / fma:.1%} of 3.93e13 lane-op/s); in these probes an exp next "
                  f"to 4 FMAs adds {mix4 - 4 * fma:.2f} cycles and next to 2 FMAs {mix2 - 2 * fma:.2f} "
                  f"({(mix4 - 4 * fma) / fma:.2f} / {(mix2 - 2 * fma) / fma:.2f} FMA slots), an upper bound: the "
                  "scan kernels issue their mix (a fifth transcendental) at 4.5 cycles per instruction "
                  "(sq_scan_long.txt), so the roofline counts every VALU instruction, a transcendental included, "
                  "as one slot against 256 x 4 x 16 x 2.4e9 = 3.93e13 slot/s"]
        with open(os.path.join(out_dir, "alu_issue_rates.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")

    # SQ counters and VALU busy
    if os.path.isdir(sub("sq")):
        sq = _counters(sub("sq"), LIB_KERNELS)
        for extra in ("sq2", "sq3"):
            if os.path.isdir(sub(extra)):
                for k, v in _counters(sub(extra), LIB_KERNELS).items():
                    sq.setdefault(k, {}).update(v)
        doc = {"source_hash": sh, "title": title, "commands": commands, "kernels": {}}
        lines = head + ["# per dispatch (mean over the run's dispatches of that launch shape); VALUBusy = 100 x "
                        "SQ_ACTIVE_INST_VALU / CU_NUM / GRBM_GUI_ACTIVE (rocprofv3's derived counter)",
                        f"# {'kernel':<24} {'grid':>9} {'counter':<26} {'value':>14}"]
        for key in sorted(sq, key=lambda k: -sq[k].get("SQ_INSTS_VALU", 0)):
            name = key[0] if key[0] not in doc["kernels"] else f"{key[0]}@{key[1]}"
            doc["kernels"][name] = dict(sq[key], grid=key[1], workgroup=key[2])
            for c in sorted(sq[key]):
                lines.append(f"  {key[0]:<24} {key[1]:>9} {c:<26} {sq[key][c]:>14.4g}")
        with open(os.path.join(out_dir, f"sq_{prefix}.json"), "w") as f:
            json.dump(doc, f, indent=1)
        with open(os.path.join(out_dir, f"sq_{prefix}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")


ALU_KINDS = {0: "v_fma_f32", 1: "v_exp_f32", 2: "4 v_fma_f32 + 1 v_exp_f32", 3: "2 v_fma_f32 + 1 v_exp_f32",
             4: "v_mul_f32 with a DPP quad-broadcast operand", 5: "v_add_f32"}


def alu_calibration(iters=20000, reps=3):
    """Issue rates of the instruction kinds the scan kernels are made of, on this GPU, from the
    calibration kernels of libssm_calib.so (built with the library's flags).  Each kind runs on
    256 CUs x waves_per_simd x 4 waves; rates are lane-operations per second and the implied cycles
    per wave64 instruction at the 2.4 GHz peak engine clock."""
    import ctypes

    from selective_state_space_35_amd import build as lib_build

    lib = ctypes.CDLL(lib_build.CALIB_LIB)
    lib.ssm_calib_alu.restype = ctypes.c_int
    d = ctypes.c_double
    lib.ssm_calib_alu.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(d)] * 3
    flags = " ".join(f for f in lib_build.COMMON if not f.startswith("-I"))
    out = {"clock_GHz_assumed": 2.4, "simds": 1024, "flags": flags, "kinds": []}
    for kind, wps in [(0, 1), (0, 2), (0, 4), (0, 8), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (2, 4), (1, 4)]:
        ms, valu, trans = d(), d(), d()
        rc = lib.ssm_calib_alu(kind, 256 * wps, iters, reps, ctypes.byref(ms), ctypes.byref(valu), ctypes.byref(trans))
        if rc != 0:
            raise RuntimeError(f"ssm_calib_alu({kind}) returned {rc}")
        sec = ms.value * 1e-3
        cyc = 2.4e9 * sec * 1024  # SIMD-cycles at the peak clock
        insts = (valu.value + trans.value) / 64
        rec = {"kind": kind, "what": ALU_KINDS[kind], "waves_per_simd": wps, "ms": round(ms.value, 3),
               "valu_lane_ops_per_s": valu.value / sec, "trans_lane_ops_per_s": trans.value / sec,
               "cycles_per_wave_inst": round(cyc / insts, 3)}
        if valu.value and trans.value:  # mixed: cycles per (one exp + its FMAs) group per wave
            rec["cycles_per_group"] = round(cyc / (trans.value / 64), 3)
        out["kinds"].append(rec)
        log(f"[alu] {rec}")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the CPU baseline sample")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration scan timings")
    ap.add_argument("--alu-calibration", action="store_true",
                    help="only time the issue-rate calibration kernels (libssm_calib.so) and print their rates")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--workload", default="long", choices=["long", "mid", "block", "tiny", "long_e640"],
                    help="the scan timed as the step (default: the long sequence, the headline; the others for "
                         "profiling their kernels alone)")
    ap.add_argument("--summarize", metavar="RUN_ROOT",
                    help="no GPU: write profiles/ summaries from the rocprofv3 runs under RUN_ROOT")
    ap.add_argument("--prefix", default="scan_long", help="--summarize: name of the summaries")
    ap.add_argument("--title", default="", help="--summarize: first line of the summaries")
    ap.add_argument("--commands", default="", help="--summarize: file with the commands that made the runs")
    ap.add_argument("--source-hash", default="", help="--summarize: bench.source_hash() of the profiled tree")
    ap.add_argument("--print-source-hash", action="store_true", help="print bench.source_hash() and exit")
    args = ap.parse_args()

    if args.print_source_hash:
        print(source_hash())
        return
    if args.summarize:
        cmds = []
        if args.commands:
            with open(args.commands) as f:
                cmds = [ln.rstrip("\n") for ln in f if ln.strip()]
        summarize(args.summarize, args.prefix, args.title, cmds, args.source_hash or None)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the scan "
              "shards over batch and channels with no communication, so there is no multi-GPU path to time.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import selective_state_space_35_amd as ssm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.alu_calibration:
        print(json.dumps(alu_calibration()), flush=True)
        return

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}))
        return

    w = {"long": workloads.LONG, "mid": workloads.MID, "block": workloads.BLOCK, "tiny": workloads.TINY,
         "long_e640": workloads.LONG_E640}[args.workload]
    log(f"[bench] generating {w.description} (seed {args.seed}) on {torch.cuda.get_device_name(dev)}")
    x = workloads.make_scan_inputs(w, seed=args.seed, device=dev, backend="torch")
    y = torch.empty_like(x["u"])
    last = torch.empty(w.b, w.E, w.N, dtype=torch.float32, device=dev)
    scan_path, chunk_len, n_chunks = ssm.ssm_scan_plan(w.b, w.L, w.E, w.N, w.dtype)

    def step():
        ssm.ssm_scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                         x["softplus"], y=y, last_state=last)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ssm.ssm_profile_read()  # drop anything recorded before the timed region
    ssm.ssm_profile_enable(True)
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ssm.ssm_profile_enable(False)
    per_kernel = ssm.ssm_profile_read()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    elems = w.b * w.L * w.E
    value = elems / (ms_per_step * 1e-3)
    s = 2 if w.dtype == "bf16" else 4
    algo = scan_bytes(w.b, w.L, w.E, w.N, s, gate=w.z is not None)
    path_gbps = algo / (ms_per_step * 1e-3) / 1e9
    kernels = {k: {"avg_us": round(1e3 * v[0] / v[1], 2), "launches": v[1]} for k, v in per_kernel.items() if v[1]}
    # the dominant kernel of the call: the single-pass scan, or the main pass of the chunked form
    main_name = max((k for k in per_kernel if per_kernel[k][1]), key=lambda k: per_kernel[k][0])
    main_ms, main_n = per_kernel[main_name]
    main_avg_s = main_ms / max(main_n, 1) * 1e-3
    achieved = algo / main_avg_s / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step, {value:.4e} elem/s, path {path_gbps:.1f} GB/s; "
        f"kernels {kernels}")

    # ALU view (the bound that holds): algorithmic VALU lane-slots of one pass over the scan
    slots = scan_slots(w.b, w.L, w.E, w.N, softplus=w.softplus, gate=w.z is not None, has_d=w.D is not None,
                       has_bias=w.delta_bias is not None, bf16=(w.dtype == "bf16"))
    main_tslots = slots / main_avg_s / 1e12
    path_tslots = slots / (ms_per_step * 1e-3) / 1e12
    alu = {"slots_per_step": slots, "path_Tslot_per_s": path_tslots,
           "path_frac": path_tslots * 1e12 / VALU_SLOT_PEAK,
           "note": f"one slot = one non-packed fp32 VALU lane-op issue, a transcendental takes {TRANS_SLOTS} "
                   "(profiles/alu_issue_rates.txt); peak 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.  The chunked "
                   "form runs a second (aggregate) pass over all but the last chunk; its slots are not "
                   "algorithmic"}
    # committed counter summaries of this workload, used when taken on the current sources
    tr_doc, tr_note = load_profile(f"traffic_scan_{w.name}")
    sq_doc, sq_note = load_profile(f"sq_scan_{w.name}")
    main_sym = KIND_SYMBOL.get(main_name, main_name)
    traffic = None
    if tr_doc and main_sym in tr_doc["kernels"]:
        traffic = tr_doc["kernels"][main_sym]["hbm_bytes_per_launch"]
    valu_busy = ({k: v.get("VALUBusy") for k, v in sq_doc["kernels"].items()} if sq_doc else None)
    roofline = {
        "bound": "alu", "kernel": main_sym, "achieved": main_tslots, "peak": VALU_SLOT_PEAK / 1e12,
        "unit": "Tslot/s", "frac": main_tslots * 1e12 / VALU_SLOT_PEAK, "traffic": traffic,
        "traffic_note": tr_note or ("L2-to-fabric bytes per launch: FETCH_SIZE and WRITE_SIZE from two rocprofv3 "
                                    "--pmc runs, each scaled by the same counter on a plain 1 GiB copy "
                                    "(profiles/traffic_scan_long.txt)"),
        "algorithmic_bytes": algo, "algorithmic_slots": slots, "kernel_avg_us": round(main_avg_s * 1e6, 2),
        "hbm": {"kernel_GBps": achieved, "kernel_frac": achieved / HBM_PEAK_GBPS,
                "call_GBps": path_gbps, "call_frac": path_gbps / HBM_PEAK_GBPS, "peak_GBps": HBM_PEAK_GBPS},
        "valu_busy_pct": valu_busy, "valu_busy_note": sq_note or "rocprofv3 VALUBusy per kernel "
                                                                 "(profiles/sq_scan_long.txt)",
        "slot_model": f"one slot = one non-packed fp32 VALU lane-op; a transcendental = {TRANS_SLOTS} slots, "
                      "measured by the calibration kernels (profiles/alu_issue_rates.txt)"}

    # state update (generation): 128 successive single-token updates, state carried in HBM
    update = None if args.no_decode else measure_decode(ssm, torch, workloads, dev, stream, args.seed)

    # backward of the scan on the same workload (gradients of every input, states recomputed)
    bwd = None if args.no_bwd else measure_backward(ssm, torch, dev, stream, x, w, args.steps, args.seed)

    # the scan with a scalar transition per head, in chunks of MFMA matrix products
    ssd = None if args.no_ssd else measure_ssd(ssm, torch, workloads, dev, stream, args.seed,
                                               cpu=not args.no_cpu_baseline)

    # causal convolution in front of the scan (long workload) and its generation-time token step
    conv = None if args.no_conv else measure_conv(ssm, torch, workloads, dev, args.seed)

    # CPU baseline: the oracle on a bounded channel sample of the same inputs
    cpu, parity = (None, None) if args.no_cpu_baseline else measure_cpu_baseline(
        torch, dev, x, w, y, last, args.cpu_seconds)

    # the other scan configurations, and the long workload's one-GPU share under channel
    # sharding: every call timed on its own (event pair on the launch stream), median and min
    configs = None
    if not args.no_configs:
        configs = scan_configs(ssm, workloads, torch, dev, stream, args.seed,
                               cpu=not args.no_cpu_baseline)
        log(f"[bench] configs {configs}")

    out = {
        "metric": "selective-scan B·L·E elems/s and achieved HBM GB/s (% of MI355X peak)",
        "value": value,
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "dtype_note": "bf16 inputs and outputs; state, exponentials and accumulation in fp32",
        "config": {"workload": "long-sequence selective scan b1 L65536 E5120 N16, bf16 I/O, fp32 state, "
                               "softplus step, silu gate, D skip",
                   "b": w.b, "L": w.L, "E": w.E, "N": w.N, "io_dtype": w.dtype,
                   "scan_form": scan_path, "chunk_len": chunk_len, "n_chunks": n_chunks,
                   "parallelism": "single GPU"},
        "hbm_GBps": path_gbps,
        "hbm_frac": path_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": algo,
        "roofline": roofline,
        "kernels": kernels,
        "alu": alu,
        "state_update": update,
        "conv": conv,
        "backward": bwd,
        "ssd": ssd,
        "cpu_baseline": cpu,
        "parity": parity,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
