#!/usr/bin/env python3
"""Benchmark of the selective state-space scan on one MI355X.

One step = one forward scan of the Mamba-2.8B layer shape
(batch 4, L 4096, D 5120, N 16; bf16 x/delta/z/B/C/y, fp32 A/D and state)
on seeded synthetic inputs already resident in HBM: both launches of the
chunked scan (chunk 0's main pass beside the pre-pass of the middle chunks,
the composition of the chunk maps, the main pass of the other chunks).
Prints one JSON line with whole-job throughput in B*L*D*N elements/s, the
roofline of the dominant kernel (the main pass), the other scan
configurations (tiny fp32, Mamba-130M layer, the 262144-step single
sequence), the recurrent decode sweep (256 sequences x 64 layers of D 5120,
N 16), the NEXT-row paths and the fp64 CPU oracle timed on a bounded sample
on this host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

The GPU's clock rises over the first ~30 ms of sustained work; an untimed
clock ramp (``--ramp-seconds``, default 0.5 s of the same step) runs before
the warm-up steps and is reported in the line (``clock_ramp``).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
# ALU roofline of the scan element.  Per element (b, t, d, n) the main pass
# must issue 6 fp32 VALU operations (delta*A, B*x, *1/A, the input-term fma,
# the update fma, the readout fma) and one transcendental (exp2).  Unit
# counts: 256 CUs x 4 SIMDs at 2.4 GHz; a SIMD issues a non-packed fp32
# wave64 instruction in 4 cycles (16 lanes per clock) and an exp2 in 8 (8
# lanes per clock), as the SQ counters of the scan kernels show
# (SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU; packed fp32 is not used).  The
# minimal mix then costs 6 x 4 + 8 = 32 cycles per 64 elements.  The
# published 157.3 TFLOP/s fp32 vector figure counts 32 lanes per clock
# (packed fp32, or two VALU instructions issued together): the same mix at
# that rate costs 6 x 2 + 8 = 20 cycles, reported beside it.
ALU_OPS_PER_ELEMENT = 7
SIMDS, CLOCK_HZ = 256 * 4, 2.4e9
FP32_CYCLES, TRANS_CYCLES = 4, 8
ALU_PEAK_ELEMS = SIMDS * CLOCK_HZ * 64 / (6 * FP32_CYCLES + TRANS_CYCLES)
ALU_PEAK_ELEMS_DUAL = SIMDS * CLOCK_HZ * 64 / (6 * FP32_CYCLES / 2 + TRANS_CYCLES)
TILE_STEPS = 16  # chunks of the chunked scan start on a multiple of this many steps
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_main_mamba2p8b_b4_l4096_d5120_traffic.md")


# Sources that define the chunked scan's kernels and plan (the committed
# traffic figure of its main pass is tied to these).
SCAN_SOURCES = ["selective_state_space_44_amd/csrc/ssm_scan.hip",
                "selective_state_space_44_amd/csrc/ssm_device.h",
                "selective_state_space_44_amd/csrc/ssm_launch.h",
                "selective_state_space_44_amd/csrc/ssm_abi.cpp", "include/ssm.h"]


def source_hash(files=None) -> str:
    """Hash of library sources with /* */ and // comments and blank lines
    removed (a comment edit does not change a kernel; any code edit does):
    every source by default, or the given files (paths from the repo root)."""
    h = hashlib.sha256()
    if files is None:
        files = sorted(glob.glob(os.path.join(ROOT, "selective_state_space_44_amd", "csrc", "*")))
        files += [os.path.join(ROOT, "include", "ssm.h")]
    else:
        files = [os.path.join(ROOT, f) for f in files]
    for f in files:
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the main kernel, from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, when it was taken on the current scan
    sources (its ``source_hash`` line matches source_hash(SCAN_SOURCES));
    None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    h = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    b = re.search(r"^hbm_bytes_per_launch:\s*(\d+)", text, re.M)
    if not h or not b or h.group(1) != source_hash(SCAN_SOURCES):
        return None
    return int(b.group(1))


def host_cpus():
    """CPUs this job may use: OMP_NUM_THREADS when the host sets it (a GPU
    box allots a share of its cores per GPU this way), else the affinity
    mask; plus what the machine shows and its model name."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    allotted = visible
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        allotted = min(visible, int(env))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return allotted, visible, model


def cpu_baseline(inp, w, target_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    the first ``nb`` batch rows, the first ``nch`` channels of each, over the
    full sequence, on every CPU the job is allotted."""
    import torch
    import oracle

    nthreads, visible, model = host_cpus()

    def take(nb, nch):
        idx = torch.arange(nch, device=inp["x"].device)
        f64 = lambda t: t.detach().to("cpu").to(torch.float64).numpy()
        sl = lambda t: f64(t[:nb].index_select(2, idx))
        return (sl(inp["x"]), sl(inp["delta"]), f64(inp["A"].index_select(0, idx)),
                f64(inp["B"][:nb]), f64(inp["C"][:nb]), f64(inp["D"].index_select(0, idx)),
                sl(inp["z"]))

    def run(nb, nch):
        args = take(nb, nch)
        t0 = time.perf_counter()
        oracle.scan(*args, nthreads=nthreads)
        return time.perf_counter() - t0

    # calibrate on a small sample, then size the timed sample to ~target_s
    probe = min(w.dim, 8 * nthreads)
    per_chan = run(1, probe) / probe
    want = max(1, int(target_s / max(per_chan, 1e-9)))
    if want >= w.dim:
        nb, nch = min(w.batch, max(1, want // w.dim)), w.dim
    else:
        nb, nch = 1, max(probe, want // nthreads * nthreads)
    dt = run(nb, nch)
    elems = nb * w.seqlen * nch * w.dstate
    return {"value": elems / dt, "unit": "elements/s", "cores": nthreads, "kind": "oracle",
            "cpus_visible": visible, "cpu_model": model,
            "sample": f"{nb} of {w.batch} batch rows x {nch} of {w.dim} channels, full "
                      f"L={w.seqlen}, N={w.dstate}: {elems:.3e} elements in {dt:.1f} s "
                      f"(fp64 C loop, gcc -O2, OpenMP over channels, {nthreads} threads)"}


def percentiles(ms):
    """p10, median and p90 of per-step times in ms (nearest rank)."""
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def chunk_rows(seqlen: int, nchunks: int) -> int:
    """Steps of each chunk (the last may be shorter) of a K-chunk plan."""
    if nchunks <= 1:
        return seqlen
    per = -(-seqlen // nchunks)
    return -(-per // TILE_STEPS) * TILE_STEPS


def scan_bytes(w, rows: int) -> int:
    """Algorithmic bytes of a scan over `rows` steps of every batch row of w:
    x, delta, z in and y out, B and C in, A and D once."""
    return (w.batch * rows * (4 * w.dim + 2 * w.dstate) * w.io_bytes
            + 4 * w.dim * w.dstate + 4 * w.dim)


def clock_ramp(step, seconds: float) -> int:
    """Untimed steps until `seconds` of wall time have passed (synchronising
    every few steps, so the GPU is busy throughout)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def bench_scan(steps: int, warmup: int, ramp_s: float):
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.MAMBA_2P8B
    dev = "cuda:0"
    # two input sets, alternated, so no step reads what the previous left in
    # the 256 MB Infinity Cache (one set is ~0.67 GB anyway)
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x"]) for s in sets]
    G, K, ph = ssm.scan_plan(w.batch, w.seqlen, w.dim, with_phase=True)
    base = ph & 4  # the plan's schedule: 0 two-launch, 4 three-pass
    nws = ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim, nchunks=K)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        s, y = sets[i % 2], outs[i % 2]
        args = (s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], None)
        kw = dict(waves_per_group=G, nchunks=K, out=y, workspace=ws)
        ssm.scan_fwd(*args, phase=base | 1, **kw)
        if ev is not None:
            ev[0].record()
        ssm.scan_fwd(*args, phase=base | 2, **kw)
        if ev is not None:
            ev[1].record()

    ramp_steps = clock_ramp(step, ramp_s) if ramp_s > 0 else 0
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # two events per step on the launch stream: between the launch groups and
    # after the main pass; a step runs from the previous step's end event (an
    # event record between kernels leaves a gap of several µs in the stream,
    # so none is added that the breakdown does not need)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_all[0].record()
    for i in range(steps):
        step(i, evs[i])
    t_all[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    starts = [t_all[0]] + [e[1] for e in evs[:-1]]
    ev_step = [a.elapsed_time(e[1]) for a, e in zip(starts, evs)]
    ev_main = [e[0].elapsed_time(e[1]) for e in evs]
    ev_first = [a.elapsed_time(e[0]) for a, e in zip(starts, evs)]
    return dict(w=w, G=G, K=K, three_pass=bool(base), wall_s=wall, step_ms=t_all[0].elapsed_time(t_all[1]) / steps,
                main_ms=sum(ev_main) / steps, first_ms=sum(ev_first) / steps, inp=sets[0],
                step_pct=percentiles(ev_step), main_pct=percentiles(ev_main),
                ramp_steps=ramp_steps)


def sweep_plans(spec: str, steps: int, ramp_s: float, wname: str = ""):
    """Chunk plans "GxK,GxK,..." of a scan workload (the Mamba-2.8B layer by
    default) under both schedules (two-launch: phases 1 and 2; three-pass:
    phases 5 and 6): median ms of each launch group and of the step over
    `steps` timed steps, with input sets rotated (two, or six for the
    Mamba-130M layer, so no step reads what an earlier one left in the 256 MB
    Infinity Cache)."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.WORKLOADS[wname] if wname else W.MAMBA_2P8B
    nsets = 6 if w.algorithmic_bytes() < 256 << 20 else 2
    dev = "cuda:0"
    plans = [tuple(int(v) for v in p.split("x")) for p in spec.split(",") if p]
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(nsets)]
    outs = [torch.empty_like(s["x"]) for s in sets]
    kmax = max(k for _, k in plans)
    ws = torch.empty(ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim, dtype=w.io_dtype,
                                              nchunks=kmax) + 256,
                     dtype=torch.uint8, device=dev)

    def run(G, K, i, phase):
        s = sets[i % nsets]
        ssm.scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], None,
                     waves_per_group=G, nchunks=K, out=outs[i % nsets], workspace=ws, phase=phase)

    G0, K0, P0 = ssm.scan_plan(w.batch, w.seqlen, w.dim, dtype=w.io_dtype, with_phase=True)
    ramp = clock_ramp(lambda i: run(G0, K0, i, P0), ramp_s) if ramp_s > 0 else 0
    med = lambda v: sorted(v)[len(v) // 2]
    rows = []
    for G, K in plans:
        for base, name in ((0, "two-launch"), (4, "three-pass")):
            for i in range(10):
                run(G, K, i, base | 3)
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
            for i in range(steps):
                ev[i][0].record()
                run(G, K, i, base | 1)
                ev[i][1].record()
                run(G, K, i, base | 2)
                ev[i][2].record()
            torch.cuda.synchronize()
            rows.append({"waves_per_group": G, "nchunks": K, "schedule": name,
                         "first_ms": med([e[0].elapsed_time(e[1]) for e in ev]),
                         "main_ms": med([e[1].elapsed_time(e[2]) for e in ev]),
                         "step_ms": med([e[0].elapsed_time(e[2]) for e in ev])})
    return {"workload": w.name, "steps": steps, "clock_ramp_steps": ramp,
            "auto_plan": [G0, K0, "three-pass" if P0 & 4 else "two-launch"],
            "plans": rows}


def bench_config(w, sets_n: int, steps: int, warmup: int):
    """One scan configuration in its automatic plan: per-step times over
    `sets_n` rotated input sets (so that no step reads what an earlier one
    left in the 256 MB Infinity Cache)."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    dev = "cuda:0"
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(sets_n)]
    outs = [torch.empty_like(s["x"]) for s in sets]
    G, K, ph = ssm.scan_plan(w.batch, w.seqlen, w.dim, dtype=w.io_dtype, with_phase=True)
    nws = ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim, dtype=w.io_dtype, nchunks=K)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % sets_n]
        ssm.scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], None,
                     waves_per_group=G, nchunks=K, out=outs[i % sets_n], workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    mean = sum(ms) / len(ms)
    nbytes = w.algorithmic_bytes()
    res = {"batch": w.batch, "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
           "io_dtype": "f32" if w.io_dtype == torch.float32 else "bf16",
           "plan": {"waves_per_group": G, "nchunks": K,
                    "schedule": "three-pass" if ph & 4 else "two-launch"}, "steps": steps,
           "input_sets": sets_n, "rotated_bytes": nbytes * sets_n,
           "ms_per_step": mean, "ms_percentiles": percentiles(ms),
           "value": w.elements / (mean * 1e-3), "unit": "elements/s",
           "hbm": {"algorithmic_bytes": nbytes, "achieved": nbytes / (mean * 1e-3) / 1e9,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": nbytes / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    del sets, outs, ws
    torch.cuda.empty_cache()
    return res


def bench_fused(steps: int, warmup: int):
    """The scan with its prologue fused (causal depthwise conv1d of width 4 +
    SiLU, softplus(delta_raw + bias)) at the same shape, automatic plan."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.MAMBA_2P8B
    dev = "cuda:0"
    sets = [W.make_fused_inputs(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x_raw"]) for s in sets]
    nws = ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def step(i):
        f = sets[i % 2]
        ssm.scan_fwd_fused(f["x_raw"], f["conv_w"], f["conv_b"], f["delta_raw"],
                           f["delta_bias"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                           conv_silu=True, out=outs[i % 2], workspace=ws)

    clock_ramp(step, 0.2)  # untimed, as for the headline scan
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": w.name + "_fused_conv4_silu_softplus", "ms_per_step": ms,
            "value": w.elements / (ms * 1e-3), "unit": "elements/s",
            "hbm_algorithmic_GBps": w.algorithmic_bytes() / (ms * 1e-3) / 1e9}


def bench_variants(steps: int, warmup: int):
    """The scan variants at the same shape and plan: A per channel (one value
    shared by a channel's states) and the Euler rule Bbar = delta*B."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.MAMBA_2P8B
    dev = "cuda:0"
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(2)]
    a_ch = [W.make_channel_A(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x"]) for s in sets]
    nws = ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    res = {}
    for tag, per_channel, disc in (("A_per_channel", True, "zoh"), ("euler", False, "euler"),
                                   ("A_per_channel_euler", True, "euler")):
        def step(i):
            f = sets[i % 2]
            A = a_ch[i % 2] if per_channel else f["A"]
            ssm.scan_fwd(f["x"], f["delta"], A, f["B"], f["C"], f["D"], f["z"], None,
                         out=outs[i % 2], workspace=ws, discretization=disc)

        clock_ramp(step, 0.2)  # untimed, as for the headline scan
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[tag] = {"ms_per_step": ms, "value": w.elements / (ms * 1e-3), "unit": "elements/s"}
    return {"workload": w.name, **res}


def bench_ssd_forward(steps: int, warmup: int):
    """The masked-matrix forward alone at the Mamba-2-like layer (two input
    sets alternated), for profiler runs."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.SSD_2P7B
    dev = "cuda:0"
    sets = [W.make_ssd_inputs(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x"]) for s in sets]

    def step(i):
        f = sets[i % 2]
        ssm.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                     out=outs[i % 2])

    clock_ramp(step, 0.3)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": w.name, "ms_per_step": ms, "value": w.elements / (ms * 1e-3),
            "unit": "elements/s"}


def bench_ssd_backward(steps: int, warmup: int):
    """The masked-matrix backward alone at the Mamba-2-like layer (one input
    set, one upstream dy), for profiler runs."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.SSD_2P7B
    dev = "cuda:0"
    f = W.make_ssd_inputs(w, device=dev, layer=0)
    P, N = w.headdim, w.dstate
    heads = w.dim // P
    g = torch.Generator(device=dev).manual_seed(19)
    dy = torch.randn(f["x"].shape, generator=g, device=dev).to(f["x"].dtype)
    nws = ssm.load_library().ssm_ssd_bwd_workspace_bytes(w.batch, w.seqlen, heads, P, N,
                                                           1 if w.io_dtype == torch.bfloat16 else 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step(i):
        ssm.ssd_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                    dy=dy, workspace=ws)

    clock_ramp(step, 0.2)  # untimed, as for the headline scan
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": w.name, "ms_per_step": ms, "workspace_bytes": nws}


def bench_ssd(steps: int, warmup: int):
    """The scan with step and decay shared per head, in its masked-matrix form
    on the matrix cores (``ssm_ssd_fwd``), at a Mamba-2-like layer: batch 4,
    L 4096, 80 heads of 64 channels, 128 states, bf16.  Two input sets are
    alternated (each ~0.5 GB, twice the Infinity Cache).  Also times the
    per-channel recurrence kernels on the same problem (dt repeated over each
    head's channels, A per channel)."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.SSD_2P7B
    dev = "cuda:0"
    sets = [W.make_ssd_inputs(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x"]) for s in sets]

    def step(i):
        f = sets[i % 2]
        ssm.ssd_scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                     out=outs[i % 2])

    clock_ramp(step, 0.2)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    # matrix-core work of the masked-matrix form at the kernel's 32-step chunks:
    # per (batch row, chunk) the lower triangle of C B^T (Q(Q+1)/2 N, shared by
    # the heads), per (batch row, head, chunk) that of P x (Q(Q+1)/2 P), C h
    # (Q N P) and the state update (Q N P) multiply-adds
    Q, P, N = 32, w.headdim, w.dstate
    heads = w.dim // P
    chunks = (w.seqlen + Q - 1) // Q
    flops = 2 * w.batch * chunks * (Q * (Q + 1) // 2 * N
                                    + heads * (Q * (Q + 1) // 2 * P + 2 * Q * N * P))
    nbytes = w.algorithmic_bytes()

    # the same problem on the per-channel recurrence kernels (one input set)
    f = sets[0]
    delta = f["dt"].repeat_interleave(P, dim=2).contiguous()
    a_ch = f["A"].repeat_interleave(P).contiguous()
    y2 = torch.empty_like(f["x"])
    rec_steps = max(3, steps // 10)
    ssm.scan_fwd(f["x"], delta, a_ch, f["B"], f["C"], f["D"], f["z"], None, out=y2)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(rec_steps):
        ssm.scan_fwd(f["x"], delta, a_ch, f["B"], f["C"], f["D"], f["z"], None, out=y2)
    e1.record()
    torch.cuda.synchronize()
    rec_ms = e0.elapsed_time(e1) / rec_steps
    del delta, a_ch, y2

    # its backward (ssm_ssd_bwd: the masked-matrix backward, chunk-parallel)
    g = torch.Generator(device=dev).manual_seed(19)
    dy = torch.randn(f["x"].shape, generator=g, device=dev).to(f["x"].dtype)
    nws = ssm.load_library().ssm_ssd_bwd_workspace_bytes(w.batch, w.seqlen, heads, P, N,
                                                           1 if w.io_dtype == torch.bfloat16 else 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    bwd = lambda: ssm.ssd_bwd(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                              dy=dy, workspace=ws)
    bwd()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(rec_steps):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / rec_steps
    del ws, dy

    # one long sequence (1 x 16384, same layer): the automatic sequence segments
    # against one block per (half head, batch row)
    q = W.make_ssd_inputs(w, device=dev, batch=1, seqlen=16384, layer=2)
    yq = torch.empty_like(q["x"])
    single = {}
    for tag, ns in (("segments_auto", 0), ("unsplit", 1)):
        nb = ssm.load_library().ssm_ssd_fwd_workspace_bytes(1, 16384, heads, P, N, ns)
        wsq = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        run = lambda: ssm.ssd_scan(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["z"], None,
                                   out=yq, nsplit=ns, workspace=wsq)
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(rec_steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        single[tag + "_ms"] = e0.elapsed_time(e1) / rec_steps
    del q, yq, sets, outs
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms_per_step": ms, "value": w.elements / (ms * 1e-3),
            "unit": "elements/s",
            "mfma": {"algorithmic_flop": flops, "achieved": flops / (ms * 1e-3) / 1e12,
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
            "hbm": {"algorithmic_bytes": nbytes, "achieved": nbytes / (ms * 1e-3) / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "recurrence_ms_per_step": rec_ms, "speedup_vs_recurrence": rec_ms / ms,
            "backward_ms_per_step": bwd_ms, "backward_time_vs_forward": bwd_ms / ms,
            "single_sequence_1x16384": single}


def bench_backward(steps: int, warmup: int):
    """Backward of the scan at the same shape: all input gradients for an
    upstream dy (states recomputed, nothing kept from a forward call)."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.MAMBA_2P8B
    dev = "cuda:0"
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(2)]
    g = torch.Generator(device=dev).manual_seed(17)
    dys = [torch.randn(s["x"].shape, generator=g, device=dev).to(s["x"].dtype) for s in sets]
    nws = ssm.scan_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, dtype=w.io_dtype)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def step(i):
        f = sets[i % 2]
        ssm.scan_bwd(f["x"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], None,
                     dy=dys[i % 2], workspace=ws)

    clock_ramp(step, 0.2)  # untimed, as for the headline scan
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del sets, dys, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms_per_step": ms, "value": w.elements / (ms * 1e-3),
            "unit": "elements/s", "workspace_bytes": nws}


def bench_decode(sweeps: int):
    """64 layers stepped back to back, each with its own state, inputs and
    parameters (5.4 GB of state, far beyond the 256 MB cache).  HIP events
    bracket whole sweeps only: per-launch event pairs would add their own
    overhead to every 30 us launch."""
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.DECODE_64L
    dev = "cuda:0"
    layers = [W.make_inputs(w, device=dev, layer=l) for l in range(w.layers)]
    ys = [torch.empty_like(l["x"]) for l in layers]

    def sweep():
        for i, l in enumerate(layers):
            ssm.decode_step(l["h"], l["x"], l["delta"], l["A"], l["B"], l["C"], l["D"], l["z"],
                            out=ys[i])

    clock_ramp(lambda i: sweep(), 0.3)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(sweeps)]
    t0 = time.perf_counter()
    for r in range(sweeps):
        evs[r][0].record()
        sweep()
        evs[r][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sweep_list = [e[0].elapsed_time(e[1]) for e in evs]
    sweep_ms = sum(sweep_list) / sweeps
    kern_ms = sweep_ms / w.layers
    per_layer_bytes = w.algorithmic_bytes()
    elems = w.elements * w.layers
    gbs = per_layer_bytes / (kern_ms * 1e-3) / 1e9
    del layers, ys
    torch.cuda.empty_cache()
    return {
        "workload": w.name,
        "value": elems / (sweep_ms * 1e-3), "unit": "elements/s",
        "ms_per_sweep_64_layers": sweep_ms,
        "sweep_ms_percentiles": percentiles(sweep_list),
        "us_per_layer": kern_ms * 1e3,
        "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "bytes_per_launch": per_layer_bytes},
        "wall_s": wall,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-seconds", type=float, default=0.5,
                    help="untimed clock ramp before the warm-up steps (0 = none)")
    ap.add_argument("--decode-sweeps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other scan configurations (tiny, Mamba-130M, long context)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward of the scan")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the A-per-channel / Euler scan variants")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the scan with the fused conv1d/softplus prologue")
    ap.add_argument("--no-ssd", action="store_true",
                    help="skip the masked-matrix scan with step and decay per head")
    ap.add_argument("--only-scan", action="store_true",
                    help="the headline scan only (for profiler runs)")
    ap.add_argument("--only-ssd", action="store_true",
                    help="the masked-matrix scan's forward only (for profiler runs)")
    ap.add_argument("--only-decode", action="store_true",
                    help="the decode sweep only (for profiler runs)")
    ap.add_argument("--only-config", default="",
                    help="one of the other scan configurations only, by workload name "
                         "(for profiler runs), e.g. mamba130m_b8_l2048_d1536")
    ap.add_argument("--only-ssd-bwd", action="store_true",
                    help="the masked-matrix scan's backward only (for profiler runs)")
    ap.add_argument("--sweep-plans", default="",
                    help="only time these chunk plans of the headline scan, e.g. 4x4,4x5,8x2 "
                         "(waves per group x chunks), under both schedules")
    ap.add_argument("--sweep-workload", default="",
                    help="the workload of --sweep-plans (default: the Mamba-2.8B layer)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (the known-size "
                         "kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "channels are independent, so a multi-GPU run would split D with no exchange", file=sys.stderr)
        sys.exit(2)
    if args.only_scan:
        args.no_configs = args.no_decode = args.no_backward = True
        args.no_variants = args.no_fused = args.no_ssd = True
        args.cpu_seconds = 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": COPY_BYTES}), flush=True)
        return

    if args.only_ssd:
        print(json.dumps({"ssd": bench_ssd_forward(args.steps, args.warmup)}), flush=True)
        return

    if args.only_decode:
        print(json.dumps({"decode": bench_decode(args.decode_sweeps)}), flush=True)
        return

    if args.only_config:
        from selective_state_space_44_amd import workloads as W
        spec = {W.TINY.name: (1, max(20, args.steps), 5),
                W.MAMBA_130M.name: (6, max(30, args.steps), 6),
                W.LONG_CTX.name: (1, args.steps, 2)}
        if args.only_config not in spec:
            print(f"bench.py: --only-config takes one of {sorted(spec)}", file=sys.stderr)
            sys.exit(2)
        w = W.WORKLOADS[args.only_config]
        print(json.dumps({"config": {w.name: bench_config(w, *spec[w.name])}}), flush=True)
        return

    if args.only_ssd_bwd:
        print(json.dumps({"ssd_bwd": bench_ssd_backward(args.steps, args.warmup)}), flush=True)
        return

    if args.sweep_plans:
        print(json.dumps({"plan_sweep": sweep_plans(args.sweep_plans, args.steps,
                                                    args.ramp_seconds, args.sweep_workload)}),
              flush=True)
        return

    r = bench_scan(args.steps, args.warmup, args.ramp_seconds)
    w = r["w"]
    elems = w.elements
    value = elems / (r["step_ms"] * 1e-3)
    alg_bytes = w.algorithmic_bytes()
    # the main-pass launch covers chunks 1 .. K-1 in the two-launch schedule
    # (chunk 0 runs in the first launch), every chunk in the three-pass one
    rows0 = chunk_rows(w.seqlen, r["K"]) if r["K"] > 1 and not r["three_pass"] else 0
    main_rows = w.seqlen - rows0
    main_elems = w.batch * main_rows * w.dim * w.dstate
    main_bytes = scan_bytes(w, main_rows)
    main_s = r["main_ms"] * 1e-3
    traffic = load_traffic()
    line = {
        "metric": "selective-scan B·L·D·N elems/s + % peak HBM GB/s, Mamba-2.8B layer shape",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": "bf16", "state_dtype": "f32",
                   "compute_dtype": "f32",
                   "plan": {"waves_per_group": r["G"], "nchunks": r["K"],
                            "schedule": "three-pass" if r["three_pass"] else "two-launch"}},
        "roofline": {
            "bound": "alu",
            "kernel": "scan_fwd_kernel (main pass, chunks %s)"
                      % ("0..K-1" if r["three_pass"] else "1..K-1"),
            "achieved": ALU_OPS_PER_ELEMENT * main_elems / main_s / 1e12,
            "peak": ALU_OPS_PER_ELEMENT * ALU_PEAK_ELEMS / 1e12,
            "unit": "TOP/s",
            "frac": main_elems / main_s / ALU_PEAK_ELEMS,
            "peak_basis": "6 fp32 ops at 16 lanes/clk + 1 exp2 at 8 lanes/clk per element, "
                          "1024 SIMDs x 2.4 GHz",
            "peak_dual_issue": ALU_OPS_PER_ELEMENT * ALU_PEAK_ELEMS_DUAL / 1e12,
            "frac_dual_issue": main_elems / main_s / ALU_PEAK_ELEMS_DUAL,
            "traffic": traffic,
            "launch_ms": r["main_ms"],
            "elements_per_launch": main_elems,
            "hbm": {"algorithmic_bytes_per_launch": main_bytes,
                    "achieved": main_bytes / main_s / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": main_bytes / main_s / 1e9 / HBM_PEAK_GBS,
                    "traffic_frac": (traffic / main_s / 1e9 / HBM_PEAK_GBS) if traffic else None},
        },
        "hbm": {
            "algorithmic_bytes": alg_bytes,
            "achieved": alg_bytes / (r["step_ms"] * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": alg_bytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "step_ms_percentiles": r["step_pct"],
        "main_pass_ms_percentiles": r["main_pct"],
        "first_launch_ms_per_step": r["first_ms"],
        "clock_ramp": {"seconds": args.ramp_seconds, "steps": r["ramp_steps"],
                       "why": "untimed steps before the warm-up: the clock rises over "
                              "the first ~30 ms of sustained work"},
        "wall_s_timed": r["wall_s"],
    }
    del r["inp"]
    if not args.no_configs:
        from selective_state_space_44_amd import workloads as W
        cfg = {}
        cfg[W.TINY.name] = bench_config(W.TINY, 1, max(20, args.steps), 5)
        # 6 sets of ~202 MB (1.2 GB) rotated past the 256 MB Infinity Cache
        cfg[W.MAMBA_130M.name] = bench_config(W.MAMBA_130M, 6, max(30, args.steps), 6)
        cfg[W.LONG_CTX.name] = bench_config(W.LONG_CTX, 1, 10, 2)
        line["configs"] = cfg
    if not args.no_decode:
        line["decode"] = bench_decode(args.decode_sweeps)
    if not args.no_fused:
        line["fused_prologue"] = bench_fused(max(20, args.steps // 4), 10)
    if not args.no_variants:
        line["variants"] = bench_variants(max(20, args.steps // 4), 10)
    if not args.no_ssd:
        line["ssd"] = bench_ssd(max(10, args.steps // 2), 10)
    if not args.no_backward:
        bwd = bench_backward(max(10, args.steps // 5), 5)
        bwd["time_vs_forward"] = bwd["ms_per_step"] / line["ms_per_step"]
        line["backward"] = bwd
    if args.cpu_seconds > 0:
        from selective_state_space_44_amd import workloads as W
        inp = W.make_inputs(W.MAMBA_2P8B, device="cuda:0", layer=0)
        line["cpu_baseline"] = cpu_baseline(inp, W.MAMBA_2P8B, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
