#!/usr/bin/env python3
"""Benchmark of the selective state-space scan on one MI355X.

One step = one forward scan of the Mamba-2.8B layer shape
(batch 4, L 4096, D 5120, N 16; bf16 x/delta/z/B/C/y, fp32 A/D and state)
on seeded synthetic inputs already resident in HBM.  Prints one JSON line
with whole-job throughput in B*L*D*N elements/s, the roofline of the
dominant kernel (the main scan pass), the HBM view, the recurrent decode
sweep (256 sequences x 64 layers of D 5120, N 16) and the fp64 CPU
baseline timed on a bounded sample on this host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
# ALU roofline of the scan element: per element (b, t, d, n) the main pass
# issues 6 fp32 VALU ops + 1 transcendental (exp2).  Per SIMD per clock: 32 fp32
# lanes (157.3 TFLOP/s fp32 vector = 256 CU x 4 SIMD x 32 lanes x 2 x 2.4 GHz)
# and a quarter of that for transcendentals.
ALU_OPS_PER_ELEMENT = 7
SIMDS, CLOCK_HZ, VALU_LANES, TRANS_LANES = 256 * 4, 2.4e9, 32, 8
ALU_PEAK_ELEMS = SIMDS * CLOCK_HZ / (6 / VALU_LANES + 1 / TRANS_LANES)
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_main_mamba2p8b_b4_l4096_d5120_traffic.md")


def source_hash() -> str:
    """Hash of the library sources with /* */ and // comments and blank lines
    removed (a comment edit does not change a kernel; any code edit does)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "selective_state_space_44_amd", "csrc", "*")))
    for f in files + [os.path.join(ROOT, "include", "ssm.h")]:
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the main kernel, from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, when it was taken on the current sources
    (its ``source_hash`` line matches); None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    h = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    b = re.search(r"^hbm_bytes_per_launch:\s*(\d+)", text, re.M)
    if not h or not b or h.group(1) != source_hash():
        return None
    return int(b.group(1))


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(inp, w, target_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    the first ``nb`` batch rows, the first ``nch`` channels of each, over the
    full sequence."""
    import torch
    import oracle

    nthreads = cpu_threads()

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
            "sample": f"{nb} of {w.batch} batch rows x {nch} of {w.dim} channels, full "
                      f"L={w.seqlen}, N={w.dstate}: {elems:.3e} elements in {dt:.1f} s "
                      f"(fp64 C loop, gcc -O2, OpenMP over channels)"}


def percentiles(ms):
    """p10, median and p90 of per-step times in ms (nearest rank)."""
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def bench_scan(steps: int, warmup: int):
    import torch
    import selective_state_space_44_amd as ssm
    from selective_state_space_44_amd import workloads as W

    w = W.MAMBA_2P8B
    dev = "cuda:0"
    # two input sets, alternated, so no step reads what the previous left in
    # the 256 MB Infinity Cache (one set is ~0.67 GB anyway)
    sets = [W.make_inputs(w, device=dev, layer=i) for i in range(2)]
    outs = [torch.empty_like(s["x"]) for s in sets]
    G, K = ssm.scan_plan(w.batch, w.seqlen, w.dim)
    nws = ssm.scan_workspace_bytes(w.batch, w.seqlen, w.dim, nchunks=K)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        s, y = sets[i % 2], outs[i % 2]
        args = (s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], None)
        kw = dict(waves_per_group=G, nchunks=K, out=y, workspace=ws)
        if ev is not None:
            ev[0].record()
        ssm.scan_fwd(*args, phase=1, **kw)
        if ev is not None:
            ev[1].record()
        ssm.scan_fwd(*args, phase=2, **kw)
        if ev is not None:
            ev[2].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_step = [e[0].elapsed_time(e[2]) for e in evs]
    ev_main = [e[1].elapsed_time(e[2]) for e in evs]
    ev_carry = [e[0].elapsed_time(e[1]) for e in evs]
    return dict(w=w, G=G, K=K, wall_s=wall, step_ms=sum(ev_step) / steps,
                main_ms=sum(ev_main) / steps, carry_ms=sum(ev_carry) / steps, inp=sets[0],
                step_pct=percentiles(ev_step), main_pct=percentiles(ev_main))


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
    # per (batch row, head, chunk) the lower triangle of C B^T (Q(Q+1)/2 N) and of
    # P x (Q(Q+1)/2 P), C h (Q N P) and the state update (Q N P) multiply-adds
    Q, P, N = 32, w.headdim, w.dstate
    heads = w.dim // P
    chunks = (w.seqlen + Q - 1) // Q
    flops = 2 * w.batch * heads * chunks * (Q * (Q + 1) // 2 * (N + P) + 2 * Q * N * P)
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
    del q, yq
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

    for _ in range(2):
        sweep()
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-sweeps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward of the scan")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the A-per-channel / Euler scan variants")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the scan with the fused conv1d/softplus prologue")
    ap.add_argument("--no-ssd", action="store_true",
                    help="skip the masked-matrix scan with step and decay per head")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (the known-size "
                         "kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "channels are independent, so a multi-GPU run would split D with no exchange", file=sys.stderr)
        sys.exit(2)

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

    r = bench_scan(args.steps, args.warmup)
    w = r["w"]
    elems = w.elements
    value = elems / (r["step_ms"] * 1e-3)
    main_elems = elems / (r["main_ms"] * 1e-3)
    alg_bytes = w.algorithmic_bytes()
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": "bf16", "state_dtype": "f32",
                   "plan": {"waves_per_group": r["G"], "nchunks": r["K"]}},
        "roofline": {
            "bound": "alu",
            "kernel": "scan_fwd_kernel (main pass)",
            "achieved": ALU_OPS_PER_ELEMENT * main_elems / 1e12,
            "peak": ALU_OPS_PER_ELEMENT * ALU_PEAK_ELEMS / 1e12,
            "unit": "TOP/s",
            "frac": main_elems / ALU_PEAK_ELEMS,
            "traffic": traffic,
            "launch_ms": r["main_ms"],
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
        "carry_ms_per_step": r["carry_ms"],
        "wall_s_timed": r["wall_s"],
    }
    if not args.no_decode:
        line["decode"] = bench_decode(args.decode_sweeps)
    if not args.no_fused:
        line["fused_prologue"] = bench_fused(max(10, args.steps // 4), max(10, args.warmup // 4))
    if not args.no_variants:
        line["variants"] = bench_variants(max(10, args.steps // 4), max(10, args.warmup // 4))
    if not args.no_ssd:
        line["ssd"] = bench_ssd(max(10, args.steps // 2), max(10, args.warmup // 10))
    if not args.no_backward:
        bwd = bench_backward(max(10, args.steps // 5), max(5, args.warmup // 20))
        bwd["time_vs_forward"] = bwd["ms_per_step"] / r["step_ms"]
        line["backward"] = bwd
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(r["inp"], w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
