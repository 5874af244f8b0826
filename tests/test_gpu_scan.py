"""GPU parity of the HIP selective scan against the CPU oracle.

Every case runs the HIP library through the binding (C ABI) on seeded
synthetic inputs and compares element by element with the oracle on the same
bytes, at the tolerances in ``parity.py``.
"""
import numpy as np
import pytest
import torch

import selective_state_space_44_amd as ssm
from selective_state_space_44_amd import workloads as W
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PLANS = [(2, 1), (4, 1), (8, 1), (16, 1), (4, 3), (2, 5), (16, 2), (8, 7)]


def _inputs(w, **kw):
    inp = W.make_inputs(w, device=DEV, **kw)
    return inp


# phase 3: the two-launch schedule (chunk 0's main pass beside the pre-pass
# of chunks 1..K-2); phase 7: the three-pass schedule (pre-pass of chunks
# 0..K-2, then the main pass of every chunk); phase 0 (the default of _run):
# the schedule the plan prefers, as ssm_scan_fwd runs it
SCHEDULES = {"two_launch": 3, "three_pass": 7}


def _run(inp, G=0, K=0, with_state=True, phase=0, **over):
    p = dict(inp, **over)
    return ssm.scan_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"),
                        p.get("h0"), return_last_state=with_state, waves_per_group=G,
                        nchunks=K, phase=phase)


@pytest.fixture(scope="module")
def tiny():
    inp = _inputs(W.TINY)
    y_ref, h_ref = parity.oracle_scan(inp)
    return inp, y_ref, h_ref


@pytest.mark.parametrize("schedule", list(SCHEDULES))
@pytest.mark.parametrize("G,K", PLANS)
def test_tiny_fp32_all_plans(tiny, G, K, schedule):
    inp, y_ref, h_ref = tiny
    print(f"tiny fp32 G={G} K={K} {schedule}", flush=True)
    y, h = _run(inp, G, K, phase=SCHEDULES[schedule])
    torch.cuda.synchronize()
    parity.check_y(parity.to_f64(y), y_ref, torch.float32)
    parity.check_state(parity.to_f64(h), h_ref)


@pytest.mark.parametrize("G,K,phase", [(2, 1, 3), (4, 1, 3), (16, 1, 3), (4, 4, 3), (8, 3, 3),
                                       (4, 2, 3), (4, 4, 7), (2, 6, 7)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_sizes_with_h0_and_no_gate(G, K, phase, dtype):
    """batch 2, L=1003 (not a tile multiple), dim=200 (not a multiple of 64),
    random initial state, with and without z and D; both schedules."""
    print(f"ragged {dtype} G={G} K={K} phase={phase}", flush=True)
    w = W.MAMBA_130M
    inp = _inputs(w, batch=2, seqlen=1003, dim=200)
    inp = {k: (v.to(dtype) if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    g = torch.Generator(device=DEV).manual_seed(77)
    inp["h0"] = torch.randn(2, 200, 16, generator=g, device=DEV)
    for variant in ("full", "no_gate", "no_skip"):
        over = {}
        if variant == "no_gate":
            over["z"] = None
        if variant == "no_skip":
            over["D"] = None
        p = dict(inp, **over)
        y_ref, h_ref = parity.oracle_scan(p)
        y, h = _run(p, G, K, phase=phase)
        torch.cuda.synchronize()
        parity.check_y(parity.to_f64(y), y_ref, dtype, what=f"y[{variant}]")
        parity.check_state(parity.to_f64(h), h_ref, what=f"h_last[{variant}]")


def _sampled_channels(dim, n, seed):
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(dim, size=min(n, dim), replace=False).tolist())
    picks |= {0, dim - 1}
    return sorted(picks)


@pytest.mark.parametrize("w", [W.MAMBA_130M, W.MAMBA_2P8B], ids=lambda w: w.name)
def test_full_size_sampled_channels(w):
    """Full benchmark shapes in the automatic plan (the launch configuration
    the benchmark times); the oracle computes 256 sampled channels (plus the
    first and last) over the whole sequence for every batch row."""
    print(f"full {w.name} plan={ssm.scan_plan(w.batch, w.seqlen, w.dim, with_phase=True)}",
          flush=True)
    inp = _inputs(w)
    y, h = _run(inp)
    torch.cuda.synchronize()
    ch = _sampled_channels(w.dim, 256, 5)
    assert len(ch) >= 256
    y_ref, h_ref = parity.oracle_scan(inp, channels=ch)
    parity.check_y(parity.pick(y, ch, 2), y_ref, w.io_dtype)
    parity.check_state(parity.pick(h, ch, 1), h_ref)


@pytest.mark.parametrize("schedule", list(SCHEDULES))
def test_full_size_five_chunks(schedule):
    """The Mamba-2.8B layer under the five-chunk plan (1280 blocks per launch,
    five per CU), which the planner rates equal in time to its four-chunk
    choice: 96 sampled channels (plus the first and last) of every batch row
    against the oracle, in both schedules."""
    w = W.MAMBA_2P8B
    print(f"full {w.name} G=4 K=5 {schedule}", flush=True)
    inp = _inputs(w)
    y, h = _run(inp, 4, 5, phase=SCHEDULES[schedule])
    torch.cuda.synchronize()
    ch = _sampled_channels(w.dim, 96, 9)
    y_ref, h_ref = parity.oracle_scan(inp, channels=ch)
    parity.check_y(parity.pick(y, ch, 2), y_ref, w.io_dtype)
    parity.check_state(parity.pick(h, ch, 1), h_ref)


def long_context_channels(delta, n=256, most_negative=8):
    """Channels of the long-context workload that span its per-channel delta
    bias: ranked by mean delta over the first 4096 steps (the bias dominates
    it), the `most_negative` longest-memory channels plus channels at evenly
    spaced ranks up to the shortest-memory one."""
    rank = torch.argsort(delta[0, :4096].float().mean(0)).tolist()
    picks = set(rank[:most_negative])
    spaced = np.linspace(0, len(rank) - 1, n - most_negative).round().astype(int)
    picks |= {rank[i] for i in spaced}
    i = most_negative
    while len(picks) < n:
        picks.add(rank[i])
        i += 1
    return sorted(picks), rank


def test_long_context_sampled_channels():
    """L = 262144 single sequence with per-channel delta bias: the plan cuts
    it into chunks, so this checks the cross-chunk carry at full length over
    256 channels spanning the bias range, including the 8 channels with the
    most negative bias (longest memory)."""
    w = W.LONG_CTX
    print(f"full {w.name} plan={ssm.scan_plan(w.batch, w.seqlen, w.dim, with_phase=True)}",
          flush=True)
    inp = _inputs(w)
    y, h = _run(inp)
    torch.cuda.synchronize()
    ch, rank = long_context_channels(inp["delta"])
    assert len(ch) >= 256 and set(rank[:8]) <= set(ch) and rank[-1] in ch
    y_ref, h_ref = parity.oracle_scan(inp, channels=ch)
    parity.check_y(parity.pick(y, ch, 2), y_ref, w.io_dtype)
    parity.check_state(parity.pick(h, ch, 1), h_ref)


@pytest.mark.parametrize("G,K", [(4, 4), (4, 2), (8, 5), (2, 3)])
def test_phases_enqueued_apart(G, K):
    """Phase 1 then phase 2 gives the same bytes as phase 3, for both
    schedules; the two schedules agree within the fp32 rule (they round the
    state entering chunk 1 along different paths)."""
    inp = _inputs(W.MAMBA_130M, batch=2, seqlen=1000, dim=192)
    g = torch.Generator(device=DEV).manual_seed(21)
    inp["h0"] = torch.randn((2, 192, 16), generator=g, device=DEV)
    res = {}
    for base in (0, 4):
        y3, h3 = _run(inp, G, K, phase=base | 3)
        ws = torch.empty(ssm.scan_workspace_bytes(2, 1000, 192, nchunks=K) + 256,
                         dtype=torch.uint8, device=DEV)
        y = torch.empty_like(inp["x"])
        hl = torch.empty_like(inp["h0"])
        for ph in (base | 1, base | 2):
            args = [inp[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0")]
            st = ssm.load_library().ssm_scan_fwd_phase(
                2, 1000, 192, 16, ssm.SSM_DTYPE_BF16, *[ssm._ptr(a) for a in args],
                ssm._ptr(y), ssm._ptr(hl), ssm._ptr(ws), ws.numel(), G, K, ph,
                ssm._stream(inp["x"].device))
            assert st == ssm.SSM_OK
        torch.cuda.synchronize()
        assert torch.equal(y, y3) and torch.equal(hl, h3), f"phase split, base {base}"
        res[base] = (y3, h3)
    parity.check_state(parity.to_f64(res[0][1]), parity.to_f64(res[4][1]), "h_last schedules")
    y_ref, h_ref = parity.oracle_scan(inp)
    for base in (0, 4):
        parity.check_y(parity.to_f64(res[base][0]), y_ref, torch.bfloat16)
        parity.check_state(parity.to_f64(res[base][1]), h_ref)


def test_chunk_and_resume_invariance():
    """scan(L) equals scan(L1) -> h_last -> h0 -> scan(L - L1), and the same
    result comes out of different chunk plans (within tolerance)."""
    inp = _inputs(W.MAMBA_130M, batch=2, seqlen=700, dim=128)
    inp = {k: (v.float() if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    y, h = _run(inp, 4, 1)
    y5, h5 = _run(inp, 4, 5)
    torch.cuda.synchronize()
    parity.check_state(parity.to_f64(y5), parity.to_f64(y), "chunked y")
    parity.check_state(parity.to_f64(h5), parity.to_f64(h), "chunked h")
    cut = 333
    a = {k: (v[:, :cut].contiguous() if k in ("x", "delta", "z", "B", "C") else v)
         for k, v in inp.items()}
    b = {k: (v[:, cut:].contiguous() if k in ("x", "delta", "z", "B", "C") else v)
         for k, v in inp.items()}
    ya, ha = _run(a, 4, 1)
    yb, hb = _run(dict(b, h0=ha), 4, 1)
    torch.cuda.synchronize()
    parity.check_state(parity.to_f64(torch.cat([ya, yb], 1)), parity.to_f64(y), "resumed y")
    parity.check_state(parity.to_f64(hb), parity.to_f64(h), "resumed h")


@pytest.mark.parametrize("K", [2, 17, 65, 100])
def test_many_chunks_carry_rounds(K):
    """The carry composes the chunk maps with an in-wave prefix scan over
    segments of up to 64 lanes; more than 65 chunks take several rounds.
    fp32 I/O against the oracle, with h0."""
    w = W.MAMBA_130M
    inp = _inputs(w, batch=2, seqlen=1600, dim=96)
    inp = {k: (v.float() if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    g = torch.Generator(device=DEV).manual_seed(11)
    inp["h0"] = torch.randn((2, 96, 16), generator=g, device=DEV)
    y, h = _run(inp, 4, K)
    torch.cuda.synchronize()
    y_ref, h_ref = parity.oracle_scan(inp)
    parity.check_y(parity.to_f64(y), y_ref, torch.float32)
    parity.check_state(parity.to_f64(h), h_ref)


def test_deterministic():
    inp = _inputs(W.MAMBA_130M, batch=2, seqlen=512, dim=256)
    y1, h1 = _run(inp, 8, 3)
    y2, h2 = _run(inp, 8, 3)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_delta_zero_keeps_state():
    inp = _inputs(W.TINY)
    g = torch.Generator(device=DEV).manual_seed(3)
    h0 = torch.randn(1, 64, 16, generator=g, device=DEV)
    p = dict(inp, delta=torch.zeros_like(inp["delta"]), h0=h0)
    for G, K in ((2, 1), (4, 2), (16, 1)):
        y, h = _run(p, G, K)
        torch.cuda.synchronize()
        # Abar = exp2(0) = 1 and Bbar*x = fma(1, q, -q) = 0 exactly, so the
        # state comes back bit-for-bit
        assert torch.equal(h, h0)
        y_ref, _ = parity.oracle_scan(p)
        parity.check_y(parity.to_f64(y), y_ref, torch.float32)


def test_zero_A_uses_the_limit():
    inp = _inputs(W.TINY)
    A = inp["A"].clone()
    A[5, 3] = 0.0
    A[17, :] = 0.0
    A[40, 15] = -0.0
    p = dict(inp, A=A)
    y_ref, h_ref = parity.oracle_scan(p)
    for G, K in ((2, 1), (4, 3), (16, 1)):
        y, h = _run(p, G, K)
        torch.cuda.synchronize()
        parity.check_y(parity.to_f64(y), y_ref, torch.float32)
        parity.check_state(parity.to_f64(h), h_ref)


def test_large_delta_overwrites_state():
    inp = _inputs(W.TINY)
    p = dict(inp, delta=torch.full_like(inp["delta"], 60.0))
    y_ref, h_ref = parity.oracle_scan(p)
    y, h = _run(p, 4, 2)
    torch.cuda.synchronize()
    parity.check_y(parity.to_f64(y), y_ref, torch.float32)
    parity.check_state(parity.to_f64(h), h_ref)


def test_edge_sizes():
    w = W.TINY
    # seqlen 0: h_last = h0 (or zeros), y empty
    inp = _inputs(w, seqlen=0)
    g = torch.Generator(device=DEV).manual_seed(4)
    h0 = torch.randn(1, 64, 16, generator=g, device=DEV)
    y, h = _run(dict(inp, h0=h0))
    torch.cuda.synchronize()
    assert y.shape == (1, 0, 64) and torch.equal(h, h0)
    _, hz = _run(inp)
    torch.cuda.synchronize()
    assert torch.all(hz == 0)
    # L = 1, dim = 1, batch 3
    for (b, L, d) in ((1, 1, 64), (3, 5, 1), (2, 17, 65)):
        inp = _inputs(w, batch=b, seqlen=L, dim=d)
        y_ref, h_ref = parity.oracle_scan(inp)
        for G, K in ((2, 1), (16, 1), (4, 4)):
            y, h = _run(inp, G, K)
            torch.cuda.synchronize()
            parity.check_y(parity.to_f64(y), y_ref, torch.float32)
            parity.check_state(parity.to_f64(h), h_ref)


def test_nan_propagates():
    inp = _inputs(W.TINY)
    x = inp["x"].clone()
    x[0, 100, 7] = float("nan")
    y, h = _run(dict(inp, x=x))
    torch.cuda.synchronize()
    assert torch.isnan(y[0, 100:, 7]).all() and not torch.isnan(y[0, :100]).any()
    assert torch.isnan(h[0, 7]).all() and not torch.isnan(h[0, 8]).any()


def test_unsupported_plan_raises():
    inp = _inputs(W.TINY)
    with pytest.raises(ssm.SsmError) as e:
        _run(inp, 1, 1)
    assert e.value.status == ssm.SSM_ERR_UNSUPPORTED


def test_unsupported_state_size_raises():
    inp = _inputs(W.TINY)
    with pytest.raises(ssm.SsmError) as e:
        ssm.scan_fwd(inp["x"], inp["delta"], inp["A"][:, :8].contiguous(),
                     inp["B"][:, :, :8].contiguous(), inp["C"][:, :, :8].contiguous())
    assert e.value.status == ssm.SSM_ERR_UNSUPPORTED


def test_native_library_is_loaded():
    import os
    ssm.load_library()
    maps = open(f"/proc/{os.getpid()}/maps").read()
    assert ssm.LIB_PATH in maps
