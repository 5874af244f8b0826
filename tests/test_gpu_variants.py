"""GPU parity of the scan variants (``ssm_scan_fwd_ex``) against the oracle:
A given per channel (one value shared by the channel's states) and the Euler
rule Bbar = delta*B, alone and combined, over several chunk plans, ragged
sizes, both I/O types and the full benchmark shape (sampled channels)."""
import numpy as np
import pytest
import torch

import selective_state_space_44_amd as ssm
from selective_state_space_44_amd import workloads as W
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
VARIANTS = [("channel", "zoh"), ("state", "euler"), ("channel", "euler")]
PLANS = [(2, 1), (4, 1), (8, 1), (4, 3), (2, 5), (8, 7)]


def _ids(v):
    return f"A_per_{v[0]}-{v[1]}"


def _inputs(w, a_kind, **kw):
    inp = W.make_inputs(w, device=DEV, **kw)
    if a_kind == "channel":
        inp["A"] = W.make_channel_A(w, device=DEV, dim=inp["x"].shape[2])
    return inp


def _oracle(p, disc, channels=None):
    return parity.oracle_scan(p, channels=channels, discretization=disc)


def _run(p, disc, G=0, K=0):
    return ssm.scan_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"),
                        p.get("h0"), return_last_state=True, waves_per_group=G, nchunks=K,
                        discretization=disc)


@pytest.mark.parametrize("variant", VARIANTS, ids=_ids)
def test_tiny_fp32_plans(variant):
    a_kind, disc = variant
    inp = _inputs(W.TINY, a_kind)
    g = torch.Generator(device=DEV).manual_seed(5)
    inp["h0"] = torch.randn(1, 64, 16, generator=g, device=DEV)
    y_ref, h_ref = _oracle(inp, disc)
    for G, K in PLANS:
        print(f"variant {variant} tiny G={G} K={K}", flush=True)
        y, h = _run(inp, disc, G, K)
        torch.cuda.synchronize()
        parity.check_y(parity.to_f64(y), y_ref, torch.float32, what=f"y G={G} K={K}")
        parity.check_state(parity.to_f64(h), h_ref, what=f"h G={G} K={K}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("variant", VARIANTS, ids=_ids)
def test_ragged_sizes(variant, dtype):
    """batch 2, L = 1003, dim = 200 with h0; with and without gate and skip."""
    a_kind, disc = variant
    inp = _inputs(W.MAMBA_130M, a_kind, batch=2, seqlen=1003, dim=200)
    inp = {k: (v.to(dtype) if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    g = torch.Generator(device=DEV).manual_seed(6)
    inp["h0"] = torch.randn(2, 200, 16, generator=g, device=DEV)
    for over in ({}, {"z": None}, {"D": None}):
        p = dict(inp, **over)
        y_ref, h_ref = _oracle(p, disc)
        for G, K in ((2, 1), (4, 4), (8, 3)):
            print(f"variant {variant} ragged {dtype} {sorted(over)} G={G} K={K}", flush=True)
            y, h = _run(p, disc, G, K)
            torch.cuda.synchronize()
            parity.check_y(parity.to_f64(y), y_ref, dtype)
            parity.check_state(parity.to_f64(h), h_ref)


@pytest.mark.parametrize("variant", VARIANTS, ids=_ids)
def test_full_size_sampled_channels(variant):
    a_kind, disc = variant
    w = W.MAMBA_2P8B
    inp = _inputs(w, a_kind)
    print(f"variant {variant} full {w.name}", flush=True)
    y, h = _run(inp, disc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    ch = sorted(set(rng.choice(w.dim, 40, replace=False).tolist()) | {0, w.dim - 1})
    y_ref, h_ref = _oracle(inp, disc, channels=ch)
    parity.check_y(parity.pick(y, ch, 2), y_ref, w.io_dtype)
    parity.check_state(parity.pick(h, ch, 1), h_ref)


def test_zero_and_delta_edge_cases():
    """Per-channel A with zeros takes the delta*B limit; delta = 0 keeps the
    state bit for bit in every variant."""
    inp = _inputs(W.TINY, "channel")
    A = inp["A"].clone()
    A[3] = 0.0
    A[40] = -0.0
    p = dict(inp, A=A)
    for disc in ("zoh", "euler"):
        y_ref, h_ref = _oracle(p, disc)
        for G, K in ((2, 1), (4, 3)):
            y, h = _run(p, disc, G, K)
            torch.cuda.synchronize()
            parity.check_y(parity.to_f64(y), y_ref, torch.float32)
            parity.check_state(parity.to_f64(h), h_ref)
    g = torch.Generator(device=DEV).manual_seed(8)
    h0 = torch.randn(1, 64, 16, generator=g, device=DEV)
    for a_kind, disc in VARIANTS:
        q = dict(_inputs(W.TINY, a_kind), h0=h0)
        q["delta"] = torch.zeros_like(q["delta"])
        for G, K in ((2, 1), (8, 2)):
            _, h = _run(q, disc, G, K)
            torch.cuda.synchronize()
            assert torch.equal(h, h0), (a_kind, disc, G, K)


def test_state_A_zeros_and_zero_delta_four_wave_plans():
    """A per (channel, state) with zeros under both rules, at the 4-wave plans
    (whose kernels give each wave 16 channels with all their states) with
    one, three and five chunks and a ragged tail (L = 203), h0 given; and a
    zero step keeps the state bit for bit under the Euler rule too."""
    inp = _inputs(W.TINY, "state", seqlen=203)
    A = inp["A"].clone()
    A[5, 3] = 0.0
    A[17, :] = 0.0
    A[40, 15] = -0.0
    g = torch.Generator(device=DEV).manual_seed(12)
    h0 = torch.randn(1, 64, 16, generator=g, device=DEV)
    p = dict(inp, A=A, h0=h0)
    for disc in ("zoh", "euler"):
        y_ref, h_ref = _oracle(p, disc)
        for K in (1, 3, 5):
            print(f"A zeros {disc} G=4 K={K}", flush=True)
            y, h = _run(p, disc, 4, K)
            torch.cuda.synchronize()
            parity.check_y(parity.to_f64(y), y_ref, torch.float32, what=f"y {disc} K={K}")
            parity.check_state(parity.to_f64(h), h_ref, what=f"h {disc} K={K}")
    q = dict(p, delta=torch.zeros_like(p["delta"]))
    for disc in ("zoh", "euler"):
        for K in (1, 3):
            _, h = _run(q, disc, 4, K)
            torch.cuda.synchronize()
            assert torch.equal(h, h0), (disc, K)


def test_variant_edge_sizes():
    for a_kind, disc in VARIANTS:
        for (b, L, d) in ((1, 1, 64), (3, 5, 1), (2, 17, 65)):
            inp = _inputs(W.TINY, a_kind, batch=b, seqlen=L, dim=d)
            y_ref, h_ref = _oracle(inp, disc)
            for G, K in ((2, 1), (4, 4)):
                y, h = _run(inp, disc, G, K)
                torch.cuda.synchronize()
                parity.check_y(parity.to_f64(y), y_ref, torch.float32)
                parity.check_state(parity.to_f64(h), h_ref)


def test_euler_differs_from_zoh():
    """The flag reaches the kernel: Euler and ZOH give different states."""
    inp = _inputs(W.TINY, "state")
    _, hz = _run(inp, "zoh", 4, 1)
    _, he = _run(inp, "euler", 4, 1)
    torch.cuda.synchronize()
    assert not torch.allclose(hz, he, rtol=1e-3, atol=1e-4)


def test_variant_rejects_sixteen_waves_and_phases():
    inp = _inputs(W.TINY, "channel")
    with pytest.raises(ssm.SsmError) as e:
        _run(inp, "zoh", 16, 1)
    assert e.value.status == ssm.SSM_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        ssm.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], phase=1)


@pytest.mark.parametrize("n", [16, 32, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("variant", VARIANTS, ids=_ids)
def test_decode_variants(variant, dtype, n):
    """ssm_decode_step_ex: one step on a resident state equals the oracle's
    scan of length 1 from h0 = that state; 8 sequences x 130 channels (ragged
    block), A = 0 on two channels."""
    a_kind, disc = variant
    print(f"decode variant {variant} {dtype} N={n}", flush=True)
    d = W.make_inputs(W.DECODE_64L, device=DEV, batch=8, dim=130, dstate=n)
    d = {k: (v.to(dtype) if k in ("x", "delta", "z", "B", "C") else v) for k, v in d.items()}
    if a_kind == "channel":
        d["A"] = W.make_channel_A(W.DECODE_64L, device=DEV, dim=130)
    d["A"][3] = 0.0
    d["A"][77] = 0.0
    h0 = d["h"].clone()
    y = ssm.decode_step(d["h"], d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        discretization=disc)
    torch.cuda.synchronize()
    as_scan = dict(x=d["x"][:, None, :], delta=d["delta"][:, None, :], A=d["A"],
                   B=d["B"][:, None, :], C=d["C"][:, None, :], D=d["D"], z=d["z"][:, None, :],
                   h0=h0)
    y_ref, h_ref = parity.oracle_scan(as_scan, discretization=disc)
    parity.check_y(parity.to_f64(y), y_ref[:, 0, :], dtype, what="decode y")
    parity.check_state(parity.to_f64(d["h"]), h_ref, what="decode state")
