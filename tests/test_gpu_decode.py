"""GPU parity of the HIP decode step against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_44_amd as ssm
from selective_state_space_44_amd import workloads as W
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_step(inp, h64):
    return oracle.decode_step(h64, parity.to_f64(inp["x"]), parity.to_f64(inp["delta"]),
                              parity.to_f64(inp["A"]), parity.to_f64(inp["B"]),
                              parity.to_f64(inp["C"]), parity.to_f64(inp["D"]),
                              parity.to_f64(inp["z"]))


@pytest.mark.parametrize("layer", [0, 63])
def test_decode_full_layer(layer):
    """One layer of the 256-sequence x 5120-channel decode workload."""
    print(f"decode layer {layer}", flush=True)
    inp = W.make_inputs(W.DECODE_64L, device=DEV, layer=layer)
    h = inp["h"].clone()
    h64 = np.ascontiguousarray(parity.to_f64(h))
    y = ssm.decode_step(h, inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"])
    torch.cuda.synchronize()
    y_ref = _oracle_step(inp, h64)
    parity.check_y(parity.to_f64(y), y_ref, torch.bfloat16)
    parity.check_state(parity.to_f64(h), h64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_steps_equal_scan(dtype):
    """L decode steps from h0 reproduce the scan's outputs and final state."""
    inp = W.make_inputs(W.MAMBA_130M, device=DEV, batch=3, seqlen=40, dim=130)
    inp = {k: (v.to(dtype) if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    g = torch.Generator(device=DEV).manual_seed(5)
    h0 = torch.randn(3, 130, 16, generator=g, device=DEV)
    y_scan, h_scan = ssm.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                  inp["D"], inp["z"], h0, return_last_state=True)
    h = h0.clone()
    ys = []
    for t in range(40):
        ys.append(ssm.decode_step(h, inp["x"][:, t].contiguous(), inp["delta"][:, t].contiguous(),
                                  inp["A"], inp["B"][:, t].contiguous(),
                                  inp["C"][:, t].contiguous(), inp["D"],
                                  inp["z"][:, t].contiguous()))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, 1)
    y_ref, h_ref = parity.oracle_scan(dict(inp, h0=h0))
    parity.check_y(parity.to_f64(y_dec), y_ref, dtype, "decode y")
    parity.check_state(parity.to_f64(h), h_ref, "decode h")
    parity.check_y(parity.to_f64(y_scan), y_ref, dtype, "scan y")
    parity.check_state(parity.to_f64(h_scan), h_ref, "scan h")


def test_decode_edge_cases():
    # ragged dim, no gate / no skip, zero A entries
    inp = W.make_inputs(W.DECODE_64L, device=DEV, batch=3, dim=37)
    inp["A"][4, 2] = 0.0
    for over in ({}, {"z": None}, {"D": None}):
        p = dict(inp, **over)
        h = p["h"].clone()
        h64 = np.ascontiguousarray(parity.to_f64(h))
        y = ssm.decode_step(h, p["x"], p["delta"], p["A"], p["B"], p["C"], p.get("D"),
                            p.get("z"))
        torch.cuda.synchronize()
        y_ref = oracle.decode_step(h64, parity.to_f64(p["x"]), parity.to_f64(p["delta"]),
                                   parity.to_f64(p["A"]), parity.to_f64(p["B"]),
                                   parity.to_f64(p["C"]), parity.to_f64(p.get("D")),
                                   parity.to_f64(p.get("z")))
        parity.check_y(parity.to_f64(y), y_ref, torch.bfloat16)
        parity.check_state(parity.to_f64(h), h64)
    with pytest.raises(ssm.SsmError):
        h = torch.zeros(2, 8, 4, device=DEV)
        ssm.decode_step(h, torch.zeros(2, 8, device=DEV), torch.zeros(2, 8, device=DEV),
                        torch.zeros(8, 4, device=DEV), torch.zeros(2, 4, device=DEV),
                        torch.zeros(2, 4, device=DEV))


@pytest.mark.parametrize("batch", [1, 2, 5])
@pytest.mark.parametrize("variant", ["zoh", "a_per_channel", "euler"])
def test_decode_row_pairs(batch, variant):
    """Each thread steps two batch rows; odd batches leave the last pair with
    one row, whose partner must be neither written nor stored.  Checked
    against the oracle's scan of length 1 from the resident state."""
    inp = W.make_inputs(W.DECODE_64L, device=DEV, batch=batch, dim=200)
    if variant == "a_per_channel":
        inp["A"] = W.make_channel_A(W.DECODE_64L, device=DEV, dim=200)
    disc = "euler" if variant == "euler" else "zoh"
    h = inp["h"].clone()
    y = ssm.decode_step(h, inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"], discretization=disc)
    torch.cuda.synchronize()
    seq = {k: inp[k][:, None] for k in ("x", "delta", "z", "B", "C")}
    y_ref, h_ref = parity.oracle_scan(dict(seq, A=inp["A"], D=inp["D"], h0=inp["h"]),
                                      discretization=disc)
    parity.check_y(parity.to_f64(y), y_ref[:, 0], torch.bfloat16)
    parity.check_state(parity.to_f64(h), h_ref)
