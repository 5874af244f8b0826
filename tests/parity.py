"""Parity helpers: run the oracle on the exact bytes the GPU read, compare.

Tolerances (per element):
  * fp32 I/O, and every fp32 state:  |got - ref| <= 1e-4 * (1 + |ref|)
  * bf16 I/O outputs y:               |got - ref| <= 2e-2 * max(|ref|, 1e-2 * rms(ref))
    (relative error, with a floor at 1% of the output's rms for outputs that
    are near zero because of the gate or cancellation; rms over the compared
    outputs).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

FP32_TOL = 1e-4
BF16_REL = 2e-2
BF16_FLOOR = 1e-2
# gradients in fp32: per element, relative to |ref| + rms of the tensor
GRAD_FP32_TOL = 1e-4


def to_f64(t):
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_y(got, ref, io_dtype, what="y"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    if io_dtype == torch.float32:
        bound = FP32_TOL * (1.0 + np.abs(ref))
    else:
        rms = float(np.sqrt(np.mean(ref * ref)))
        bound = BF16_REL * np.maximum(np.abs(ref), BF16_FLOOR * rms)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)),
                             ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside tolerance; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def check_state(got, ref, what="state"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = FP32_TOL * (1.0 + np.abs(ref))
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside tolerance; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    return float(np.max(err / bound)) if err.size else 0.0


def oracle_scan(inp: dict, channels=None, nthreads: int = 0, discretization: str = "zoh"):
    """Oracle on the inputs dict of the scan (device tensors); ``channels``
    optionally restricts to a subset of d (channels are independent).  A may
    be [d, n] or [d] (one value per channel)."""
    x, delta, A, B, C = inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"]
    D, z, h0 = inp.get("D"), inp.get("z"), inp.get("h0")
    if channels is not None:
        idx = torch.as_tensor(channels, device=x.device, dtype=torch.long)
        x, delta = x.index_select(2, idx), delta.index_select(2, idx)
        z = z.index_select(2, idx) if z is not None else None
        A = A.index_select(0, idx)
        D = D.index_select(0, idx) if D is not None else None
        h0 = h0.index_select(1, idx) if h0 is not None else None
    return oracle.scan(to_f64(x), to_f64(delta), to_f64(A), to_f64(B), to_f64(C),
                       to_f64(D), to_f64(z), to_f64(h0), nthreads=nthreads,
                       discretization=discretization)


def pick(t, channels, axis):
    idx = torch.as_tensor(channels, device=t.device, dtype=torch.long)
    return to_f64(t.index_select(axis, idx))


def check_grad(got, ref, io_dtype, what):
    """Gradients: fp32 outputs |err| <= GRAD_FP32_TOL * (|ref| + rms(ref));
    bf16 outputs as check_y's bf16 bound.  The rms term is the scale of the
    tensor: reduced gradients (sums over channels or time) and the adjoint
    carry cancellation, so a pure relative bound is undefined near zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    if io_dtype == torch.float32:
        bound = GRAD_FP32_TOL * (np.abs(ref) + rms)
    else:
        bound = BF16_REL * np.maximum(np.abs(ref), BF16_FLOOR * rms)
    bound = np.maximum(bound, 1e-30)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside tolerance; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return float(np.max(err / bound))


def oracle_ssd(inp: dict, headdim: int = 64, heads=None, nthreads: int = 0,
               discretization: str = "zoh"):
    """Oracle of the scan with step and decay shared per head on the inputs
    dict of ``ssd_scan`` (device tensors); ``heads`` optionally restricts to a
    subset of heads (heads are independent).  Returns (y, h_last) over the
    selected heads' channels."""
    x, dt, A, B, C = inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"]
    D, z, h0 = inp.get("D"), inp.get("z"), inp.get("h0")
    if heads is not None:
        hidx = torch.as_tensor(heads, device=x.device, dtype=torch.long)
        cidx = (hidx[:, None] * headdim + torch.arange(headdim, device=x.device)).reshape(-1)
        x = x.index_select(2, cidx)
        z = z.index_select(2, cidx) if z is not None else None
        D = D.index_select(0, cidx) if D is not None else None
        h0 = h0.index_select(1, cidx) if h0 is not None else None
        dt = dt.index_select(2, hidx)
        A = A.index_select(0, hidx)
    return oracle.scan_heads(to_f64(x), to_f64(dt), to_f64(A), to_f64(B), to_f64(C),
                             to_f64(D), to_f64(z), to_f64(h0), headdim=headdim,
                             nthreads=nthreads, discretization=discretization)
