"""Plain fp64 CPU oracle for the selective state-space scan and decode step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls anything here, and nothing here imports the HIP library.

The arithmetic lives in ``oracle.c`` (compiled with gcc into
``liboracle.so``); this module only widens inputs to float64 numpy arrays and
calls it.  The page citations for every step are in the header of
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-shared", "-fPIC", "-std=c11"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``src`` with gcc into the shared library ``out``."""
    cmd = ["gcc", *GCC_FLAGS, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib):
    i64, dp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_scan.restype = c_int
    lib.oracle_scan.argtypes = [i64, i64, i64, i64] + [dp] * 10 + [c_int]
    lib.oracle_scan_ex.restype = c_int
    lib.oracle_scan_ex.argtypes = ([i64, i64, i64, i64, dp, dp, dp, c_int, c_int]
                                   + [dp] * 7 + [c_int])
    lib.oracle_scan_bwd_ex.restype = c_int
    lib.oracle_scan_bwd_ex.argtypes = ([i64, i64, i64, i64, dp, dp, dp, c_int, c_int]
                                       + [dp] * 15 + [c_int])
    lib.oracle_decode_step.restype = c_int
    lib.oracle_decode_step.argtypes = [i64, i64, i64] + [dp] * 9
    lib.oracle_conv1d.restype = c_int
    lib.oracle_conv1d.argtypes = [i64, i64, i64, i64, dp, dp, dp, c_int, dp]
    lib.oracle_delta_softplus.restype = c_int
    lib.oracle_delta_softplus.argtypes = [i64, i64, i64, dp, dp, dp]
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_zoh.restype = None
    lib.oracle_zoh.argtypes = [ctypes.c_double, ctypes.c_double,
                               ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(ctypes.c_double)]
    return lib


def load_library(path: str | None = None):
    """Load a compiled oracle library (building the default one if absent)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(a):
    """Widen any array-like (numpy or CPU torch tensor) to contiguous float64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: exact widening through float64
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def zoh(delta: float, a: float):
    """(Abar, Bbar/B) for one diagonal entry, from the compiled oracle."""
    lib = load_library()
    abar, bcoef = ctypes.c_double(), ctypes.c_double()
    lib.oracle_zoh(float(delta), float(a), ctypes.byref(abar), ctypes.byref(bcoef))
    return abar.value, bcoef.value


def scan(x, delta, A, B, C, D=None, z=None, h0=None, nthreads: int = 0, lib=None,
         discretization: str = "zoh"):
    """Selective scan in fp64.  Shapes: x, delta, z [b, L, d]; B, C [b, L, n];
    A [d, n] (or [d]: one value per channel shared by its states); D [d];
    h0 [b, d, n].  ``discretization`` is "zoh" or "euler" (Bbar = delta*B).
    Returns (y [b, L, d], h_last [b, d, n])."""
    lib = lib or load_library()
    x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
    D, z, h0 = _f64(D), _f64(z), _f64(h0)
    batch, seqlen, dim = x.shape
    assert discretization in ("zoh", "euler")
    per_channel = A.ndim == 1
    dstate = B.shape[2] if per_channel else A.shape[1]
    assert delta.shape == x.shape
    assert A.shape == ((dim,) if per_channel else (dim, dstate))
    assert B.shape == (batch, seqlen, dstate) and C.shape == B.shape
    assert D is None or D.shape == (dim,)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (batch, dim, dstate)
    y = np.zeros_like(x)
    h_last = np.zeros((batch, dim, dstate), dtype=np.float64)
    rc = lib.oracle_scan_ex(batch, seqlen, dim, dstate, _ptr(x), _ptr(delta), _ptr(A),
                            int(per_channel), int(discretization == "euler"),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
                            _ptr(h_last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan rejected its arguments (code {rc})")
    return y, h_last


def scan_heads(x, dt, A, B, C, D=None, z=None, h0=None, headdim: int = 64,
               nthreads: int = 0, lib=None, discretization: str = "zoh"):
    """Selective scan whose step size and decay rate are shared by each head of
    ``headdim`` consecutive channels (A reduced to one scalar per head, as the
    ihouse article's section on Mamba's evolution describes for Mamba-2).
    Shapes: x, z [b, L, H*P]; dt [b, L, H]; A [H]; B, C [b, L, n]; D [H*P];
    h0 [b, H*P, n].  Channel d = h*P + p takes dt[..., h] and A[h]; everything
    else is ``scan`` with A given per channel.  Returns (y, h_last)."""
    x, dt, A = _f64(x), _f64(dt), _f64(A)
    batch, seqlen, dim = x.shape
    assert headdim > 0 and dim % headdim == 0
    nheads = dim // headdim
    assert dt.shape == (batch, seqlen, nheads) and A.shape == (nheads,)
    delta = np.repeat(dt, headdim, axis=2)
    a_chan = np.repeat(A, headdim)
    return scan(x, delta, a_chan, B, C, D, z, h0, nthreads=nthreads, lib=lib,
                discretization=discretization)


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None,
             nthreads: int = 0, lib=None, discretization: str = "zoh"):
    """Gradients of the scan in fp64 for upstream dy [b, L, d] and optional
    dh_last [b, d, n].  Returns a dict with dx, ddelta, dz (None without z)
    [b, L, d]; dA (shape of A); dB, dC [b, L, n]; dD [d]; dh0 [b, d, n]."""
    lib = lib or load_library()
    x, delta, A, B, C, dy = map(_f64, (x, delta, A, B, C, dy))
    D, z, h0, dh_last = _f64(D), _f64(z), _f64(h0), _f64(dh_last)
    batch, seqlen, dim = x.shape
    assert discretization in ("zoh", "euler")
    per_channel = A.ndim == 1
    dstate = B.shape[2] if per_channel else A.shape[1]
    assert delta.shape == x.shape and dy.shape == x.shape
    assert A.shape == ((dim,) if per_channel else (dim, dstate))
    assert B.shape == (batch, seqlen, dstate) and C.shape == B.shape
    assert D is None or D.shape == (dim,)
    assert z is None or z.shape == x.shape
    for s in (h0, dh_last):
        assert s is None or s.shape == (batch, dim, dstate)
    g = dict(dx=np.zeros_like(x), ddelta=np.zeros_like(x), dA=np.zeros_like(A),
             dB=np.zeros_like(B), dC=np.zeros_like(C), dD=np.zeros(dim),
             dz=np.zeros_like(x) if z is not None else None,
             dh0=np.zeros((batch, dim, dstate)))
    rc = lib.oracle_scan_bwd_ex(batch, seqlen, dim, dstate, _ptr(x), _ptr(delta), _ptr(A),
                                int(per_channel), int(discretization == "euler"), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_last),
                                _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]),
                                int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd_ex rejected its arguments (code {rc})")
    return g


def scan_heads_bwd(x, dt, A, B, C, D=None, z=None, h0=None, dy=None, dh_last=None,
                   headdim: int = 64, nthreads: int = 0, lib=None,
                   discretization: str = "zoh"):
    """Gradients of ``scan_heads``: the per-channel backward of the scan with
    dt and A repeated over each head's channels; a parameter shared by a
    head's channels gets the sum of their gradients (chain rule).  Returns the
    dict of ``scan_bwd`` with ``ddt`` [b, L, H] and dA [H] in place of the
    per-channel ddelta and dA."""
    x, dt, A = _f64(x), _f64(dt), _f64(A)
    batch, seqlen, dim = x.shape
    assert headdim > 0 and dim % headdim == 0
    nheads = dim // headdim
    assert dt.shape == (batch, seqlen, nheads) and A.shape == (nheads,)
    g = scan_bwd(x, np.repeat(dt, headdim, axis=2), np.repeat(A, headdim), B, C, D, z, h0,
                 dy=dy, dh_last=dh_last, nthreads=nthreads, lib=lib,
                 discretization=discretization)
    g["ddt"] = g.pop("ddelta").reshape(batch, seqlen, nheads, headdim).sum(axis=3)
    g["dA"] = g["dA"].reshape(nheads, headdim).sum(axis=1)
    return g


def decode_step(h, x, delta, A, B, C, D=None, z=None, lib=None):
    """One recurrent step.  h [b, d, n] float64 numpy array, updated in place;
    x, delta, z [b, d]; B, C [b, n].  Returns y [b, d]."""
    lib = lib or load_library()
    assert isinstance(h, np.ndarray) and h.dtype == np.float64 and h.flags.c_contiguous
    x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
    D, z = _f64(D), _f64(z)
    batch, dim, dstate = h.shape
    y = np.zeros((batch, dim), dtype=np.float64)
    rc = lib.oracle_decode_step(batch, dim, dstate, _ptr(h), _ptr(x), _ptr(delta),
                                _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle_decode_step rejected its arguments (code {rc})")
    return y


def softplus(v: float) -> float:
    """softplus(v) = log(1 + exp(v)) from the compiled oracle."""
    return load_library().oracle_softplus(float(v))


def conv1d(x_raw, w, bias=None, silu: bool = False, lib=None):
    """Causal depthwise convolution over time.  x_raw [b, L, d]; w [d, d_conv]
    (tap d_conv-1 multiplies the current step); bias [d].  Returns [b, L, d]."""
    lib = lib or load_library()
    x_raw, w, bias = _f64(x_raw), _f64(w), _f64(bias)
    batch, seqlen, dim = x_raw.shape
    d_conv = w.shape[1]
    assert w.shape == (dim, d_conv) and (bias is None or bias.shape == (dim,))
    out = np.zeros_like(x_raw)
    rc = lib.oracle_conv1d(batch, seqlen, dim, d_conv, _ptr(x_raw), _ptr(w), _ptr(bias),
                           int(bool(silu)), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv1d rejected its arguments (code {rc})")
    return out


def delta_softplus(delta_raw, bias=None, lib=None):
    """delta = softplus(delta_raw + bias[d]).  delta_raw [b, L, d]."""
    lib = lib or load_library()
    delta_raw, bias = _f64(delta_raw), _f64(bias)
    batch, seqlen, dim = delta_raw.shape
    assert bias is None or bias.shape == (dim,)
    out = np.zeros_like(delta_raw)
    rc = lib.oracle_delta_softplus(batch, seqlen, dim, _ptr(delta_raw), _ptr(bias), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_delta_softplus rejected its arguments (code {rc})")
    return out


def scan_fused(x_raw, conv_w, conv_b, conv_silu, delta_raw, delta_bias, A, B, C, D=None, z=None,
               h0=None, nthreads: int = 0, lib=None):
    """The prologue (conv1d, softplus) followed by the scan, all in fp64.
    Returns (y, h_last, x, delta) with x and delta the prologue outputs."""
    lib = lib or load_library()
    x = conv1d(x_raw, conv_w, conv_b, conv_silu, lib=lib)
    delta = delta_softplus(delta_raw, delta_bias, lib=lib)
    y, h_last = scan(x, delta, A, B, C, D, z, h0, nthreads=nthreads, lib=lib)
    return y, h_last, x, delta
