"""Selective state-space scan (the S6 core of Mamba) on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/ssm.h`` (library
``libssm.so``, built in-tree by ``selective_state_space_44_amd._build``).
This module only checks and marshals arguments: tensors are PyTorch device
tensors (PyTorch provides device memory and the current stream); every step
of the computation runs in the HIP kernels.  There is no fallback path: if
the library is missing or a request has no kernel, calls raise.

Entry points: ``scan_fwd`` (the scan; A per channel and the Euler rule as
options; d_state 16, 32, 64, 128), ``scan_fwd_fused`` (with the causal
conv1d + softplus prologue), ``scan_bwd`` and the autograd wrapper
``SelectiveScan`` (all input gradients), ``decode_step`` (one recurrent step
on a resident state), ``ssd_scan`` (step and decay shared per head of 64
channels, on the matrix cores) and its backward ``ssd_bwd``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["scan_fwd", "scan_fwd_noalloc", "scan_fwd_fused", "scan_bwd", "SelectiveScan", "decode_step", "ssd_scan",
           "ssd_bwd",
           "scan_plan", "scan_workspace_bytes", "scan_bwd_workspace_bytes", "load_library",
           "LIB_PATH", "SsmError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssm.so")

SSM_DTYPE_F32 = 0
SSM_DTYPE_BF16 = 1
SSM_DISC_ZOH = 0
SSM_DISC_EULER = 1
SSM_OK = 0
SSM_ERR_INVALID_ARG = 1
SSM_ERR_UNSUPPORTED = 2
SSM_ERR_WORKSPACE = 3
SSM_ERR_HIP = 4
SSM_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/ssm.h declares, with its ctypes signature.
_i64, _vp, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "ssm_abi_version": (_int, []),
    "ssm_status_str": (ctypes.c_char_p, [_int]),
    "ssm_scan_plan": (_int, [_i64, _i64, _i64, _i64, _int, ctypes.POINTER(_int),
                             ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "ssm_scan_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64, _int, _int]),
    "ssm_scan_fwd": (_int, [_i64, _i64, _i64, _i64, _int] + [_vp] * 10 + [_vp, _sz, _vp]),
    "ssm_scan_fwd_planned": (_int, [_i64, _i64, _i64, _i64, _int] + [_vp] * 10
                             + [_vp, _sz, _int, _int, _vp]),
    "ssm_scan_fwd_phase": (_int, [_i64, _i64, _i64, _i64, _int] + [_vp] * 10
                           + [_vp, _sz, _int, _int, _int, _vp]),
    "ssm_scan_fwd_noalloc": (_int, [_i64, _i64, _i64, _i64, _int] + [_vp] * 10
                             + [_int, _int, _vp]),
    "ssm_scan_fwd_ex": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _int, _int]
                        + [_vp] * 7 + [_vp, _sz, _int, _int, _vp]),
    "ssm_scan_fwd_fused": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _int, _int, _vp,
                                  _vp] + [_vp] * 8 + [_vp, _sz, _int, _int, _vp]),
    "ssm_decode_step": (_int, [_i64, _i64, _i64, _int] + [_vp] * 9 + [_vp]),
    "ssm_decode_step_ex": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _int, _int]
                           + [_vp] * 6),
    "ssm_scan_bwd_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64, _int]),
    "ssm_scan_bwd": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _int, _int]
                     + [_vp] * 15 + [_vp, _sz, _vp]),
    "ssm_ssd_fwd": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int] + [_vp] * 10
                    + [_vp, _sz, _vp]),
    "ssm_ssd_fwd_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64, _i64, _int]),
    "ssm_ssd_fwd_planned": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int] + [_vp] * 10
                            + [_int, _vp, _sz, _vp]),
    "ssm_ssd_bwd_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64, _i64, _int]),
    "ssm_ssd_bwd": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int] + [_vp] * 18
                    + [_vp, _sz, _vp]),
}

_lock = threading.Lock()
_lib = None


class SsmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


def load_library(path: str = LIB_PATH):
    """Load libssm.so (raises OSError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise OSError(f"{path} is missing: build it with "
                              "`python -m selective_state_space_44_amd._build`")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype, fn.argtypes = res, args
            _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load_library().ssm_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != SSM_OK:
        raise SsmError(status, what)


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return SSM_DTYPE_F32
    if dtype == torch.bfloat16:
        return SSM_DTYPE_BF16
    raise ValueError(f"unsupported I/O dtype {dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def scan_plan(batch: int, seqlen: int, dim: int, dstate: int = 16,
              dtype: torch.dtype = torch.bfloat16, with_phase: bool = False):
    """(waves_per_group, nchunks) that ``scan_fwd`` uses for these sizes; with
    ``with_phase`` also the phase value of its schedule (3: two-launch, 7:
    three-pass, as ``scan_fwd``'s ``phase`` takes them)."""
    g, k, ph = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load_library().ssm_scan_plan(batch, seqlen, dim, dstate, _io_code(dtype),
                                        ctypes.byref(g), ctypes.byref(k), ctypes.byref(ph)),
           "ssm_scan_plan")
    return (g.value, k.value, ph.value) if with_phase else (g.value, k.value)


def scan_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int = 16,
                         dtype: torch.dtype = torch.bfloat16, nchunks: int = 0) -> int:
    n = load_library().ssm_scan_workspace_bytes(batch, seqlen, dim, dstate, _io_code(dtype),
                                                nchunks)
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, return_last_state=False,
             waves_per_group: int = 0, nchunks: int = 0, out=None, workspace=None,
             phase: int = 0, discretization: str = "zoh"):
    """Selective scan.  x, delta, z: [batch, L, dim]; B, C: [batch, L, dstate]
    (all float32 or all bfloat16); A [dim, dstate], D [dim], h0
    [batch, dim, dstate] float32.  Returns y (and the final state when
    ``return_last_state``).  ``waves_per_group``/``nchunks`` override the
    automatic plan (0 = automatic).  ``phase`` 0 runs the whole scan in the
    schedule the plan prefers (``ssm_scan_fwd_planned``); 1, 2 or 3 enqueue
    the first, the second or both launches of the two-launch schedule, 5, 6
    or 7 those of the three-pass schedule (``ssm_scan_fwd_phase``); the
    phases of one scan must get the same ``workspace`` and ``out``.

    Variants (``ssm_scan_fwd_ex``): ``A`` of shape [dim] holds one value per
    channel shared by its states (then ``B``/``C`` fix dstate);
    ``discretization="euler"`` uses Bbar = delta*B instead of the zero-order
    hold.  Both run as one call (``phase`` must be 0), in the plan's schedule."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, seqlen, dim] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    batch, seqlen, dim = x.shape
    if discretization not in ("zoh", "euler"):
        raise ValueError("discretization must be 'zoh' or 'euler'")
    if not isinstance(A, torch.Tensor) or A.dim() not in (1, 2):
        raise ValueError("A must be a [dim, dstate] or [dim] tensor")
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a [batch, seqlen, dstate] tensor")
    per_channel = A.dim() == 1
    dstate = B.shape[2] if per_channel else A.shape[1]
    variant = per_channel or discretization != "zoh"
    if variant and phase != 0:
        raise ValueError("the A-per-channel and Euler variants run as one call (phase 0)")
    if phase not in (0, 1, 2, 3, 5, 6, 7):
        raise ValueError("phase must be 0 (the plan's schedule), 1, 2 or 3 (two-launch "
                         "schedule) or 5, 6 or 7 (three-pass schedule)")
    io = x.dtype
    code = _io_code(io)
    _require(x, "x", (batch, seqlen, dim), io, device)
    _require(delta, "delta", (batch, seqlen, dim), io, device)
    _require(A, "A", (dim,) if per_channel else (dim, dstate), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    if delta is None or B is None or C is None:
        raise ValueError("delta, B and C are required")
    y = out if out is not None else torch.empty_like(x)
    _require(y, "out", (batch, seqlen, dim), io, device)
    h_last = (torch.empty((batch, dim, dstate), dtype=torch.float32, device=device)
              if return_last_state else None)
    lib = load_library()
    nbytes = lib.ssm_scan_workspace_bytes(batch, seqlen, dim, dstate, code, nchunks)
    if nbytes < 0:
        raise ValueError("invalid sizes")
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if variant:
        st = lib.ssm_scan_fwd_ex(batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta),
                                 _ptr(A), int(per_channel),
                                 SSM_DISC_EULER if discretization == "euler" else SSM_DISC_ZOH,
                                 _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
                                 _ptr(h_last), _ptr(workspace), ws_bytes, int(waves_per_group),
                                 int(nchunks), _stream(device))
        _check(st, "ssm_scan_fwd_ex")
        return (y, h_last) if return_last_state else y
    if phase == 0:
        st = lib.ssm_scan_fwd_planned(batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta),
                                      _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(y), _ptr(h_last), _ptr(workspace), ws_bytes,
                                      int(waves_per_group), int(nchunks), _stream(device))
        _check(st, "ssm_scan_fwd_planned")
    else:
        st = lib.ssm_scan_fwd_phase(batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta),
                                    _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                    _ptr(y), _ptr(h_last), _ptr(workspace), ws_bytes,
                                    int(waves_per_group), int(nchunks), int(phase),
                                    _stream(device))
        _check(st, "ssm_scan_fwd_phase")
    return (y, h_last) if return_last_state else y


def scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, *, out,
                     h_last=None, waves_per_group: int = 0, nchunks: int = 0):
    """``ssm_scan_fwd_noalloc``: the scan of ``scan_fwd`` (per-state A, zero-
    order hold) with its chunk-carry workspace in the library's device scratch
    array, so that the call allocates nothing: the caller passes the output
    ``out`` [batch, L, dim] and, optionally, ``h_last`` [batch, dim, dstate]
    float32.  Raises SsmError(SSM_ERR_WORKSPACE) when the plan's workspace
    exceeds SSM_NOALLOC_SCRATCH_BYTES.  Calls that overlap on one GPU race on
    the scratch array."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, seqlen, dim] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    batch, seqlen, dim = x.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a [dim, dstate] tensor")
    dstate = A.shape[1]
    io = x.dtype
    code = _io_code(io)
    _require(x, "x", (batch, seqlen, dim), io, device)
    _require(delta, "delta", (batch, seqlen, dim), io, device)
    _require(A, "A", (dim, dstate), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    _require(out, "out", (batch, seqlen, dim), io, device)
    _require(h_last, "h_last", (batch, dim, dstate), torch.float32, device)
    if delta is None or B is None or C is None or out is None:
        raise ValueError("delta, B, C and out are required")
    st = load_library().ssm_scan_fwd_noalloc(
        batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
        _ptr(D), _ptr(z), _ptr(h0), _ptr(out), _ptr(h_last), int(waves_per_group),
        int(nchunks), _stream(device))
    _check(st, "ssm_scan_fwd_noalloc")
    return out


def ssd_scan(x, dt, A, B, C, D=None, z=None, h0=None, return_last_state=False,
             discretization: str = "zoh", out=None, nsplit: int = 0, workspace=None):
    """Scan with the step and decay rate shared by each head
    (``ssm_ssd_fwd_planned``).  x, z: [batch, L, nheads * headdim]; dt:
    [batch, L, nheads]; B, C: [batch, L, dstate] (all bfloat16); A [nheads],
    D [nheads * headdim], h0 [batch, nheads * headdim, dstate] float32.
    headdim = x.shape[2] // dt.shape[2].  ``nsplit`` sequence segments (0 =
    automatic, 1 = none).  Returns y (and the final state when
    ``return_last_state``)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, seqlen, dim] tensor")
    if not isinstance(dt, torch.Tensor) or dt.dim() != 3:
        raise ValueError("dt must be a [batch, seqlen, nheads] tensor")
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a [batch, seqlen, dstate] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    if discretization not in ("zoh", "euler"):
        raise ValueError("discretization must be 'zoh' or 'euler'")
    batch, seqlen, dim = x.shape
    nheads = dt.shape[2]
    if nheads == 0 or dim % nheads:
        raise ValueError("x's channels must split evenly into dt's heads")
    headdim = dim // nheads
    dstate = B.shape[2]
    io = x.dtype
    code = _io_code(io)
    _require(x, "x", (batch, seqlen, dim), io, device)
    _require(dt, "dt", (batch, seqlen, nheads), io, device)
    _require(A, "A", (nheads,), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    if A is None or C is None:
        raise ValueError("A and C are required")
    y = out if out is not None else torch.empty_like(x)
    _require(y, "out", (batch, seqlen, dim), io, device)
    h_last = (torch.empty((batch, dim, dstate), dtype=torch.float32, device=device)
              if return_last_state else None)
    lib = load_library()
    nbytes = lib.ssm_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, int(nsplit))
    if nbytes < 0:
        raise ValueError("invalid sizes")
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssm_ssd_fwd_planned(
        batch, seqlen, nheads, headdim, dstate, code,
        SSM_DISC_EULER if discretization == "euler" else SSM_DISC_ZOH, _ptr(x), _ptr(dt),
        _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
        int(nsplit), _ptr(workspace), ws_bytes, _stream(device))
    _check(st, "ssm_ssd_fwd_planned")
    return (y, h_last) if return_last_state else y


def ssd_bwd(x, dt, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None,
            discretization: str = "zoh", need_dD: bool = True, need_dh0: bool = True,
            workspace=None):
    """Gradients of ``ssd_scan`` for upstream dy (and dh_last).  Returns a dict:
    dx, dz (None without z), ddt, dB, dC in the I/O dtype; dA [nheads], dD
    (None unless need_dD), dh0 (None unless need_dh0) in float32."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, seqlen, dim] tensor")
    if not isinstance(dt, torch.Tensor) or dt.dim() != 3:
        raise ValueError("dt must be a [batch, seqlen, nheads] tensor")
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a [batch, seqlen, dstate] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    if discretization not in ("zoh", "euler"):
        raise ValueError("discretization must be 'zoh' or 'euler'")
    batch, seqlen, dim = x.shape
    nheads = dt.shape[2]
    if nheads == 0 or dim % nheads:
        raise ValueError("x's channels must split evenly into dt's heads")
    headdim, dstate = dim // nheads, B.shape[2]
    io = x.dtype
    code = _io_code(io)
    _require(x, "x", (batch, seqlen, dim), io, device)
    _require(dt, "dt", (batch, seqlen, nheads), io, device)
    _require(A, "A", (nheads,), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    _require(dy, "dy", (batch, seqlen, dim), io, device)
    _require(dh_last, "dh_last", (batch, dim, dstate), torch.float32, device)
    if A is None or C is None or dy is None:
        raise ValueError("A, C and dy are required")
    g = {
        "dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
        "dz": torch.empty_like(x) if z is not None else None,
        "dA": torch.empty_like(A), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
        "dD": torch.empty(dim, dtype=torch.float32, device=device) if need_dD else None,
        "dh0": (torch.empty((batch, dim, dstate), dtype=torch.float32, device=device)
                if need_dh0 else None),
    }
    lib = load_library()
    nbytes = lib.ssm_ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, code)
    if nbytes < 0:
        raise ValueError("invalid sizes")
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssm_ssd_bwd(batch, seqlen, nheads, headdim, dstate, code,
                         SSM_DISC_EULER if discretization == "euler" else SSM_DISC_ZOH,
                         _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddt"]),
                         _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                         _ptr(g["dz"]), _ptr(g["dh0"]), _ptr(workspace), ws_bytes,
                         _stream(device))
    _check(st, "ssm_ssd_bwd")
    return g


def scan_fwd_fused(x_raw, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D=None, z=None,
                   h0=None, *, conv_silu: bool, return_last_state=False,
                   waves_per_group: int = 0, nchunks: int = 0, out=None, workspace=None):
    """Selective scan with its prologue fused: x = act(causal depthwise
    conv1d(x_raw) + conv_b), delta = softplus(delta_raw + delta_bias), then the
    scan of ``scan_fwd``.  x_raw, delta_raw: [batch, L, dim] (float32 or
    bfloat16); conv_w [dim, d_conv] float32 (d_conv <= 4, the last tap
    multiplies the current step); conv_b, delta_bias [dim] float32 or None;
    ``conv_silu`` selects SiLU after the convolution (keyword, no default)."""
    if not isinstance(x_raw, torch.Tensor) or x_raw.dim() != 3:
        raise ValueError("x_raw must be a [batch, seqlen, dim] tensor")
    device = x_raw.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    batch, seqlen, dim = x_raw.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a [dim, dstate] tensor")
    if not isinstance(conv_w, torch.Tensor) or conv_w.dim() != 2:
        raise ValueError("conv_w must be a [dim, d_conv] tensor")
    dstate = A.shape[1]
    d_conv = conv_w.shape[1]
    io = x_raw.dtype
    code = _io_code(io)
    _require(x_raw, "x_raw", (batch, seqlen, dim), io, device)
    _require(delta_raw, "delta_raw", (batch, seqlen, dim), io, device)
    _require(conv_w, "conv_w", (dim, d_conv), torch.float32, device)
    _require(conv_b, "conv_b", (dim,), torch.float32, device)
    _require(delta_bias, "delta_bias", (dim,), torch.float32, device)
    _require(A, "A", (dim, dstate), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    if delta_raw is None or B is None or C is None:
        raise ValueError("delta_raw, B and C are required")
    y = out if out is not None else torch.empty_like(x_raw)
    _require(y, "out", (batch, seqlen, dim), io, device)
    h_last = (torch.empty((batch, dim, dstate), dtype=torch.float32, device=device)
              if return_last_state else None)
    lib = load_library()
    nbytes = lib.ssm_scan_workspace_bytes(batch, seqlen, dim, dstate, code, nchunks)
    if nbytes < 0:
        raise ValueError("invalid sizes")
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssm_scan_fwd_fused(batch, seqlen, dim, dstate, code, _ptr(x_raw), _ptr(conv_w),
                                _ptr(conv_b), int(d_conv), int(bool(conv_silu)),
                                _ptr(delta_raw), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
                                _ptr(workspace), ws_bytes, int(waves_per_group), int(nchunks),
                                _stream(device))
    _check(st, "ssm_scan_fwd_fused")
    return (y, h_last) if return_last_state else y


def decode_step(h, x, delta, A, B, C, D=None, z=None, out=None, discretization: str = "zoh"):
    """One recurrent step.  h: [batch, dim, dstate] float32, updated in place;
    x, delta, z: [batch, dim]; B, C: [batch, dstate] (float32 or bfloat16);
    A [dim, dstate] (or [dim]: one value per channel), D [dim] float32.
    ``discretization="euler"`` uses Bbar = delta*B.  Returns y [batch, dim]."""
    if not isinstance(h, torch.Tensor) or h.dim() != 3:
        raise ValueError("h must be a [batch, dim, dstate] tensor")
    device = h.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    if discretization not in ("zoh", "euler"):
        raise ValueError("discretization must be 'zoh' or 'euler'")
    batch, dim, dstate = h.shape
    if not isinstance(x, torch.Tensor):
        raise ValueError("x must be a tensor")
    if not isinstance(A, torch.Tensor) or A.dim() not in (1, 2):
        raise ValueError("A must be a [dim, dstate] or [dim] tensor")
    per_channel = A.dim() == 1
    io = x.dtype
    code = _io_code(io)
    _require(h, "h", (batch, dim, dstate), torch.float32, device)
    _require(x, "x", (batch, dim), io, device)
    _require(delta, "delta", (batch, dim), io, device)
    _require(A, "A", (dim,) if per_channel else (dim, dstate), torch.float32, device)
    _require(B, "B", (batch, dstate), io, device)
    _require(C, "C", (batch, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, dim), io, device)
    if delta is None or B is None or C is None:
        raise ValueError("delta, B and C are required")
    y = out if out is not None else torch.empty_like(x)
    _require(y, "out", (batch, dim), io, device)
    lib = load_library()
    if per_channel or discretization != "zoh":
        st = lib.ssm_decode_step_ex(batch, dim, dstate, code, _ptr(h), _ptr(x), _ptr(delta),
                                    _ptr(A), int(per_channel),
                                    SSM_DISC_EULER if discretization == "euler" else SSM_DISC_ZOH,
                                    _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _stream(device))
        _check(st, "ssm_decode_step_ex")
        return y
    st = lib.ssm_decode_step(batch, dim, dstate, code, _ptr(h), _ptr(x), _ptr(delta), _ptr(A),
                             _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _stream(device))
    _check(st, "ssm_decode_step")
    return y


def scan_bwd_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int = 16,
                             dtype: torch.dtype = torch.bfloat16) -> int:
    n = load_library().ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, _io_code(dtype))
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None,
             discretization: str = "zoh", need_dD: bool = True, need_dh0: bool = True,
             workspace=None):
    """Gradients of the scan for upstream dy [batch, L, dim] (and dh_last
    [batch, dim, dstate] float32).  Inputs as ``scan_fwd``.  Returns a dict:
    dx, ddelta, dz (None without z) [batch, L, dim] and dB, dC [batch, L,
    dstate] in the I/O dtype; dA (shape of A), dD [dim] (None unless
    need_dD), dh0 [batch, dim, dstate] (None unless need_dh0) in float32."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, seqlen, dim] tensor")
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    batch, seqlen, dim = x.shape
    if discretization not in ("zoh", "euler"):
        raise ValueError("discretization must be 'zoh' or 'euler'")
    if not isinstance(A, torch.Tensor) or A.dim() not in (1, 2):
        raise ValueError("A must be a [dim, dstate] or [dim] tensor")
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a [batch, seqlen, dstate] tensor")
    per_channel = A.dim() == 1
    dstate = B.shape[2] if per_channel else A.shape[1]
    io = x.dtype
    code = _io_code(io)
    _require(x, "x", (batch, seqlen, dim), io, device)
    _require(delta, "delta", (batch, seqlen, dim), io, device)
    _require(A, "A", (dim,) if per_channel else (dim, dstate), torch.float32, device)
    _require(B, "B", (batch, seqlen, dstate), io, device)
    _require(C, "C", (batch, seqlen, dstate), io, device)
    _require(D, "D", (dim,), torch.float32, device)
    _require(z, "z", (batch, seqlen, dim), io, device)
    _require(h0, "h0", (batch, dim, dstate), torch.float32, device)
    _require(dy, "dy", (batch, seqlen, dim), io, device)
    _require(dh_last, "dh_last", (batch, dim, dstate), torch.float32, device)
    if delta is None or C is None or dy is None:
        raise ValueError("delta, C and dy are required")
    g = {
        "dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
        "dz": torch.empty_like(x) if z is not None else None,
        "dA": torch.empty_like(A), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
        "dD": torch.empty(dim, dtype=torch.float32, device=device) if need_dD else None,
        "dh0": (torch.empty((batch, dim, dstate), dtype=torch.float32, device=device)
                if need_dh0 else None),
    }
    lib = load_library()
    nbytes = lib.ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, code)
    if nbytes < 0:
        raise ValueError("invalid sizes")
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssm_scan_bwd(batch, seqlen, dim, dstate, code, _ptr(x), _ptr(delta), _ptr(A),
                          int(per_channel),
                          SSM_DISC_EULER if discretization == "euler" else SSM_DISC_ZOH,
                          _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy),
                          _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                          _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                          _ptr(g["dh0"]), _ptr(workspace), ws_bytes, _stream(device))
    _check(st, "ssm_scan_bwd")
    return g


class SelectiveScan(torch.autograd.Function):
    """Autograd wrapper: forward = ``scan_fwd`` (returns y and h_last),
    backward = ``scan_bwd``; both run the HIP kernels only.

    ``y, h_last = SelectiveScan.apply(x, delta, A, B, C, D, z, h0, discretization)``
    (D, z, h0 may be None)."""

    @staticmethod
    def forward(ctx, x, delta, A, B, C, D, z, h0, discretization="zoh"):
        y, h_last = scan_fwd(x, delta, A, B, C, D, z, h0, return_last_state=True,
                             discretization=discretization)
        ctx.save_for_backward(x, delta, A, B, C, D, z, h0)
        ctx.discretization = discretization
        return y, h_last

    @staticmethod
    def backward(ctx, dy, dh_last):
        x, delta, A, B, C, D, z, h0 = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        g = scan_bwd(x, delta, A, B, C, D, z, h0, dy=dy.contiguous(),
                     dh_last=None if dh_last is None else dh_last.contiguous(),
                     discretization=ctx.discretization,
                     need_dD=D is not None and ctx.needs_input_grad[5],
                     need_dh0=h0 is not None and ctx.needs_input_grad[7])
        return (g["dx"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"], g["dh0"],
                None)
