"""Seeded synthetic workloads for the selective scan and the decode step.

This module only draws random inputs.  It holds none of the scan's arithmetic:
the distributions below are the input recipe, and both the HIP path and the
CPU oracle read the exact same bytes that it produces.

The pages measure on no public dataset; every workload is synthetic, with the
distributions of the benchmark configurations:

* ``A[d, n]      = -U(0.5, 1.5)``                    (fp32, real, negative)
* ``Dskip[d]     ~ N(0, 1)``                          (fp32)
* ``x, z[b,t,d]  ~ N(0, 1)``                          (rounded to the I/O dtype)
* ``delta[b,t,d] = softplus(0.5 * N(0, 1) + bias)``   (bias = -3, or per channel
  ``bias_d ~ U(-6, -1)`` for the long-context workload; rounded to I/O dtype)
* ``B, C[b,t,n]  ~ N(0, 1)``                          (rounded to the I/O dtype)
* ``h0 = 0`` for the scan; the decode state is ``h[b,d,n] ~ N(0, 1)`` (fp32).

Inputs of the scan with step and decay shared per head (``make_ssd_inputs``;
heads of 64 channels, Mamba-2-like layer of 80 heads and 128 states): the
same distributions drawn per head instead of per channel,
``A[h] = -U(0.5, 1.5)`` and ``dt[b,t,h] = softplus(0.5 * N(0, 1) - 3)``.

Inputs of the fused scan (prologue + scan; ``make_fused_inputs``): the raw
block inputs before the causal depthwise convolution and the softplus:

* ``x_raw[b,t,d] ~ N(0, 1)`` (I/O dtype), taps ``conv_w[d,k] ~ U(-0.5, 0.5)``
  and ``conv_b[d] ~ U(-0.1, 0.1)`` (fp32, width 4);
* ``delta_raw[b,t,d] = 0.5 * N(0, 1)`` (I/O dtype) and ``delta_bias[d] = -3``
  (or the per-channel ``U(-6, -1)`` bias), so that
  ``softplus(delta_raw + delta_bias)`` has the distribution of ``delta`` above.

Every tensor has its own seed ``1_000_000 * workload.seed_id + 1_000 * layer + k``
with ``k`` = 0 A, 1 Dskip, 2 x, 3 delta noise, 4 z, 5 B, 6 C, 7 delta bias,
8 initial decode state, 9 x_raw, 10 conv taps, 11 conv bias, 12 delta_raw.  Values are drawn in fp32 and rounded to bf16 by
round-to-nearest-even (torch's ``.to(torch.bfloat16)``).  The small fp32
workload is drawn on the CPU so that CPU-only tests see the same bytes as the
GPU tests; the large ones are drawn with a generator on the target device.
"""
from __future__ import annotations

import dataclasses

import torch
import torch.nn.functional as F

(K_A, K_DSKIP, K_X, K_DELTA, K_Z, K_B, K_C, K_BIAS, K_HINIT, K_XRAW, K_CONVW, K_CONVB,
 K_DRAW, K_ACH) = range(14)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    kind: str            # "scan", "decode" or "ssd" (step and decay per head)
    batch: int
    seqlen: int          # 1 for decode
    dim: int
    dstate: int
    io_dtype: torch.dtype
    layers: int = 1
    per_channel_bias: bool = False
    cpu_draw: bool = False
    headdim: int = 0     # channels per head ("ssd" workloads)

    @property
    def elements(self) -> int:
        """B*L*D*N per layer (the unit of the throughput metric)."""
        return self.batch * self.seqlen * self.dim * self.dstate

    @property
    def io_bytes(self) -> int:
        return 2 if self.io_dtype == torch.bfloat16 else 4

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move per layer: x, delta, z in and y out
        ([b, L, d]); B, C in ([b, L, n]); A and Dskip (fp32).  The decode
        step also reads and writes its fp32 state [b, d, n]."""
        s = self.io_bytes
        b, L, d, n = self.batch, self.seqlen, self.dim, self.dstate
        if self.kind == "ssd":
            # x, z in and y out ([b, L, d]); dt ([b, L, heads]); B, C; A [heads], Dskip
            heads = d // self.headdim
            return b * L * (3 * d + heads + 2 * n) * s + 4 * heads + 4 * d
        total = b * L * (4 * d + 2 * n) * s + 4 * d * n + 4 * d
        if self.kind == "decode":
            total += 2 * 4 * b * d * n
        return total


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_b1_l256_d64", 0, "scan", 1, 256, 64, 16, torch.float32,
                 cpu_draw=True),
        Workload("mamba130m_b8_l2048_d1536", 1, "scan", 8, 2048, 1536, 16, torch.bfloat16),
        Workload("mamba2p8b_b4_l4096_d5120", 2, "scan", 4, 4096, 5120, 16, torch.bfloat16),
        Workload("longctx_b1_l262144_d4096", 3, "scan", 1, 262144, 4096, 16,
                 torch.bfloat16, per_channel_bias=True),
        Workload("decode_b256_d5120_64layers", 4, "decode", 256, 1, 5120, 16,
                 torch.bfloat16, layers=64),
        Workload("mamba2_2p7b_b4_l4096_h80_p64_n128", 5, "ssd", 4, 4096, 5120, 128,
                 torch.bfloat16, headdim=64),
    ]
}
TINY = WORKLOADS["tiny_f32_b1_l256_d64"]
MAMBA_130M = WORKLOADS["mamba130m_b8_l2048_d1536"]
MAMBA_2P8B = WORKLOADS["mamba2p8b_b4_l4096_d5120"]
LONG_CTX = WORKLOADS["longctx_b1_l262144_d4096"]
DECODE_64L = WORKLOADS["decode_b256_d5120_64layers"]
SSD_2P7B = WORKLOADS["mamba2_2p7b_b4_l4096_h80_p64_n128"]


def seed(w: Workload, layer: int, k: int) -> int:
    return 1_000_000 * w.seed_id + 1_000 * layer + k


def _gen(w: Workload, layer: int, k: int, device) -> torch.Generator:
    dev = "cpu" if (w.cpu_draw or torch.device(device).type == "cpu") else device
    g = torch.Generator(device=dev)
    g.manual_seed(seed(w, layer, k))
    return g


def _draw(kind: str, shape, w: Workload, layer: int, k: int, device) -> torch.Tensor:
    g = _gen(w, layer, k, device)
    f = torch.randn if kind == "normal" else torch.rand
    t = f(shape, generator=g, device=g.device, dtype=torch.float32)
    return t.to(device)


def make_inputs(w: Workload, device="cpu", layer: int = 0,
                batch: int | None = None, seqlen: int | None = None,
                dim: int | None = None, dstate: int | None = None) -> dict:
    """Inputs of workload ``w`` (optionally with overridden sizes, which keeps
    the distributions and seeds), as tensors on ``device``.

    Scan: x, delta, z [b, L, d]; B, C [b, L, n] in the I/O dtype; A [d, n] and
    Dskip [d] fp32; h0 None.  Decode: the same with L squeezed out
    (x, delta, z [b, d]; B, C [b, n]) plus the fp32 state h [b, d, n]."""
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    n = w.dstate if dstate is None else dstate
    io = w.io_dtype
    shp = (b, d) if w.kind == "decode" else (b, L, d)
    shp_bc = (b, n) if w.kind == "decode" else (b, L, n)

    A = -(0.5 + _draw("uniform", (d, n), w, layer, K_A, device))
    Dskip = _draw("normal", (d,), w, layer, K_DSKIP, device)
    x = _draw("normal", shp, w, layer, K_X, device).to(io)
    noise = _draw("normal", shp, w, layer, K_DELTA, device)
    if w.per_channel_bias:
        bias = -6.0 + 5.0 * _draw("uniform", (d,), w, layer, K_BIAS, device)
        delta = F.softplus(0.5 * noise + bias)
    else:
        delta = F.softplus(0.5 * noise - 3.0)
    del noise
    delta = delta.to(io)
    z = _draw("normal", shp, w, layer, K_Z, device).to(io)
    B = _draw("normal", shp_bc, w, layer, K_B, device).to(io)
    C = _draw("normal", shp_bc, w, layer, K_C, device).to(io)
    out = dict(x=x, delta=delta, A=A.contiguous(), B=B, C=C, D=Dskip, z=z)
    if w.kind == "decode":
        out["h"] = _draw("normal", (b, d, n), w, layer, K_HINIT, device)
    else:
        out["h0"] = None
    return out


def make_channel_A(w: Workload, device="cpu", layer: int = 0, dim: int | None = None):
    """A with one value per channel, [dim] fp32, drawn like the per-state A:
    -(0.5 + U(0, 1))."""
    d = w.dim if dim is None else dim
    return -(0.5 + _draw("uniform", (d,), w, layer, K_ACH, device))


def make_fused_inputs(w: Workload, device="cpu", layer: int = 0, batch: int | None = None,
                      seqlen: int | None = None, dim: int | None = None,
                      d_conv: int = 4) -> dict:
    """Inputs of the fused scan: x_raw, conv_w [d, d_conv], conv_b [d],
    delta_raw, delta_bias [d], plus A, B, C, D, z of ``make_inputs`` (same
    seeds) and h0 None."""
    assert w.kind == "scan"
    base = make_inputs(w, device, layer, batch, seqlen, dim)
    b, L, d = base["x"].shape
    io = w.io_dtype
    x_raw = _draw("normal", (b, L, d), w, layer, K_XRAW, device).to(io)
    conv_w = (_draw("uniform", (d, d_conv), w, layer, K_CONVW, device) - 0.5).contiguous()
    conv_b = 0.2 * (_draw("uniform", (d,), w, layer, K_CONVB, device) - 0.5)
    delta_raw = (0.5 * _draw("normal", (b, L, d), w, layer, K_DRAW, device)).to(io)
    if w.per_channel_bias:
        delta_bias = -6.0 + 5.0 * _draw("uniform", (d,), w, layer, K_BIAS, device)
    else:
        delta_bias = torch.full((d,), -3.0, dtype=torch.float32, device=device)
    return dict(x_raw=x_raw, conv_w=conv_w, conv_b=conv_b, delta_raw=delta_raw,
                delta_bias=delta_bias, A=base["A"], B=base["B"], C=base["C"], D=base["D"],
                z=base["z"], h0=None)


def make_ssd_inputs(w: Workload, device="cpu", layer: int = 0, batch: int | None = None,
                    seqlen: int | None = None, nheads: int | None = None,
                    dstate: int | None = None) -> dict:
    """Inputs of the scan with step and decay shared per head: x, z
    [b, L, heads * headdim], dt [b, L, heads], B, C [b, L, n] in the I/O dtype;
    A [heads] and Dskip [heads * headdim] fp32; h0 None."""
    assert w.kind == "ssd" and w.headdim > 0
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    H = w.dim // w.headdim if nheads is None else nheads
    n = w.dstate if dstate is None else dstate
    d = H * w.headdim
    io = w.io_dtype
    A = -(0.5 + _draw("uniform", (H,), w, layer, K_A, device))
    Dskip = _draw("normal", (d,), w, layer, K_DSKIP, device)
    x = _draw("normal", (b, L, d), w, layer, K_X, device).to(io)
    dt = F.softplus(0.5 * _draw("normal", (b, L, H), w, layer, K_DELTA, device) - 3.0).to(io)
    z = _draw("normal", (b, L, d), w, layer, K_Z, device).to(io)
    B = _draw("normal", (b, L, n), w, layer, K_B, device).to(io)
    C = _draw("normal", (b, L, n), w, layer, K_C, device).to(io)
    return dict(x=x, dt=dt, A=A.contiguous(), B=B, C=C, D=Dskip, z=z, h0=None)
