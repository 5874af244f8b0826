"""Build step of the HIP library: hipcc for gfx950 -> libssm.so (in-tree).

``build()`` always recompiles.  It is called by ``__graft_entry__.build()``
and can be run directly: ``python -m selective_state_space_44_amd._build``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")
SOURCES = ["ssm_abi.cpp", "ssm_scan.hip", "ssm_scan_wide.hip", "ssm_scan_bwd.hip", "ssm_decode.hip",
           "ssm_ssd.hip", "ssm_ssd_bwd.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for every HIP translation unit.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, build_dir: str, verbose: bool) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-x", "hip", "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB) -> str:
    """Compiles the sources in parallel (one hipcc per source), then links."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(lambda s: _compile(s, build_dir, verbose), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def asm(src: str = "ssm_scan.hip", out: str | None = None) -> str:
    """Device assembly of one source (for inspection)."""
    out = out or os.path.join(PKG, "_build", os.path.splitext(src)[0] + ".s")
    cmd = [hipcc(), *HIPCC_FLAGS, "-x", "hip", "-I", INCLUDE, "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
