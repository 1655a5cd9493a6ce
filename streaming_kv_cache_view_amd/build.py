"""Build the HIP library in-tree: streaming_kv_cache_view_amd/libfdattn.so (gfx950).

    python -m streaming_kv_cache_view_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfdattn.so")
SOURCES = ["fd_api.cpp", "fd_kernels.hip"]
ARCH = os.environ.get("FD_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def command(out: str = LIB, extra=()) -> list[str]:
    return [
        hipcc(), "-O3", "-std=c++17", "-fPIC", "-shared",
        f"--offload-arch={ARCH}",
        # packed fp32 VALU forms stay disabled (ordinary float code only)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in ordinary VGPRs: the softmax reads S and rescales O with VALU
        # instructions, which cannot address AGPRs; this avoids per-tile AGPR<->VGPR copies
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # device code never produces or tests NaN: lets fmaxf lower to a bare v_max / v_max3
        # (no canonicalising max per operand); host argument checks are unaffected
        "-Xarch_device", "-fno-honor-nans",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *extra,
        "-o", out,
    ]


def build(verbose: bool = True) -> str:
    cmd = command(LIB + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
