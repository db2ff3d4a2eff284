"""Build libdg.so in-tree with hipcc for gfx950.

    python -m moe_grouped_gemm_block_amd.build

Host and device code are compiled in one hipcc invocation.  Packed FP32
instructions are disabled for the device code (the host pass warns that it
does not know the feature; that warning is harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdg.so")
SOURCES = ["dg_api.hip"]
ARCH = os.environ.get("DG_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core results in ordinary VGPRs: the FP32 rescale reads them
            # directly instead of copying each one out of an accumulation register
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", INCLUDE, "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES],
            *(extra or []), "-o", out]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
