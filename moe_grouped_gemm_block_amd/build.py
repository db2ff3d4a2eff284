"""Build libdg.so in-tree with hipcc for gfx950.

    python -m moe_grouped_gemm_block_amd.build

Each source under csrc/ (the host side plus one translation unit per pair of
operand formats, see csrc/kernels.hpp) is compiled to an object in parallel,
then the objects are linked into libdg.so.  Packed FP32 instructions are
disabled for the device code (the host pass warns that it does not know the
feature; that warning is harmless).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdg.so")
LIB_STAGES1 = os.path.join(PKG, "libdg_stages1.so")
SOURCES = ["dg_api.hip", "kernels_e4m3.hip", "kernels_e4m3_e5m2.hip", "kernels_e5m2_e4m3.hip",
           "kernels_e5m2.hip"]
ARCH = os.environ.get("DG_OFFLOAD_ARCH", "gfx950")
HARMLESS = "packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def compile_command(src: str, obj: str, stages: int = 2) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", f"-DDG_STAGES={stages}",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core results in ordinary VGPRs: the FP32 rescale reads them
            # directly instead of copying each one out of an accumulation register
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if HARMLESS not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{errs}")
    return errs


def build(verbose: bool = True) -> str:
    """Build libdg.so and its single-stage twin libdg_stages1.so (the same
    library compiled with -DDG_STAGES=1: every GEMM pipeline with one LDS
    stage, a debugging aid whose results must equal libdg.so's bit for bit);
    returns the path of libdg.so."""
    with tempfile.TemporaryDirectory(prefix="dg_build_") as tmp:
        jobs_list = []
        for stages, lib in ((2, LIB), (1, LIB_STAGES1)):
            objs = [os.path.join(tmp, f"s{stages}_" + os.path.splitext(s)[0] + ".o") for s in SOURCES]
            jobs_list.append((lib, objs, [compile_command(s, o, stages) for s, o in zip(SOURCES, objs)]))
        cmds = [c for _, _, cs in jobs_list for c in cs]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = min(len(cmds), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            warnings = list(pool.map(_run, cmds))
        for lib, objs, _ in jobs_list:
            warnings.append(_run(link_command(objs, lib + ".tmp")))
    if verbose and any(w.strip() for w in warnings):
        print("\n".join(w for w in warnings if w.strip()), file=sys.stderr)
    for lib, _, _ in jobs_list:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    build()
