"""The single-stage build: libdg_stages1.so is libdg.so compiled with
DG_STAGES=1, i.e. every GEMM pipeline (shared-B tile, 128-row tiles, split
K, few rows, packed segments) loads a K-block into LDS only after the
previous one has been used.  The arithmetic and its order are unchanged, so
the two libraries must give identical bytes; a difference would point at a
race between the loads into one stage and the reads of the other (the
"drop to a single buffer" check of the DeepGEMM FP8 kernel write-up,
section 6.2).  Each library runs in a child process (tests/stages_child.py).
Needs a GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

from moe_grouped_gemm_block_amd import build, dg

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def run_child(lib, out):
    env = dict(os.environ, DG_LIBRARY=lib)
    for k in ("DG_FORCE_TILE", "DG_TAIL_TILE", "DG_SPLITK"):
        env.pop(k, None)
    r = subprocess.run([sys.executable, os.path.join(HERE, "stages_child.py"), out], env=env,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout, file=sys.stderr)
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]


def test_single_stage_build_gives_identical_bytes(tmp_path):
    assert os.path.exists(build.LIB_STAGES1), "libdg_stages1.so is not built"
    a, b = str(tmp_path / "two.npz"), str(tmp_path / "one.npz")
    run_child(dg.LIB_PATH, a)
    run_child(build.LIB_STAGES1, b)
    A, B = np.load(a), np.load(b)
    assert sorted(A.files) == sorted(B.files)
    for k in A.files:
        assert np.array_equal(A[k], B[k]), f"{k}: single-stage output differs"
        print(f"  {k}: {A[k].size} bytes identical", file=sys.stderr)
