"""C-ABI of libdg.so on the host: exports and argument validation (CPU only).

Every call below fails validation (or is empty work) and returns before any
HIP call, so no GPU is needed.  The fake device addresses are never
dereferenced.
"""
import ctypes
import glob
import os
import re
import subprocess
import sys

import pytest

from moe_grouped_gemm_block_amd import dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUP = dg.DG_OK, dg.DG_ERR_INVALID_ARG, dg.DG_ERR_UNSUPPORTED
P = 1 << 20          # a 16-byte aligned fake address, never dereferenced


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        names |= set(re.findall(r"\b(dg_\w+)\s*\(", src))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dg.LIB_PATH):
        from moe_grouped_gemm_block_amd import build
        build.build(verbose=False)
    return dg.lib()


def test_header_declares_the_entry_points():
    assert declared_functions() >= {"dg_gemm_fp8_blockscaled", "dg_grouped_gemm_fp8",
                                    "dg_gemm_fp8_ex", "dg_grouped_gemm_fp8_ex",
                                    "dg_quantize_fp8_blockscaled", "dg_status_string"}


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s+(dg_\w+)", out))
    assert declared_functions() <= exported
    assert set(dg.EXPORTED) == declared_functions()


def test_status_strings(L):
    for st in (OK, INVALID, UNSUP, dg.DG_ERR_LAUNCH):
        assert dg.dg_status_string(st).startswith("DG_")
    assert "unknown" in dg.dg_status_string(42)


def dense(A=P, sA=P, B=P, sB=P, C=P, M=256, N=256, K=256, out=1):
    return dg.dg_gemm_fp8_blockscaled(A, sA, B, sB, C, M, N, K, out, None)


def grouped(A=P, sA=P, B=P, sB=P, C=P, offs=P, G=4, M=512, N=256, K=256, out=1):
    return dg.dg_grouped_gemm_fp8(A, sA, B, sB, C, offs, G, M, N, K, out, None)


@pytest.mark.parametrize("kw,want", [
    (dict(A=None), INVALID), (dict(B=None), INVALID), (dict(sA=None), INVALID),
    (dict(sB=None), INVALID), (dict(C=None), INVALID),
    (dict(M=-1), INVALID), (dict(N=-8), INVALID), (dict(K=-128), INVALID),
    (dict(M=1 << 31), INVALID), (dict(K=1 << 40), INVALID),
    (dict(out=2), INVALID), (dict(out=-1), INVALID),
    (dict(A=P + 8), INVALID), (dict(B=P + 4), INVALID), (dict(C=P + 2), INVALID),
    (dict(sA=P + 2), INVALID), (dict(sB=P + 1), INVALID),
    (dict(K=200), UNSUP), (dict(K=72), UNSUP), (dict(K=1), UNSUP), (dict(K=(1 << 22) + 16), UNSUP),
    (dict(M=0), OK), (dict(N=0), OK), (dict(M=0, A=None, C=None), OK),
    (dict(M=0, K=144), OK), (dict(M=0, N=13), OK), (dict(N=0, K=16), OK),   # tails are supported
])
def test_dense_validation(L, kw, want):
    assert dense(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(G=0), INVALID), (dict(G=-3), INVALID), (dict(M=300), INVALID), (dict(M=-128), INVALID),
    (dict(offs=None), INVALID), (dict(offs=P + 2), INVALID), (dict(A=None), INVALID),
    (dict(out=7), INVALID), (dict(K=100), UNSUP), (dict(K=136), UNSUP), (dict(M=0, N=20, K=144), OK),
    (dict(M=0), OK), (dict(N=0), OK),
])
def test_grouped_validation(L, kw, want):
    assert grouped(**kw) == want


def dense_ex(fa=1, fb=1, rows=128, **kw):
    d = dict(A=P, sA=P, B=P, sB=P, C=P, M=256, N=256, K=256, out=1)
    d.update(kw)
    return dg.dg_gemm_fp8_ex(d["A"], fa, d["sA"], rows, d["B"], fb, d["sB"], d["C"], d["M"], d["N"],
                             d["K"], d["out"], None)


def grouped_ex(fa=1, fb=0, rows=128, **kw):
    d = dict(A=P, sA=P, B=P, sB=P, C=P, offs=P, G=4, M=512, N=256, K=256, out=1)
    d.update(kw)
    return dg.dg_grouped_gemm_fp8_ex(d["A"], fa, d["sA"], rows, d["B"], fb, d["sB"], d["C"], d["offs"],
                                     d["G"], d["M"], d["N"], d["K"], d["out"], None)


@pytest.mark.parametrize("rows", [128, 1])
@pytest.mark.parametrize("fa,fb,kw,want", [
    (2, 0, {}, INVALID), (0, -1, {}, INVALID), (1, 1, dict(A=None), INVALID), (1, 0, dict(K=200), UNSUP),
    (0, 1, dict(out=3), INVALID), (1, 1, dict(M=0), OK), (0, 1, dict(K=24), UNSUP),
    (0, 0, dict(sA=P + 2), INVALID), (0, 0, dict(sA=None), INVALID),
])
def test_general_entry_points_validation(L, fa, fb, rows, kw, want):
    assert dense_ex(fa, fb, rows, **kw) == want
    gkw = {k: v for k, v in kw.items() if k != "M"}
    if "M" not in kw:
        assert grouped_ex(fa, fb, rows, **gkw) == want
    assert grouped_ex(1, 1, rows, G=0) == INVALID and grouped_ex(7, 1, rows) == INVALID


@pytest.mark.parametrize("rows", [0, 2, 64, 127, 129, -1])
def test_general_entry_points_reject_scale_granularity(L, rows):
    assert dense_ex(0, 0, rows) == INVALID
    assert grouped_ex(0, 0, rows) == INVALID
    assert dense_ex(0, 0, rows, M=0) == INVALID        # checked before the empty-work shortcut


def segments(fa=0, fb=0, **kw):
    d = dict(A=P, sA=P, B=P, sB=P, C=P, offs=P, G=4, M=300, N=256, K=256, out=1)
    d.update(kw)
    return dg.dg_grouped_gemm_fp8_segments(d["A"], fa, d["sA"], d["B"], fb, d["sB"], d["C"], d["offs"],
                                           d["G"], d["M"], d["N"], d["K"], d["out"], None)


@pytest.mark.parametrize("fa,fb,kw,want", [
    (2, 0, {}, INVALID), (0, 5, {}, INVALID), (0, 0, dict(G=0), INVALID), (0, 0, dict(G=-1), INVALID),
    (0, 0, dict(offs=None), INVALID), (0, 0, dict(offs=P + 2), INVALID), (0, 0, dict(A=None), INVALID),
    (0, 0, dict(sA=P + 1), INVALID), (1, 1, dict(out=9), INVALID), (0, 0, dict(M=-5), INVALID),
    (0, 0, dict(K=100), UNSUP), (0, 0, dict(K=8), UNSUP), (0, 0, dict(M=0), OK), (1, 0, dict(N=0), OK),
])
def test_segments_validation(L, fa, fb, kw, want):
    assert segments(fa, fb, **kw) == want


def quant(X=P, dt=1, Q=P, S=P, M=256, K=256, R=128):
    return dg.dg_quantize_fp8_blockscaled(X, dt, Q, S, M, K, R, None)


@pytest.mark.parametrize("kw,want", [
    (dict(dt=2), INVALID), (dict(dt=-1), INVALID), (dict(R=64), INVALID), (dict(R=0), INVALID),
    (dict(X=None), INVALID), (dict(Q=None), INVALID), (dict(S=None), INVALID),
    (dict(X=P + 8), INVALID), (dict(Q=P + 4), INVALID), (dict(S=P + 2), INVALID),
    (dict(M=-1), INVALID), (dict(K=-128), INVALID), (dict(M=1 << 31), INVALID),
    (dict(K=200), UNSUP), (dict(K=1 << 23), UNSUP), (dict(K=64, R=1), UNSUP),
    (dict(M=0), OK), (dict(K=0), OK), (dict(M=0, X=None, Q=None, S=None), OK),
])
def test_quantize_validation(L, kw, want):
    assert quant(**kw) == want


def test_product_path_does_not_touch_the_oracle():
    """The package never imports the oracle, and the oracle never imports the package."""
    pkg = os.path.join(ROOT, "moe_grouped_gemm_block_amd")
    for f in glob.glob(os.path.join(pkg, "**", "*.py"), recursive=True):
        assert not re.search(r"^\s*(from|import)\s+oracle", open(f).read(), re.M), f
    for f in glob.glob(os.path.join(pkg, "csrc", "*")):
        assert "oracle" not in open(f).read(), f
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        assert "moe_grouped_gemm_block_amd" not in open(f).read(), f


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        dg.lib()


def test_operand_format_follows_float8_dtype():
    """The torch helpers take an operand's FP8 format from its float8 dtype
    and reject an explicit format that contradicts it (CPU tensors: only the
    dtype is looked at)."""
    import torch
    e4, e5, u8 = (torch.zeros(2, dtype=d) for d in (torch.float8_e4m3fn, torch.float8_e5m2, torch.uint8))
    assert dg.operand_fmt(e5, None, "A") == dg.DG_FP8_E5M2
    assert dg.operand_fmt(e4, None, "A") == dg.DG_FP8_E4M3
    assert dg.operand_fmt(u8, None, "A") == dg.DG_FP8_E4M3
    assert dg.operand_fmt(u8, "e5m2", "A") == dg.DG_FP8_E5M2
    assert dg.operand_fmt(e5, "e5m2", "B") == dg.DG_FP8_E5M2
    with pytest.raises(ValueError):
        dg.operand_fmt(e5, "e4m3", "A")
    with pytest.raises(ValueError):
        dg.operand_fmt(e4, dg.DG_FP8_E5M2, "B")


def test_binding_loads_one_hip_runtime():
    """With torch installed, the binding loads it before libdg.so, so the
    process holds one HIP runtime (torch's ROCm build carries its own; a
    second, system runtime initialised after it cannot use the GPU)."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from moe_grouped_gemm_block_amd import dg\n"
            "dg.lib()\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(sorted(libs))\n"
            "sys.exit(0 if len(libs) == 1 else 1)\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]


def test_counts_entry_point_validation(L):
    """dg_grouped_gemm_fp8_ex_counts: a null or misaligned count array is an
    argument error; everything else is checked as for dg_grouped_gemm_fp8_ex."""
    def call(counts=P, **kw):
        d = dict(A=P, sA=P, B=P, sB=P, C=P, offs=P, G=4, M=512, N=256, K=256, out=1, fa=0, fb=0, rows=128)
        d.update(kw)
        return dg.dg_grouped_gemm_fp8_ex_counts(d["A"], d["fa"], d["sA"], d["rows"], d["B"], d["fb"], d["sB"],
                                                d["C"], d["offs"], counts, d["G"], d["M"], d["N"], d["K"],
                                                d["out"], None)
    assert call(counts=None) == INVALID
    assert call(counts=P + 2) == INVALID
    assert call(K=200) == UNSUP
    assert call(G=0) == INVALID
    assert call(M=500) == INVALID                 # M_total not a multiple of 128
    assert call(N=0) == OK

