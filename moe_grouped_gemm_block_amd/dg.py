"""ctypes binding of libdg.so (argument marshalling only).

The functions named like the C entry points take raw integers (device
addresses, sizes, a hipStream_t handle) and return the dg_status code.  The
torch-facing helpers below them only check dtypes / shapes / devices, pass
``data_ptr()`` values and the current stream, and raise on a non-zero status;
every step of the computation runs in the library's HIP kernels.

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DG_LIBRARY", os.path.join(_PKG, "libdg.so"))

DG_OUT_F32 = 0
DG_OUT_BF16 = 1
DG_IN_F32 = 0
DG_IN_BF16 = 1
DG_FP8_E4M3 = 0
DG_FP8_E5M2 = 1
DG_OK = 0
DG_ERR_INVALID_ARG = -1
DG_ERR_UNSUPPORTED = -2
DG_ERR_LAUNCH = -3

EXPORTED = ("dg_gemm_fp8_blockscaled", "dg_grouped_gemm_fp8", "dg_gemm_fp8_ex", "dg_gemm_fp8_ex_noalloc",
            "dg_grouped_gemm_fp8_ex", "dg_grouped_gemm_fp8_ex_counts", "dg_grouped_gemm_fp8_segments",
            "dg_quantize_fp8_blockscaled", "dg_status_string")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libdg.so once; raise if it is missing.

    torch is imported first when it is installed: torch's ROCm build carries
    its own HIP runtime, and libdg.so's dependency on the HIP runtime is then
    satisfied by that already-loaded copy.  Loaded the other way round, the
    process would hold two HIP runtimes (the system one for libdg.so, torch's
    for the tensors), and the library's runtime, initialised second, cannot
    use the GPU (its device queries fail).
    """
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m moe_grouped_gemm_block_amd.build` "
                "(there is no non-HIP fallback)")
        try:
            import torch  # noqa: F401  (one HIP runtime for torch and the library)
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.dg_gemm_fp8_blockscaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, vp]
        L.dg_gemm_fp8_blockscaled.restype = ci
        L.dg_grouped_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.dg_grouped_gemm_fp8.restype = ci
        L.dg_gemm_fp8_ex.argtypes = [vp, ci, vp, ci, vp, ci, vp, vp, i64, i64, i64, ci, vp]
        L.dg_gemm_fp8_ex.restype = ci
        L.dg_gemm_fp8_ex_noalloc.argtypes = [vp, ci, vp, ci, vp, ci, vp, vp, i64, i64, i64, ci, vp]
        L.dg_gemm_fp8_ex_noalloc.restype = ci
        L.dg_grouped_gemm_fp8_ex.argtypes = [vp, ci, vp, ci, vp, ci, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.dg_grouped_gemm_fp8_ex.restype = ci
        L.dg_grouped_gemm_fp8_ex_counts.argtypes = [vp, ci, vp, ci, vp, ci, vp, vp, vp, vp, ci, i64, i64, i64,
                                                    ci, vp]
        L.dg_grouped_gemm_fp8_ex_counts.restype = ci
        L.dg_grouped_gemm_fp8_segments.argtypes = [vp, ci, vp, vp, ci, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.dg_grouped_gemm_fp8_segments.restype = ci
        L.dg_quantize_fp8_blockscaled.argtypes = [vp, ci, vp, vp, i64, i64, ci, vp]
        L.dg_quantize_fp8_blockscaled.restype = ci
        L.dg_status_string.argtypes = [ci]
        L.dg_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- raw C names

def dg_gemm_fp8_blockscaled(A, sA, B, sB, C, M, N, K, out_dtype, stream) -> int:
    return lib().dg_gemm_fp8_blockscaled(A, sA, B, sB, C, M, N, K, out_dtype, stream)


def dg_grouped_gemm_fp8(A, sA, B, sB, C, group_offsets, num_groups, M_total, N, K,
                        out_dtype, stream) -> int:
    return lib().dg_grouped_gemm_fp8(A, sA, B, sB, C, group_offsets, num_groups, M_total,
                                     N, K, out_dtype, stream)


def dg_gemm_fp8_ex(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream) -> int:
    return lib().dg_gemm_fp8_ex(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream)


def dg_gemm_fp8_ex_noalloc(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream) -> int:
    return lib().dg_gemm_fp8_ex_noalloc(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream)


def dg_grouped_gemm_fp8_ex(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets, num_groups, M_total,
                           N, K, out_dtype, stream) -> int:
    return lib().dg_grouped_gemm_fp8_ex(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets, num_groups,
                                        M_total, N, K, out_dtype, stream)


def dg_grouped_gemm_fp8_ex_counts(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets, group_counts,
                                  num_groups, M_total, N, K, out_dtype, stream) -> int:
    return lib().dg_grouped_gemm_fp8_ex_counts(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets,
                                               group_counts, num_groups, M_total, N, K, out_dtype, stream)


def dg_grouped_gemm_fp8_segments(A, a_fmt, sA, B, b_fmt, sB, C, group_offsets, num_groups, M_total, N, K,
                                 out_dtype, stream) -> int:
    return lib().dg_grouped_gemm_fp8_segments(A, a_fmt, sA, B, b_fmt, sB, C, group_offsets, num_groups,
                                              M_total, N, K, out_dtype, stream)


def dg_quantize_fp8_blockscaled(X, in_dtype, Q, S, M, K, block_rows, stream) -> int:
    return lib().dg_quantize_fp8_blockscaled(X, in_dtype, Q, S, M, K, block_rows, stream)


def dg_status_string(status: int) -> str:
    return lib().dg_status_string(status).decode()


class DGError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {dg_status_string(status)} ({status})")
        self.status = status


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _check_fp8(t, name):
    torch = _torch()
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2):
        raise TypeError(f"{name} must be uint8 FP8 codes, float8_e4m3fn or float8_e5m2, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def operand_fmt(t, fmt, name) -> int:
    """FP8 format code of operand tensor t.  A float8 dtype names its format;
    uint8 codes take `fmt` ("e4m3" when None).  An explicit `fmt` that
    disagrees with a float8 dtype is an error (the bytes would otherwise be
    decoded in the wrong format)."""
    torch = _torch()
    implied = {torch.float8_e4m3fn: DG_FP8_E4M3, torch.float8_e5m2: DG_FP8_E5M2}.get(t.dtype)
    if fmt is None:
        return DG_FP8_E4M3 if implied is None else implied
    code = fmt_code(fmt)
    if implied is not None and code != implied:
        raise ValueError(f"{name} is {t.dtype} but its format is given as {fmt!r}")
    return code


def _check_f32(t, name, shape):
    torch = _torch()
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _out(C, rows, N, out_dtype, like):
    torch = _torch()
    dt = torch.float32 if out_dtype == DG_OUT_F32 else torch.bfloat16
    if C is None:
        return torch.empty((rows, N), dtype=dt, device=like.device)
    if C.dtype != dt or tuple(C.shape) != (rows, N) or not C.is_contiguous():
        raise ValueError("C has the wrong dtype, shape or layout")
    return C


def out_code(out_dtype) -> int:
    if out_dtype in (DG_OUT_F32, "f32", "float32"):
        return DG_OUT_F32
    if out_dtype in (DG_OUT_BF16, "bf16", "bfloat16"):
        return DG_OUT_BF16
    raise ValueError(f"unknown out_dtype {out_dtype!r}")


def fmt_code(fmt) -> int:
    if fmt in (DG_FP8_E4M3, "e4m3"):
        return DG_FP8_E4M3
    if fmt in (DG_FP8_E5M2, "e5m2"):
        return DG_FP8_E5M2
    raise ValueError(f"unknown FP8 format {fmt!r}")


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _sa_rows(sA, M, K):
    """Rows per A scale block implied by sA's shape: 128 ([ceil(M/128)][K/128])
    or 1 ([M][K/128]); the first wins where both fit (M <= 1)."""
    if tuple(sA.shape) == (-(-M // 128), -(-K // 128)):
        return 128
    if tuple(sA.shape) == (M, -(-K // 128)):
        return 1
    raise ValueError(f"sA has shape {tuple(sA.shape)}; expected {(-(-M // 128), -(-K // 128))} "
                     f"(128 x 128 blocks) or {(M, -(-K // 128))} (1 x 128 blocks)")


def gemm_fp8_blockscaled(A, sA, B, sB, out_dtype="bf16", C=None, stream=None, a_fmt=None, b_fmt=None):
    """C[M][N] = block-scaled A[M][K] x B (stored [N][K]) on the device; the
    operands' FP8 formats are "e4m3" or "e5m2" (None: from a float8 dtype,
    E4M3 for uint8 codes).  sA holds one scale per 128 x 128 block
    ([ceil(M/128)][K/128]) or per row and 128 columns ([M][K/128])."""
    _check_fp8(A, "A")
    _check_fp8(B, "B")
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    rows = _sa_rows(sA, M, K)
    _check_f32(sA, "sA", tuple(sA.shape))
    _check_f32(sB, "sB", (-(-N // 128), -(-K // 128)))
    code = out_code(out_dtype)
    C = _out(C, M, N, code, A)
    fa, fb = operand_fmt(A, a_fmt, "A"), operand_fmt(B, b_fmt, "B")
    if fa == DG_FP8_E4M3 and fb == DG_FP8_E4M3 and rows == 128:
        st = dg_gemm_fp8_blockscaled(A.data_ptr(), sA.data_ptr(), B.data_ptr(), sB.data_ptr(),
                                     C.data_ptr(), M, N, K, code, _stream(stream))
    else:
        st = dg_gemm_fp8_ex(A.data_ptr(), fa, sA.data_ptr(), rows, B.data_ptr(), fb, sB.data_ptr(),
                            C.data_ptr(), M, N, K, code, _stream(stream))
    if st != DG_OK:
        raise DGError(st, "dg_gemm_fp8_blockscaled")
    return C


def grouped_gemm_fp8(A, sA, B, sB, group_offsets, out_dtype="bf16", C=None, stream=None,
                     a_fmt=None, b_fmt=None, group_counts=None):
    """MoE grouped GEMM over contiguous 128-row-padded expert segments.
    group_counts (device int32 [G], optional): real rows per expert; the
    padding rows after them come out as zeros and skip the work where whole
    wave sub-tiles are padding (dg_grouped_gemm_fp8_ex_counts)."""
    torch = _torch()
    _check_fp8(A, "A")
    _check_fp8(B, "B")
    M_total, K = A.shape
    G, N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    rows = _sa_rows(sA, M_total, K)
    _check_f32(sA, "sA", tuple(sA.shape))
    _check_f32(sB, "sB", (G, -(-N // 128), -(-K // 128)))
    if (group_offsets.dtype != torch.int32 or not group_offsets.is_cuda
            or tuple(group_offsets.shape) != (G + 1,)):
        raise ValueError("group_offsets must be a device int32 tensor of G + 1 entries")
    code = out_code(out_dtype)
    C = _out(C, M_total, N, code, A)
    fa, fb = operand_fmt(A, a_fmt, "A"), operand_fmt(B, b_fmt, "B")
    if group_counts is not None:
        if (group_counts.dtype != torch.int32 or not group_counts.is_cuda
                or tuple(group_counts.shape) != (G,)):
            raise ValueError("group_counts must be a device int32 tensor of G entries")
        st = dg_grouped_gemm_fp8_ex_counts(A.data_ptr(), fa, sA.data_ptr(), rows, B.data_ptr(), fb,
                                           sB.data_ptr(), C.data_ptr(), group_offsets.data_ptr(),
                                           group_counts.data_ptr(), G, M_total, N, K, code, _stream(stream))
    elif fa == DG_FP8_E4M3 and fb == DG_FP8_E4M3 and rows == 128:
        st = dg_grouped_gemm_fp8(A.data_ptr(), sA.data_ptr(), B.data_ptr(), sB.data_ptr(),
                                 C.data_ptr(), group_offsets.data_ptr(), G, M_total, N, K, code,
                                 _stream(stream))
    else:
        st = dg_grouped_gemm_fp8_ex(A.data_ptr(), fa, sA.data_ptr(), rows, B.data_ptr(), fb, sB.data_ptr(),
                                    C.data_ptr(), group_offsets.data_ptr(), G, M_total, N, K, code,
                                    _stream(stream))
    if st != DG_OK:
        raise DGError(st, "dg_grouped_gemm_fp8")
    return C


def grouped_gemm_fp8_segments(A, sA, B, sB, group_offsets, out_dtype="bf16", C=None, stream=None,
                              a_fmt=None, b_fmt=None):
    """MoE grouped GEMM over packed (unpadded) expert segments with one A
    scale per row, sA [M_total][K/128]; meant for few rows per expert."""
    torch = _torch()
    _check_fp8(A, "A")
    _check_fp8(B, "B")
    M_total, K = A.shape
    G, N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    _check_f32(sA, "sA", (M_total, -(-K // 128)))
    _check_f32(sB, "sB", (G, -(-N // 128), -(-K // 128)))
    if (group_offsets.dtype != torch.int32 or not group_offsets.is_cuda
            or tuple(group_offsets.shape) != (G + 1,)):
        raise ValueError("group_offsets must be a device int32 tensor of G + 1 entries")
    code = out_code(out_dtype)
    C = _out(C, M_total, N, code, A)
    st = dg_grouped_gemm_fp8_segments(A.data_ptr(), operand_fmt(A, a_fmt, "A"), sA.data_ptr(), B.data_ptr(),
                                      operand_fmt(B, b_fmt, "B"), sB.data_ptr(), C.data_ptr(), group_offsets.data_ptr(),
                                      G, M_total, N, K, code, _stream(stream))
    if st != DG_OK:
        raise DGError(st, "dg_grouped_gemm_fp8_segments")
    return C


def quantize_fp8_blockscaled(X, block_rows=128, Q=None, S=None, stream=None):
    """E4M3 codes and FP32 block scales of X[M][K] (float32 or bfloat16), one
    scale per block_rows x 128 block (block_rows = 128 or 1)."""
    torch = _torch()
    if X.dtype == torch.float32:
        code = DG_IN_F32
    elif X.dtype == torch.bfloat16:
        code = DG_IN_BF16
    else:
        raise TypeError(f"X must be float32 or bfloat16, got {X.dtype}")
    if not X.is_cuda or not X.is_contiguous() or X.dim() != 2:
        raise ValueError("X must be a contiguous 2-D device tensor")
    M, K = X.shape
    if Q is None:
        Q = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty((-(-M // block_rows), K // 128), dtype=torch.float32, device=X.device)
    _check_fp8(Q, "Q")
    _check_f32(S, "S", (-(-M // block_rows), K // 128))
    if tuple(Q.shape) != (M, K):
        raise ValueError("Q must have the shape of X")
    st = dg_quantize_fp8_blockscaled(X.data_ptr(), code, Q.data_ptr(), S.data_ptr(), M, K, block_rows,
                                     _stream(stream))
    if st != DG_OK:
        raise DGError(st, "dg_quantize_fp8_blockscaled")
    return Q, S
