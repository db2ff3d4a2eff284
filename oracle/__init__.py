"""CPU oracle for the FP8 block-scaled GEMM and the activation quantisation
that feeds it -- test infrastructure only.

Used by tests/, the smoke check and the benchmark's CPU-baseline leg; never by
the product path.
"""
from .blockscaled import (BLOCK, decode, decode_table, e4m3_value,  # noqa: F401
                          e5m2_value, gemm_blockscaled, grouped_gemm, tolerance)
from .quantize import encode_nearest, quantize_blockscaled  # noqa: F401
