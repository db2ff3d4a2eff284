"""MI355X-native FP8 (E4M3) GEMM with 128x128 block scales, dense and MoE-grouped.

The compute path is the C-ABI library ``libdg.so`` (hand-written HIP kernels
for gfx950); :mod:`moe_grouped_gemm_block_amd.dg` is its thin ctypes binding.
:mod:`moe_grouped_gemm_block_amd.inputs` builds seeded synthetic operands.
The binding is imported lazily so that the input generator works on hosts
without the built library.
"""

__all__ = ["dg", "inputs"]


def __getattr__(name):
    if name in ("dg", "inputs"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
