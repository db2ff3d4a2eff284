"""Child process of tests/test_gpu_stages.py (not collected by pytest).

Runs a fixed set of seeded GEMMs, one per kernel family and pipeline shape,
through the library named by DG_LIBRARY and saves every output's raw bytes
to the .npz file named on the command line.  The parent runs it once with
libdg.so and once with libdg_stages1.so (the same sources built with one LDS
stage) and compares the two files byte for byte."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from moe_grouped_gemm_block_amd import dg  # noqa: E402
from moe_grouped_gemm_block_amd import inputs as I  # noqa: E402

DEV = "cuda:0"


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def raw(C):
    return C.contiguous().view(torch.uint8).cpu().numpy().copy()


def dense(name, M, N, K, out, **kw):
    p = I.dense_problem(M, N, K, seed=M + 3 * N + K, out_dtype=out, block_log2_range=3.0, **kw)
    return name, raw(dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), out, a_fmt=p.a_fmt,
                                             b_fmt=p.b_fmt))


def main():
    lib = os.environ.get("DG_LIBRARY", dg.LIB_PATH)
    print(f"stages child: {os.path.basename(lib)}", flush=True)
    res = {}
    cases = [
        # shared-B 256 x 256 tile (4 and 4 K-blocks, the second partial)
        ("sb256_k512", 4096, 4096, 512, "bf16", {}), ("sb256_k400", 4096, 4096, 400, "f32", {}),
        # 128 x 512 tiles with a narrow last round; narrow tiles; split K
        ("t512_tail", 33 * 128, 1024, 1024, "bf16", {}), ("narrow", 1024, 4096, 640, "f32", {}),
        ("splitk", 256, 4096, 4096, "bf16", {}),
        # per-token A scales, E5M2
        ("rowscale", 300, 2048, 1024, "f32", {"sa_rows": 1}),
        ("e5m2", 512, 1024, 1024, "f32", {"a_fmt": "e5m2", "b_fmt": "e5m2"}),
        # few rows (its own per-wave pipeline)
        ("skinny64", 64, 4096, 2048, "bf16", {}), ("skinny17", 17, 1000, 384, "f32", {}),
    ]
    for name, M, N, K, out, kw in cases:
        k, v = dense(name, M, N, K, out, **kw)
        res[k] = v
    p = I.grouped_problem(8, 1024, 1024, 2048, seed=4, out_dtype="bf16")
    res["grouped"] = raw(dg.grouped_gemm_fp8(t(p.A), t(p.sA), t(p.B), t(p.sB), t(p.group_offsets), "bf16"))
    p = I.decode_problem(16, 1024, 1024, 64, seed=6)
    res["segments"] = raw(dg.grouped_gemm_fp8_segments(t(p.A), t(p.sA), t(p.B), t(p.sB), t(p.group_offsets),
                                                       "bf16"))
    torch.cuda.synchronize()
    np.savez(sys.argv[1], **res)
    print(f"  saved {len(res)} outputs", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
