#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled GEMM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload I]
    python bench.py --op quantize [--block-rows 128|1]

A step is one GEMM call (dense or grouped) over one batch of seeded synthetic
operands already resident in HBM.  W untimed warm-up steps are followed by
exactly K timed steps, bracketed by torch.cuda.synchronize() on both sides.
Operand copies are rotated so that the working set of consecutive steps
exceeds the 256 MB Infinity Cache: every step reads its inputs from HBM.

One JSON line is printed on stdout.  `value` is throughput over the timed
region (TFLOP/s of algorithmic work = 2 * real_rows * N * K, or GB/s of
algorithmic bytes for the memory-bound skinny shape).  `roofline.achieved`
uses the kernel's average duration from HIP events recorded on the launch
stream around the timed steps.  `kernel_ms_eager` is the same kernel timed
with launches one by one after the timed region, for comparison with the
per-dispatch durations of a kernel trace (the committed profile summaries
list the profiled and the unprofiled figures side by side).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
on this host.

Workloads (seeded, synthetic; see inputs.make_config):
  1  dense 256^3, FP32 out                      (parity case)
  2  dense 4096^3, per-block magnitudes, BF16   (default)
  3  skinny 64 x 12288 x 4096, outliers, BF16   (HBM-bound)
  4  MoE 8 experts, N = K = 4096, top-2 uniform
  5  MoE 64 experts, N = K = 2048, top-2 Zipf(1.1)
  6  one decode step of workload 5's MoE: 128 tokens, packed segments,
     per-token A scales                        (HBM-bound)

--op quantize times the activation quantisation that produces A instead
(4096 x 4096 BF16 in, E4M3 codes and FP32 block scales out; HBM-bound).
--op torch-matmul times the vendor library's plain BF16 (or FP16) GEMM,
torch.matmul on 4096^3, as a reference point for the matrix cores' rate.

Clock settling: right before the timed region the same work is run,
untimed, for --settle-ms milliseconds (default 300; graph mode replays the
captured graph).  Under load the GPU's clock takes some 20-30 ms to reach
its sustained level (on 4096^3 the first ~200 launches from idle run up to
35 % slower than later ones), and capturing the graph leaves the GPU idle
for a while; without the settle phase a short timed region (20 steps of
0.1 ms) lands on that ramp.  --settle-ms 0 gives the cold figure.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS (% of FP8 MFMA peak); HBM GB/s for M≤64"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (no sparsity)
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense FP16 MFMA: the unit the products run on (exact FP8 -> FP16)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
INFINITY_CACHE = 256 << 20
HBM_BOUND = {3, 5, 6}        # workloads whose roofline is HBM bandwidth
GBS_VALUE = {3, 6}           # workloads whose `value` is GB/s (streaming B once)
QUANT_METRIC = "FP8 activation quantisation HBM GB/s (BF16 in, E4M3 + FP32 block scales out)"


def gemm_tflops(M: int, N: int, K: int, seconds: float) -> float:
    """Algorithmic throughput of an M x N x K GEMM: 2 M N K FLOP / time."""
    return 2.0 * M * N * K / seconds / 1e12


def intensity(M: int, N: int, K: int, elem_bytes: float) -> float:
    """FLOP per byte when A, B and C each cross memory once."""
    return 2.0 * M * N * K / ((M * K + K * N + M * N) * elem_bytes)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources and of the build script (its compiler flags shape the code)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "moe_grouped_gemm_block_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "moe_grouped_gemm_block_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str):
    """HBM bytes per step (all launches of one step) from the committed
    rocprofv3 counter summary, or None when it is missing or was taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload_name]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    return int(rec["hbm_bytes_per_step"])


def cpu_baseline(p, target_s: float = 12.0):
    """Time the oracle (as it stands) on rows of the same workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d["num_threads"] for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    M = p.M
    rng = np.random.default_rng(0)

    def run(rows):
        t = time.perf_counter()
        if p.grouped:
            oracle.grouped_gemm(p.A, p.sA, p.B, p.sB, p.group_offsets, rows=rows, sa_rows=p.sa_rows)
        else:
            oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, rows=rows, a_fmt=p.a_fmt, b_fmt=p.b_fmt,
                                    sa_rows=p.sa_rows)
        return time.perf_counter() - t

    calib = np.sort(rng.choice(M, size=min(M, 64), replace=False))
    dt = run(calib)
    n = int(min(M, max(64, len(calib) * target_s / max(dt, 1e-6))))
    rows = np.sort(rng.choice(M, size=n, replace=False)) if n < M else np.arange(M)
    dt = run(rows)
    flop = 2.0 * len(rows) * p.N * p.K
    if p.grouped:
        # pad rows cost the oracle as much as real ones; count only the real share
        flop *= p.real_rows / p.M
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{len(rows)} of {M} output rows (all {p.N} columns, K={p.K}) of workload "
                      f"{p.name}, float64 numpy/BLAS"}


def cpu_baseline_quant(x, block_rows: int, target_s: float = 10.0):
    """Time the quantisation oracle (as it stands) on rows of the same input."""
    import numpy as np

    import oracle
    M, K = x.shape
    step = block_rows                       # whole row blocks
    t = time.perf_counter()
    oracle.quantize_blockscaled(x[:step], block_rows)
    dt = time.perf_counter() - t
    n = int(min(M, max(step, step * round(target_s / max(dt, 1e-6)))))
    n = max(step, n - n % step)
    t = time.perf_counter()
    oracle.quantize_blockscaled(x[:n], block_rows)
    dt = time.perf_counter() - t
    nbytes = n * K * (2 + 1) + 4 * (n // block_rows) * (K // 128)
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {n} of {M} rows (all {K} columns) of the same input, numpy float64, "
                      "one thread (per-block Python loop)"}


def settle(launch, settle_ms: float, per_batch: int = 1):
    """Enqueue launch() back to back, untimed, for about settle_ms
    milliseconds of wall time (a synchronisation after every per_batch
    launches), so that the GPU clock has reached its level under sustained
    load.  Returns the number of launches."""
    import torch
    if settle_ms <= 0:
        return 0
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(per_batch):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    return n


def run_timed(step, K: int, W: int, use_graph: bool, settle_ms: float = 0.0):
    """W untimed warm-up steps, an untimed settle phase of about settle_ms
    right before the timed region (see settle()), then exactly K timed steps
    between torch.cuda.synchronize() calls.  step(i, stream_handle) enqueues
    step i.

    With use_graph the K timed steps are captured once into a HIP graph and
    the timed region is one replay of it: kernels of a few microseconds are
    otherwise paced by the host's launch rate rather than by the GPU.  The
    settle phase then replays the same graph (at least once).  Returns
    (wall ms per step, kernel ms per step from HIP events on the launch
    stream, per-step event times or None)."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    for i in range(W):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            h = torch.cuda.current_stream().cuda_stream
            for i in range(K):
                step(W + i, h)
        torch.cuda.synchronize()
        n = settle(lambda _: g.replay(), settle_ms) if settle_ms > 0 else 0
        if n == 0:
            g.replay()
            torch.cuda.synchronize()
        log(f"settle: {max(n, 1)} untimed replays of the {K}-step graph right before the timed one")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t_start = time.perf_counter()
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        per = None
        kern_ms = float(ev[0].elapsed_time(ev[1])) / K
    else:
        n = settle(lambda i: step(W + K + i, stream.cuda_stream), settle_ms, per_batch=16)
        if n:
            log(f"settle: {n} untimed steps right before the timed ones")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        t_start = time.perf_counter()
        for i in range(K):
            ev[i].record(stream)
            step(W + i, stream.cuda_stream)
        ev[K].record(stream)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])
        kern_ms = float(ev[0].elapsed_time(ev[K])) / K
    ms_step = (t_end - t_start) * 1e3 / K
    if per is None:
        log(f"kernel ms (HIP events, graph of {K} steps): mean {kern_ms:.4f}; wall ms/step {ms_step:.4f}")
    else:
        log(f"kernel ms (HIP events): mean {kern_ms:.4f}  p10 {np.percentile(per, 10):.4f}  "
            f"p50 {np.percentile(per, 50):.4f}  p90 {np.percentile(per, 90):.4f}; wall ms/step {ms_step:.4f}")
    return ms_step, kern_ms, per


def eager_kernel_ms(step, K: int, use_graph: bool):
    """Per-launch kernel time with the steps launched one by one (HIP events
    on the launch stream), measured after the timed region: the launch mode
    of a kernel trace's per-dispatch durations.  None when the timed region
    itself was eager."""
    if not use_graph:
        return None
    _, ms, _ = run_timed(step, min(K, 50), 5, False)
    return round(ms, 5)


def bench_torch_matmul(args):
    """The vendor library's plain GEMM on the same shape, for comparison:
    torch.matmul on BF16 (or FP16) operands, which runs hipBLASLt.  No FP8
    decode, no block scales: a reference point for the matrix cores' rate,
    not the block-scaled operation."""
    import torch
    dev = torch.device("cuda:0")
    M = N = K = 4096
    gen = torch.Generator(device="cpu").manual_seed(2)
    R = args.rotate or 8
    dt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    ops = [(torch.randn(M, K, generator=gen).to(dt).to(dev),
            torch.randn(K, N, generator=gen).to(dt).to(dev).t().contiguous().t(),   # stored N x K, as B
            torch.empty(M, N, dtype=dt, device=dev)) for _ in range(R)]

    def step(i, sh):                 # torch enqueues on its current stream, which is sh here
        a, b, c = ops[i % R]
        torch.matmul(a, b, out=c)

    ms_step, kern_ms, _ = run_timed(step, args.steps, args.warmup, not args.no_graph, args.settle_ms)
    flop = 2.0 * M * N * K
    achieved = flop / (kern_ms * 1e-3) / 1e12
    line = {"metric": f"vendor {args.dtype.upper()} GEMM TFLOPS (torch.matmul / hipBLASLt), same shape, for comparison",
            "value": round(flop / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
            "data": "synthetic",
            "config": {"workload": f"torch_matmul_4096_{args.dtype}", "M": M, "N": N, "K": K,
                       "operand_copies": R, "launch": "eager" if args.no_graph else "hip_graph"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "traffic": None},
            "cpu_baseline": None, "kernel_ms": round(kern_ms, 5)}
    print(json.dumps(line), flush=True)


def bench_quantize(args):
    import numpy as np
    import torch

    from moe_grouped_gemm_block_amd import dg
    dev = torch.device("cuda:0")
    dg.lib()
    M = K = 4096
    R_blk = args.block_rows
    rng = np.random.default_rng(2)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.repeat(np.repeat(np.exp2(rng.uniform(-4, 4, (M // 128, K // 128))).astype(np.float32),
                             128, axis=0), 128, axis=1)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    x_seen = xb.float().numpy()
    step_bytes = M * K * 2 + M * K + 4 * (-(-M // R_blk)) * (K // 128)
    R = args.rotate or max(1, -(-2 * INFINITY_CACHE // step_bytes))
    copies = []
    for _ in range(R):
        X = xb.to(dev)
        Q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        S = torch.empty((-(-M // R_blk), K // 128), dtype=torch.float32, device=dev)
        copies.append((X, Q, S))
    ptrs = [(X.data_ptr(), Q.data_ptr(), S.data_ptr()) for X, Q, S in copies]

    def step(i, sh):
        x, q, s = ptrs[i % R]
        st = dg.dg_quantize_fp8_blockscaled(x, dg.DG_IN_BF16, q, s, M, K, R_blk, sh)
        if st != dg.DG_OK:
            raise dg.DGError(st, "bench step")

    n = args.steps
    ms_step, kern_ms, _ = run_timed(step, n, args.warmup, not args.no_graph, args.settle_ms)
    kern_eager = eager_kernel_ms(step, n, not args.no_graph)
    name = f"quantize_{M}x{K}_bf16_{R_blk}x128"
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name)}
    cpu = None if args.no_cpu_baseline else cpu_baseline_quant(x_seen, R_blk)
    line = {"metric": QUANT_METRIC, "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e4m3",
            "data": "synthetic",
            "config": {"workload": name, "M": M, "K": K, "block_rows": R_blk, "seed": 2, "operand_copies": R,
                       "launch": "eager" if args.no_graph else "hip_graph"},
            "roofline": roof, "cpu_baseline": cpu, "kernel_ms": round(kern_ms, 5),
            "kernel_ms_eager": kern_eager}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--shape", default="", metavar="M,N,K",
                    help="a dense problem of this shape instead of a named workload (BF16 out, B ~ N(0, 0.02))")
    ap.add_argument("--rotate", type=int, default=0, help="operand copies (0 = enough to exceed the Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps one by one from Python instead of replaying a HIP graph")
    ap.add_argument("--op", choices=["gemm", "quantize", "torch-matmul"], default="gemm",
                    help="torch-matmul: the vendor BF16/FP16 GEMM on 4096^3, for comparison")
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default="bf16", help="operand type of --op torch-matmul")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed run of the step right before the timed region, so that the GPU clock has "
                         "reached its sustained level (0: none)")
    ap.add_argument("--a-scale", choices=["128x128", "1x128"], default="128x128",
                    help="A scale blocks of the GEMM: 128x128, or one per token and 128 columns")
    ap.add_argument("--counts", action="store_true",
                    help="grouped workloads: pass the real per-expert row counts "
                         "(dg_grouped_gemm_fp8_ex_counts: padding rows skipped where whole waves are padding)")
    ap.add_argument("--fmt", choices=["e4m3", "e5m2"], default="e4m3",
                    help="operand FP8 format of the dense workloads 1-3 (both operands)")
    ap.add_argument("--block-rows", type=int, default=128, choices=[1, 128],
                    help="--op quantize: rows per scale block")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and exit; "
                         "used to scale the HBM byte counters of the profiler")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_grouped_gemm_block_amd import dg
    from moe_grouped_gemm_block_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB x 5 (reads {n} B, writes {n} B per copy)")
        return
    if args.op == "quantize":
        bench_quantize(args)
        return
    if args.op == "torch-matmul":
        bench_torch_matmul(args)
        return
    dg.lib()

    t0 = time.perf_counter()
    sa_rows = 1 if args.a_scale == "1x128" else 128
    if args.shape:
        M, N, K = (int(v) for v in args.shape.split(","))
        p = I.dense_problem(M, N, K, seed=0, out_dtype="bf16", b_std=0.02, a_fmt=args.fmt, b_fmt=args.fmt,
                            sa_rows=sa_rows, name=f"dense_{M}x{N}x{K}_{args.fmt}")
    else:
        p = I.make_config(args.workload, fmt=args.fmt, sa_rows=sa_rows)
    # memory-bound: few rows (the few-rows kernel streams B once) or the decode step
    hbm_bound = (p.M <= 64 and not p.grouped) if args.shape else args.workload in HBM_BOUND
    gbs_value = hbm_bound if args.shape else args.workload in GBS_VALUE
    log(f"generated {p.name} in {time.perf_counter() - t0:.1f}s: M={p.M} N={p.N} K={p.K} "
        f"G={p.G} real_rows={p.real_rows}")

    step_bytes = p.algorithmic_bytes()
    R = args.rotate or max(1, -(-2 * INFINITY_CACHE // step_bytes))
    cdt = torch.float32 if p.out_dtype == "f32" else torch.bfloat16
    host = {k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in
            dict(A=p.A, sA=p.sA, B=p.B, sB=p.sB).items()}
    if p.grouped:
        host["offs"] = torch.from_numpy(p.group_offsets.astype(np.int32))
    use_counts = args.counts and p.grouped and not p.packed
    if use_counts:
        host["counts"] = torch.from_numpy(p.group_counts.astype(np.int32))
    copies = []
    for _ in range(R):
        d = {k: v.to(dev) for k, v in host.items()}
        d["C"] = torch.empty((p.M, p.N), dtype=cdt, device=dev)
        copies.append(d)
    log(f"{R} operand copies resident ({R * step_bytes / 2**20:.0f} MiB)")
    code = dg.out_code(p.out_dtype)
    ptrs = [{k: v.data_ptr() for k, v in d.items()} for d in copies]
    plain = p.a_fmt == "e4m3" and p.b_fmt == "e4m3" and p.sa_rows == 128
    fa, fb = dg.fmt_code(p.a_fmt), dg.fmt_code(p.b_fmt)

    def step(i, sh):
        d = ptrs[i % R]
        if use_counts:
            st = dg.dg_grouped_gemm_fp8_ex_counts(d["A"], fa, d["sA"], p.sa_rows, d["B"], fb, d["sB"], d["C"],
                                                  d["offs"], d["counts"], p.G, p.M, p.N, p.K, code, sh)
        elif p.packed:
            st = dg.dg_grouped_gemm_fp8_segments(d["A"], fa, d["sA"], d["B"], fb, d["sB"], d["C"], d["offs"],
                                                 p.G, p.M, p.N, p.K, code, sh)
        elif p.grouped and plain:
            st = dg.dg_grouped_gemm_fp8(d["A"], d["sA"], d["B"], d["sB"], d["C"], d["offs"],
                                        p.G, p.M, p.N, p.K, code, sh)
        elif p.grouped:
            st = dg.dg_grouped_gemm_fp8_ex(d["A"], fa, d["sA"], p.sa_rows, d["B"], fb, d["sB"], d["C"],
                                           d["offs"], p.G, p.M, p.N, p.K, code, sh)
        elif plain:
            st = dg.dg_gemm_fp8_blockscaled(d["A"], d["sA"], d["B"], d["sB"], d["C"], p.M, p.N, p.K, code, sh)
        else:
            st = dg.dg_gemm_fp8_ex(d["A"], fa, d["sA"], p.sa_rows, d["B"], fb, d["sB"], d["C"],
                                   p.M, p.N, p.K, code, sh)
        if st != dg.DG_OK:
            raise dg.DGError(st, "bench step")

    K = args.steps
    ms_step, kern_ms, _ = run_timed(step, K, args.warmup, not args.no_graph, args.settle_ms)
    kern_eager = eager_kernel_ms(step, K, not args.no_graph)

    flop = p.algorithmic_flop()
    if gbs_value:
        value = step_bytes / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
    else:
        value = flop / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    if hbm_bound:
        achieved = step_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flop / (kern_ms * 1e-3) / 1e12   # == gemm_tflops for dense problems
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                # the products run on the FP16 matrix cores (FP8 operands converted exactly), whose
                # dense peak is half the FP8 one; the FP8 peak above is the metric's reference
                "mfma_unit": "f16", "unit_peak": PEAK_FP16_TFLOPS,
                "unit_frac": round(achieved / PEAK_FP16_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(p.name)
    log(f"algorithmic: {flop / 1e9:.2f} GFLOP, {step_bytes / 2**20:.1f} MiB per step; "
        f"TFLOP/s (kernel) {flop / (kern_ms * 1e-3) / 1e12:.1f}, "
        f"GB/s (kernel) {step_bytes / (kern_ms * 1e-3) / 1e9:.0f}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p)
        if unit == "GB/s":
            # same sample, expressed in the metric's unit (bytes of the full step
            # scaled by the share of rows the oracle covered per second)
            cpu = dict(cpu, value=round(cpu["value"] * 1e12 / flop * step_bytes / 1e9, 6), unit="GB/s")
        log(f"cpu oracle: {cpu}")

    cfg = {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "out_dtype": p.out_dtype,
           "scale_block": "128x128" if p.sa_rows == 128 else "A 1x128, B 128x128", "seed": p.seed,
           "operand_copies": R, "launch": "eager" if args.no_graph else "hip_graph"}
    if p.a_fmt != "e4m3" or p.b_fmt != "e4m3":
        cfg.update({"a_fmt": p.a_fmt, "b_fmt": p.b_fmt})
    if use_counts:
        cfg["padding_aware"] = True
    if p.grouped:
        cfg.update({"groups": p.G, "real_rows": p.real_rows, "active_groups": p.active_groups(),
                    "segments": "packed" if p.packed else "padded to 128 rows"})
    line = {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8_e4m3" if p.a_fmt == p.b_fmt == "e4m3" else f"fp8_{p.a_fmt}x{p.b_fmt}",
            "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "kernel_ms": round(kern_ms, 5), "kernel_ms_eager": kern_eager}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
