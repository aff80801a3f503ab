"""Benchmark of the pipelined FP32 GEMM (and its tile copy) on one MI355X.

A step is one call of the pipelined GEMM on the 8192^3 workload (A, B ~ U[-1,1)
seeded, row-major, 128x128x16 block tile, LDS ring filled asynchronously,
FP32-MFMA compute): the whole hot path (tiling, asynchronous fill with
zero-filled edges, ring waits and barriers, compute tile, epilogue) runs in
that one kernel. Inputs are resident in HBM before timing starts.

Before timing, the timed variant must be bit-identical to the synchronous
fill on the full output (its oracle parity is a GPU test). After the timed region
the same run measures the stage/fill table at 4096^3 and 8192^3, the VALU
variant, the pipelined 1 GiB tile copy, and the oracle on a bounded sample of
host cores, and prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP32 GEMM GFLOP/s + % FP32 peak at 4096³/8192³; piped/sync speedup; copy GB/s"
PEAK_FP32_TFLOPS = 157.3   # MI355X dense FP32 (MFMA and packed vector), AMD spec
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, AMD spec


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--size", type=int, default=8192)
    p.add_argument("--stages", type=int, default=3)
    p.add_argument("--compute", default="mfma", choices=["mfma", "valu"])
    p.add_argument("--no-extra", action="store_true", help="skip the tables after the timed region")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    return p.parse_args()


def timed_launches(fn, warmup=3, runs=10, repeats=1):
    """The pages' protocol ("pipelined_gemm.cu", timeKernel): warm-up launches,
    then the mean of `runs` launches between two events; `repeats` blocks give
    min and median."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    means = []
    for _ in range(repeats):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(runs):
            fn()
        e.record()
        e.synchronize()
        means.append(s.elapsed_time(e) / runs)
    means.sort()
    return {"ms_min": means[0], "ms_median": means[len(means) // 2]}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the GEMM would shard by C row bands; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import async_global_shared_amd as m
    import datagen

    torch.cuda.set_device(0)
    n = args.size
    M = N = K = n
    flop = 2.0 * M * N * K
    Ad = datagen.uniform_pm1_torch(datagen.SEED_A, M * K, device="cuda").view(M, K)
    Bd = datagen.uniform_pm1_torch(datagen.SEED_B, K * N, device="cuda").view(K, N)
    Cd = torch.empty((M, N), device="cuda")
    variant = dict(stages=args.stages, fill="piped", compute=args.compute, tile="128x128")
    plan = m.plan(M, N, K, stages=args.stages, fill="piped", compute=args.compute, tile="128x128")

    # ---- parity gate before any timing: the piped output must be bit-identical
    # to the synchronous fill (the oracle comparison of this exact launch is
    # tests/test_gpu_fullsize.py; the oracle is only timed here, below) ----
    m.sgemm(Ad, Bd, Cd, **variant)
    Cs = torch.empty_like(Cd)
    m.sgemm(Ad, Bd, Cs, stages=1, fill="sync", compute=args.compute, tile="128x128")
    torch.cuda.synchronize()
    if not torch.equal(Cd.view(torch.int32), Cs.view(torch.int32)):
        print("parity gate: piped output differs from sync output", file=sys.stderr)
        sys.exit(1)
    if not bool(torch.isfinite(Cd).all()):
        print("parity gate: non-finite output", file=sys.stderr)
        sys.exit(1)
    del Cs

    # ---- timed region: exactly `steps` steps ----
    stream = torch.cuda.current_stream()
    step = lambda: m.sgemm(Ad, Bd, Cd, **variant)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = sum(s.elapsed_time(e) for s, e in evs) / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e9
    achieved_tflops = flop / (kernel_ms * 1e-3) / 1e12

    props = torch.cuda.get_device_properties(0)
    extra = {
        "device": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
        "pct_fp32_peak_8192": round(100.0 * value / 1e3 / PEAK_FP32_TFLOPS, 2),
        "kernel_ms": round(kernel_ms, 4), "parity_gate": "piped == sync (bitwise, full output)",
        "plan": plan,
    }

    if not args.no_extra:
        extra.update(tables(m, datagen, torch, Ad, Bd, Cd))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(Ad, Bd)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"FP32 GEMM M=N=K={n}, row-major, A,B~U[-1,1) seeded; 128x128x16 block tile, "
                               f"{args.stages}-stage asynchronous LDS ring (buffer_load...lds), "
                               f"{args.compute.upper()} compute tile",
                   "M": M, "N": N, "K": K, "stages": args.stages, "fill": "piped", "compute": args.compute,
                   "tile": "128x128"},
        "roofline": {"bound": "mfma" if args.compute == "mfma" else "alu",
                     "achieved": round(achieved_tflops, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_FP32_TFLOPS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def tables(m, datagen, torch, Ad8, Bd8, Cd8):
    """Stage/fill table (GFLOP/s, speedups), VALU variant, tile copy GB/s."""
    res = {}
    gemm = {}
    for n in (4096, 8192):
        if n == 8192:
            A, B, C = Ad8, Bd8, Cd8
        else:
            A, B, C = Ad8[:n, :n].contiguous(), Bd8[:n, :n].contiguous(), torch.empty((n, n), device="cuda")
        flop = 2.0 * n ** 3
        row = {}
        for compute in ("mfma", "valu"):
            for fill in ("sync", "piped"):
                for S in (1, 2, 3):
                    if compute == "valu" and n == 8192 and (fill, S) not in (("sync", 1), ("piped", 2), ("piped", 3)):
                        continue
                    t = timed_launches(lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute,
                                                       tile="128x128"), repeats=3)
                    row[f"{compute}_{fill}_S{S}"] = {
                        "ms": round(t["ms_median"], 4), "gflops": round(flop / (t["ms_median"] * 1e-3) / 1e9, 1),
                        "pct_peak": round(100 * flop / (t["ms_median"] * 1e-3) / 1e12 / 157.3, 2)}
        for compute in ("mfma", "valu"):
            base = row.get(f"{compute}_sync_S1")
            for S in (1, 2, 3):
                p = row.get(f"{compute}_piped_S{S}")
                s = row.get(f"{compute}_sync_S{S}")
                if base and p:
                    p["speedup_vs_sync_S1"] = round(base["ms"] / p["ms"], 3)
                    p["time_ratio_piped_over_sync_S1"] = round(p["ms"] / base["ms"], 3)
                if s and p:
                    p["speedup_vs_sync_same_S"] = round(s["ms"] / p["ms"], 3)
        gemm[str(n)] = row
        if n != 8192:
            del A, B, C
    res["gemm"] = gemm
    # tile copy: 1 GiB fp32 ~ N(0,1), 64x64 tiles, 2 x bytes moved
    rows = cols = 16384
    src = datagen.normal01_torch(datagen.SEED_COPY, rows * cols, device="cuda").view(rows, cols)
    dst = torch.empty_like(src)
    nbytes = 2.0 * src.numel() * 4
    copy = {}
    for S in (1, 2, 3):
        t = timed_launches(lambda: m.tile_copy(src, dst, stages=S), repeats=3)
        copy[f"S{S}"] = {"ms": round(t["ms_median"], 4), "GBps": round(nbytes / (t["ms_median"] * 1e-3) / 1e9, 1)}
        copy[f"S{S}"]["pct_hbm_peak"] = round(100 * copy[f"S{S}"]["GBps"] / PEAK_HBM_GBS, 2)
    t = timed_launches(lambda: dst.copy_(src), repeats=3)
    copy["torch_copy_context"] = {"ms": round(t["ms_median"], 4),
                                  "GBps": round(nbytes / (t["ms_median"] * 1e-3) / 1e9, 1)}
    res["tile_copy_1GiB"] = copy
    del src, dst
    return res


def cpu_baseline(Ad, Bd, budget_s=12.0):
    """The oracle (fp64 C loops, OpenMP over rows) on the first rows of the
    same problem: a bounded sample (about `budget_s` of wall time on the host
    cores), scaled to GFLOP/s."""
    import oracle
    lib = oracle.load()
    threads = oracle.num_threads(lib)
    B_host = Bd.cpu().numpy()
    probe = Ad[:threads].cpu().numpy()
    dt, fl = oracle.timed_gemm_rows(probe, B_host, threads, lib=lib)
    rows = int(min(Ad.shape[0], max(threads, threads * int(budget_s / max(dt, 1e-3)))))
    A_host = Ad[:rows].cpu().numpy()
    dt, fl = oracle.timed_gemm_rows(A_host, B_host, rows, lib=lib)
    return {"value": round(fl / dt / 1e9, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {Ad.shape[0]} rows of the {Ad.shape[0]}x{Bd.shape[1]}x{Ad.shape[1]} product "
                      f"(fp64 accumulate), {dt:.1f} s wall"}


if __name__ == "__main__":
    main()
