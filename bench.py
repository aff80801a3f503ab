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
PEAK_16BIT_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA (no sparsity), AMD spec
# The 1 GiB fp32 array in 64x64 tiles, read two ways: as a 16384 x 16384
# matrix (each tile row is 256 contiguous bytes, rows 64 KiB apart) and as a
# 4194304 x 64 matrix (each tile is 16 KiB of contiguous memory).
COPY_VIEWS = ((16384, 16384), (4194304, 64))


KERNEL_SOURCES = ("async_global_shared_amd/csrc/device.hpp", "async_global_shared_amd/csrc/ring.h",
                  "async_global_shared_amd/csrc/attention.hpp", "async_global_shared_amd/csrc/mgemm.hip")
COUNTERS_FILE = "profiles/counters_gemm8192_copy1GiB_gemm16_attention.txt"


def kernel_source_hash() -> str:
    """sha256 over the kernel and launch sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel_name: str, grid: int):
    """HBM bytes per launch of `kernel_name` from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the calibration copy),
    or None when the summary is missing or the kernel sources changed since."""
    path = os.path.join(ROOT, COUNTERS_FILE)
    if not os.path.exists(path):
        return None
    section, vals, top = None, {}, {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            section = line[1:-1]
            continue
        k, _, v = line.partition("=")
        (vals.setdefault(section, {}) if section else top)[k] = v
    if top.get("kernel_src_sha256") != kernel_source_hash():
        return None
    sec = vals.get(f"{kernel_name} grid={grid}")
    if not sec or "hbm_bytes_per_launch" not in sec:
        return None
    return float(sec["hbm_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--size", type=int, default=8192)
    p.add_argument("--stages", type=int, default=2)
    p.add_argument("--compute", default="mfma", choices=["mfma", "valu"])
    p.add_argument("--no-extra", action="store_true", help="skip the tables after the timed region")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    p.add_argument("--oracle-full", action="store_true",
                   help="also time the oracle once on the whole problem (all rows; about 20 s on 16 host cores)")
    p.add_argument("--profile", action="store_true",
                   help="only run a few launches of the timed GEMM, the 1 GiB tile copy (3 stages), the plain "
                        "1 GiB copy (the calibration kernel for hardware byte counters), the 16-bit GEMM "
                        "and the attention kernel, for rocprofv3")
    return p.parse_args()


def profile_mode(args):
    """Launches for counter collection, `steps` of each, no timing: the timed
    GEMM, its VALU twin, the automatic MFMA plan of the same problem (the
    256x128 tile), the ragged and tall-skinny GEMMs (MFMA, piped S=2),
    the 1 GiB tile copy in both array views, the plain
    1 GiB copy (mgemm_plain_copy, the calibration kernel for hardware byte
    counters), the 16-bit GEMM and the attention kernel in their default
    plans."""
    import torch

    import async_global_shared_amd as m
    import datagen
    n = args.size
    Ad = datagen.uniform_pm1_torch(datagen.SEED_A, n * n, device="cuda").view(n, n)
    Bd = datagen.uniform_pm1_torch(datagen.SEED_B, n * n, device="cuda").view(n, n)
    Cd = torch.empty((n, n), device="cuda")
    for compute in (args.compute, "valu" if args.compute == "mfma" else "mfma"):
        for _ in range(args.steps):
            m.sgemm(Ad, Bd, Cd, stages=args.stages, fill="piped", compute=compute, tile="128x128")
        torch.cuda.synchronize()
        print(f"profile: {args.steps} x sgemm {n}^3 {compute} piped S={args.stages}", flush=True)
    for _ in range(args.steps):
        m.sgemm(Ad, Bd, Cd, stages=args.stages, fill="piped", compute="mfma")
    torch.cuda.synchronize()
    print(f"profile: {args.steps} x sgemm {n}^3 mfma piped S={args.stages}, automatic plan "
          f"{m.plan(n, n, n, stages=args.stages, compute='mfma')}", flush=True)
    del Ad, Bd, Cd
    for name, M, N, K in CONFIG5:
        A = datagen.uniform_pm1_torch(datagen.SEED_A, M * K, device="cuda").view(M, K)
        B = datagen.uniform_pm1_torch(datagen.SEED_B, K * N, device="cuda").view(K, N)
        C = torch.empty((M, N), device="cuda")
        for _ in range(args.steps):
            m.sgemm(A, B, C, stages=2, fill="piped", compute="mfma")
        torch.cuda.synchronize()
        print(f"profile: {args.steps} x sgemm {name} mfma piped S=2, plan {m.plan(M, N, K, compute='mfma')}",
              flush=True)
        del A, B, C
    src = datagen.normal01_torch(datagen.SEED_COPY, 1 << 28, device="cuda")
    dst = torch.empty_like(src)
    for shape in COPY_VIEWS:
        for _ in range(args.steps):
            m.tile_copy(src.view(*shape), dst.view(*shape), stages=3)
        torch.cuda.synchronize()
        print(f"profile: {args.steps} x tile_copy 1 GiB as {shape[0]}x{shape[1]} S=3", flush=True)
    for _ in range(args.steps):
        m.plain_copy(src.view(*COPY_VIEWS[0]), dst.view(*COPY_VIEWS[0]))
    torch.cuda.synchronize()
    print(f"profile: {args.steps} x plain copy 1 GiB (the copy ceiling and the counters' calibration: "
          f"2^30 B read, 2^30 B written)", flush=True)
    del src, dst
    A16 = datagen.grid16_torch(datagen.SEED_A, n, n, "bf16", device="cuda")
    B16 = datagen.grid16_torch(datagen.SEED_B, n, n, "bf16", device="cuda")
    C = torch.empty((n, n), device="cuda")
    for _ in range(args.steps):
        m.gemm16(A16, B16, C)
    torch.cuda.synchronize()
    print(f"profile: {args.steps} x gemm16 {n}^3 bf16, default plan {m.plan16(n, n, n)}", flush=True)
    del A16, B16, C
    B_, H_, S_ = ATTN_SHAPE
    Q, K, V = (datagen.grid16_torch(seed, 1, B_ * H_ * S_ * 128, "bf16", device="cuda").view(B_, H_, S_, 128)
               for seed in (datagen.SEED_A, datagen.SEED_B, datagen.SEED_COPY))
    O = torch.empty((B_, H_, S_, 128), device="cuda")
    for _ in range(args.steps):
        m.attention(Q, K, V, O)
    torch.cuda.synchronize()
    print(f"profile: {args.steps} x attention {B_}x{H_}x{S_}x128 bf16, default plan "
          f"{m.plan_attention(B_, H_, S_, S_, 128)}", flush=True)


def peak_clock_mhz():
    """The device's peak shader clock in MHz from the HIP runtime
    (hipDeviceGetAttribute with hipDeviceAttributeClockRate, which is entry 5
    of hipDeviceAttribute_t and reports kHz), or None if unavailable. The
    clock under load is lower and varies: the kernel timings are the truth."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    v = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) != 0:
        return None
    return round(v.value / 1000.0, 1)


# blocks of 10 timed launches per table entry: the median and the minimum are reported
REPEATS = 5


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
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the GEMM would shard by row bands of C, one band per GPU, with B broadcast)", file=sys.stderr)
        sys.exit(2)
    if args.profile:
        profile_mode(args)
        return

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
    arch = getattr(props, "gcnArchName", "")
    extra = {
        "device": props.name or f"AMD {arch.split(':')[0]} ({props.multi_processor_count} CUs)", "arch": arch,
        "cus": props.multi_processor_count, "peak_clock_mhz": peak_clock_mhz(),
        "l2_bytes": getattr(props, "L2_cache_size", None),
        "pct_fp32_peak_8192": round(100.0 * value / 1e3 / PEAK_FP32_TFLOPS, 2),
        "kernel_ms": round(kernel_ms, 4), "parity_gate": "piped == sync (bitwise, full output)",
        "plan": plan,
    }

    clock = extra["peak_clock_mhz"]
    if clock:
        # 256 FLOP per clock per CU: 4 SIMDs, each a 32x32x2 fp32 MFMA (4096 FLOP) every 64 clocks
        extra["peak_fp32_tflops_from_device"] = round(props.multi_processor_count * 256 * clock / 1e6, 1)
    if not args.no_extra:
        extra.update(tables(m, datagen, torch, Ad, Bd, Cd, with_oracle=not args.no_cpu))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(Ad, Bd)
        extra["oracle_timing"] = oracle_timing(Ad, Bd, datagen, full=args.oracle_full)

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
                     "frac": round(achieved_tflops / PEAK_FP32_TFLOPS, 4),
                     "traffic": measured_traffic(
                         f"void mgemm::sgemm_kernel<mgemm::Cfg{'Mfma' if args.compute == 'mfma' else 'Valu'}128, "
                         f"{args.stages}, true, 16>(mgemm::GemmArgs)", plan["blocks"] * plan["threads"])},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


class Gate:
    """Bitwise parity gate of a table: the first variant run becomes the
    reference output and every later variant must reproduce it bit for bit
    before it is timed (the pages' program compares the piped output with
    the synchronous one before timing either, "pipelined_gemm.cu", main)."""

    def __init__(self, torch, what):
        self.torch, self.what, self.ref = torch, what, None

    def check(self, run, out, variant):
        torch = self.torch
        out.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        if self.ref is None:
            self.ref = out.clone()
        elif not torch.equal(out.view(torch.int32), self.ref.view(torch.int32)):
            raise SystemExit(f"bench parity gate: {self.what} {variant} differs from the first variant")


def oracle_rate(Ad, Bd, budget_s=3.0):
    """The oracle (fp64, OpenMP over rows, all host threads) on the same
    inputs: as many leading rows of A as fit about `budget_s` of wall time
    (all of them for the smaller problems), in GFLOP/s."""
    import oracle
    lib = oracle.load()
    threads = oracle.num_threads(lib)
    B_host = Bd.cpu().numpy()
    M = Ad.shape[0]
    probe = min(M, threads)
    dt, _ = oracle.timed_gemm_rows(Ad[:probe].cpu().numpy(), B_host, probe, lib=lib)
    rows = int(min(M, max(probe, probe * int(budget_s / max(dt, 1e-4)))))
    dt, fl = oracle.timed_gemm_rows(Ad[:rows].cpu().numpy(), B_host, rows, lib=lib)
    return {"gflops": round(fl / dt / 1e9, 3), "threads": threads, "rows": rows, "of_rows": M, "s": round(dt, 3)}


def copy_oracle_rate(host, nbytes):
    """The oracle's copy (row memcpy, OpenMP over rows, all host threads) of
    the same 1 GiB on the host: the best of 3 runs, the bytes checked."""
    import numpy as np
    import oracle
    lib = oracle.load()
    best = None
    for _ in range(3):
        dt, out = oracle.timed_copy(host, lib=lib)
        best = dt if best is None else min(best, dt)
    if not np.array_equal(out.view(np.int32), host.view(np.int32)):
        raise SystemExit("oracle copy changed bytes")
    return {"s": round(best, 4), "GBps": round(nbytes / best / 1e9, 1), "cores": oracle.num_threads(lib),
            "what": "oracle_copy_f32 on the host cores, the 16384x16384 view (read + write bytes over time)"}


def tables(m, datagen, torch, Ad8, Bd8, Cd8, with_oracle=True):
    """Stage/fill table (GFLOP/s, speedups), VALU variant, tile copy GB/s."""
    res = {}
    gemm = {}
    big = Ad8.shape[0]
    for n in sorted({min(4096, big), big}):
        if n == big:
            A, B, C = Ad8, Bd8, Cd8
        else:
            A, B, C = Ad8[:n, :n].contiguous(), Bd8[:n, :n].contiguous(), torch.empty((n, n), device="cuda")
        flop = 2.0 * n ** 3
        row = {}
        for compute in ("mfma", "valu"):
            gate = Gate(torch, f"{n}^3 {compute} 128x128")
            for fill in ("sync", "piped"):
                for S in (1, 2, 3):
                    if compute == "valu" and n > 4096 and (fill, S) not in (("sync", 1), ("piped", 2), ("piped", 3)):
                        continue
                    run = lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute, tile="128x128")
                    gate.check(run, C, f"{fill} S={S}")
                    t = timed_launches(run, repeats=REPEATS)
                    row[f"{compute}_{fill}_S{S}"] = {
                        "ms": round(t["ms_median"], 4), "ms_min": round(t["ms_min"], 4),
                        "gflops": round(flop / (t["ms_median"] * 1e-3) / 1e9, 1),
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
        # the vendor library's fp32 product on the same operands, as context
        # (full fp32: TF32-style reduced-precision paths switched off)
        prev = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False
        try:
            t = timed_launches(lambda: torch.mm(A, B, out=C), repeats=REPEATS)
        finally:
            torch.backends.cuda.matmul.allow_tf32 = prev
        row["torch_mm_fp32_context"] = {"ms": round(t["ms_median"], 4),
                                        "gflops": round(flop / (t["ms_median"] * 1e-3) / 1e9, 1),
                                        "pct_peak": round(100 * flop / (t["ms_median"] * 1e-3) / 1e12 / 157.3, 2)}
        if with_oracle and n != big:  # the full size's oracle rate is the cpu_baseline record
            row["oracle"] = oracle_rate(A, B)
        gemm[str(n)] = row
        if n != big:
            del A, B, C
    res["gemm"] = gemm
    res["gemm_small"] = small_gemm_table(m, datagen, torch, with_oracle)
    res["gemm_ragged_tall_skinny"] = config5_table(m, datagen, torch, with_oracle)
    res["stage_study"] = stage_study(m, torch, Ad8, Bd8, Cd8)
    res["gemm16"] = gemm16_table(m, datagen, torch, sorted({min(4096, big), big}))
    res["attention"] = attention_table(m, datagen, torch)
    # tile copy: 1 GiB fp32 ~ N(0,1), 64x64 tiles, 2 x bytes moved
    n_el = 1 << 28
    src = datagen.normal01_torch(datagen.SEED_COPY, n_el, device="cuda")
    dst = torch.empty_like(src)
    nbytes = 2.0 * n_el * 4
    copy = {}
    t = timed_launches(lambda: m.plain_copy(src.view(*COPY_VIEWS[0]), dst.view(*COPY_VIEWS[0])), repeats=REPEATS)
    if not torch.equal(src, dst):
        raise SystemExit("plain copy changed bytes")
    ceiling = nbytes / (t["ms_median"] * 1e-3) / 1e9
    copy["plain_copy_ceiling"] = {"ms": round(t["ms_median"], 4), "ms_min": round(t["ms_min"], 4),
                                  "GBps": round(ceiling, 1), "pct_hbm_peak": round(100 * ceiling / PEAK_HBM_GBS, 2),
                                  "what": "mgemm_plain_copy: no LDS ring, one 16-byte lane per chunk, non-temporal"}
    for shape in COPY_VIEWS:
        view = f"{shape[0]}x{shape[1]}"
        for S in (1, 2, 3):
            dst.fill_(float("nan"))
            m.tile_copy(src.view(*shape), dst.view(*shape), stages=S)
            torch.cuda.synchronize()
            if not torch.equal(src, dst):
                raise SystemExit(f"tile copy changed bytes ({view} S={S})")
            t = timed_launches(lambda: m.tile_copy(src.view(*shape), dst.view(*shape), stages=S), repeats=REPEATS)
            gbs = nbytes / (t["ms_median"] * 1e-3) / 1e9
            copy[f"{view}_S{S}"] = {"ms": round(t["ms_median"], 4), "ms_min": round(t["ms_min"], 4), "GBps": round(gbs, 1),
                                    "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                                    "frac_of_plain_copy": round(gbs / ceiling, 3)}
    t = timed_launches(lambda: dst.copy_(src), repeats=REPEATS)
    copy["torch_copy_context"] = {"ms": round(t["ms_median"], 4),
                                  "GBps": round(nbytes / (t["ms_median"] * 1e-3) / 1e9, 1)}
    if with_oracle:
        copy["oracle"] = copy_oracle_rate(src.view(*COPY_VIEWS[0]).cpu().numpy(), nbytes)
    res["tile_copy_1GiB"] = copy
    del src, dst
    return res


GEMM16_VARIANTS = (("128x128", "sync", 1), ("128x128", "piped", 2), ("256x128", "sync", 1), ("256x128", "piped", 1),
                   ("256x128", "piped", 2), ("256x128", "piped", 3), ("256x256", "sync", 1), ("256x256", "sync", 2),
                   ("256x256", "piped", 1), ("256x256", "piped", 2))


def gemm16_table(m, datagen, torch, sizes):
    """bfloat16 / binary16 inputs, fp32 accumulation and output
    (mgemm_gemm16): TFLOP/s and share of the 2.5 PFLOP/s dense 16-bit MFMA
    peak per tile, fill and ring depth, after a bitwise piped == sync gate on
    the whole output; torch.matmul (16-bit output) and torch.mm with an
    fp32 output as context."""
    out = {}
    for fmt in ("bf16", "f16"):
        for n in sizes:
            A = datagen.grid16_torch(datagen.SEED_A, n, n, fmt, device="cuda")
            B = datagen.grid16_torch(datagen.SEED_B, n, n, fmt, device="cuda")
            C = torch.empty((n, n), device="cuda")
            C1 = torch.empty((n, n), device="cuda")
            flop = 2.0 * n ** 3
            row = {}
            for tile, fill, S in GEMM16_VARIANTS:
                try:
                    m.plan16(n, n, n, dtype=fmt, stages=S, fill=fill, tile=tile)
                except m.MgemmError:
                    continue
                m.gemm16(A, B, C, stages=S, fill=fill, tile=tile)
                m.gemm16(A, B, C1, stages=1, fill="sync", tile=tile)
                torch.cuda.synchronize()
                if not torch.equal(C.view(torch.int32), C1.view(torch.int32)):
                    raise SystemExit(f"gemm16 parity gate: {fmt} {n} {tile} {fill} S{S} differs from sync S1")
                t = timed_launches(lambda: m.gemm16(A, B, C, stages=S, fill=fill, tile=tile), repeats=REPEATS)
                tf = flop / (t["ms_median"] * 1e-3) / 1e12
                row[f"{tile}_{fill}_S{S}"] = {"ms": round(t["ms_median"], 4), "tflops": round(tf, 1),
                                              "pct_peak": round(100 * tf / PEAK_16BIT_TFLOPS, 2)}
            t = timed_launches(lambda: torch.matmul(A, B), repeats=REPEATS)
            row["torch_matmul_context"] = {"ms": round(t["ms_median"], 4),
                                           "tflops": round(flop / (t["ms_median"] * 1e-3) / 1e12, 1)}
            # the same product with an fp32 output, like this library's
            t = timed_launches(lambda: torch.mm(A, B, out_dtype=torch.float32, out=C1), repeats=REPEATS)
            row["torch_mm_fp32_out_context"] = {"ms": round(t["ms_median"], 4),
                                                "tflops": round(flop / (t["ms_median"] * 1e-3) / 1e12, 1)}
            best = max((k for k in row if not k.startswith("torch_")), key=lambda k: row[k]["tflops"])
            row["best"] = best
            out[f"{fmt}_{n}"] = row
            del A, B, C, C1
    return out


ATTN_SHAPE = (16, 16, 4096)  # batch, heads, sequence length (queries = keys)


def attention_table(m, datagen, torch):
    """Attention forward (softmax(Q K^T / sqrt(D)) V, 16-bit Q, K, V, fp32 O)
    at batch 16, 16 heads, 4096 queries and keys, head dims 128 and 64:
    TFLOP/s (4 B H Sq Sk D per call) and share of the 2.5 PFLOP/s dense 16-bit
    MFMA peak per fill and ring depth, after a bitwise piped == sync gate on
    the whole output; torch's scaled_dot_product_attention as context."""
    import torch.nn.functional as F
    B, H, S = ATTN_SHAPE
    out = {}
    for fmt in ("bf16", "f16"):
        for D in (128, 64):
            Q, K, V = (datagen.grid16_torch(seed, 1, B * H * S * D, fmt, device="cuda").view(B, H, S, D)
                       for seed in (datagen.SEED_A, datagen.SEED_B, datagen.SEED_COPY))
            O = torch.empty((B, H, S, D), device="cuda")
            O1 = torch.empty_like(O)
            flop = 4.0 * B * H * S * S * D
            row = {}
            for fill in ("sync", "piped"):
                for St in (1, 2, 3, 4):
                    try:
                        m.plan_attention(B, H, S, S, D, dtype=fmt, stages=St, fill=fill)
                    except m.MgemmError:
                        continue
                    m.attention(Q, K, V, O, stages=St, fill=fill)
                    m.attention(Q, K, V, O1, stages=1, fill="sync")
                    torch.cuda.synchronize()
                    if not torch.equal(O.view(torch.int32), O1.view(torch.int32)):
                        raise SystemExit(f"attention parity gate: {fmt} D{D} {fill} S{St} differs from sync S1")
                    t = timed_launches(lambda: m.attention(Q, K, V, O, stages=St, fill=fill), repeats=REPEATS)
                    tf = flop / (t["ms_median"] * 1e-3) / 1e12
                    row[f"{fill}_S{St}"] = {"ms": round(t["ms_median"], 4), "tflops": round(tf, 1),
                                            "pct_peak": round(100 * tf / PEAK_16BIT_TFLOPS, 2)}
            t = timed_launches(lambda: F.scaled_dot_product_attention(Q, K, V), repeats=REPEATS)
            row["torch_sdpa_context"] = {"ms": round(t["ms_median"], 4),
                                         "tflops": round(flop / (t["ms_median"] * 1e-3) / 1e12, 1)}
            row["best"] = max((k for k in row if k != "torch_sdpa_context"), key=lambda k: row[k]["tflops"])
            out[f"{fmt}_D{D}"] = row
            del Q, K, V, O, O1
    return out


def stage_study(m, torch, Ad8, Bd8, Cd8):
    """The lesson's exercise (ring depth swept, ratio to the synchronous fill,
    LDS per block and what it costs in resident blocks), for its own 64x64x16
    4x4 VALU kernel at N = 2048 and for the MFMA kernel at the full size."""
    out = {}
    for name, n, compute, tile in (("valu64_N2048", 2048, "valu", "64x64"),
                                   (f"mfma128_N{Ad8.shape[0]}", Ad8.shape[0], "mfma", "128x128")):
        if n == Ad8.shape[0]:
            A, B, C = Ad8, Bd8, Cd8
        else:
            A, B = Ad8[:n, :n].contiguous(), Bd8[:n, :n].contiguous()
            C = torch.empty((n, n), device="cuda")
        flop = 2.0 * n ** 3
        rows = {}
        gate = Gate(torch, f"stage study {name}")
        run = lambda: m.sgemm(A, B, C, stages=1, fill="sync", compute=compute, tile=tile)
        gate.check(run, C, "sync S=1")
        base = timed_launches(run, repeats=REPEATS)["ms_median"]
        rows["sync_S1"] = {"ms": round(base, 4), "gflops": round(flop / base / 1e6, 1)}
        for fill in ("piped", "piped_ws"):
            for S in range(1, 7):
                run = lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute, tile=tile)
                gate.check(run, C, f"{fill} S={S}")
                ms = timed_launches(run, repeats=REPEATS)["ms_median"]
                p = m.plan(n, n, n, stages=S, fill=fill, compute=compute, tile=tile)
                rows[f"{fill}_S{S}"] = {"ms": round(ms, 4), "gflops": round(flop / ms / 1e6, 1),
                                        "speedup_vs_sync_S1": round(base / ms, 3),
                                        "time_ratio_piped_over_sync_S1": round(ms / base, 3),
                                        "lds_bytes": p["lds_bytes"],
                                        "blocks_per_cu": m.blocks_per_cu(n, n, n, stages=S, fill=fill,
                                                                         compute=compute, tile=tile)}
        out[name] = rows
    return out


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


def small_gemm_table(m, datagen, torch, with_oracle=True):
    """The pages' own small shapes on the seeded U[-1,1) inputs: 256^3 with
    their 64x64x16 tile (4x4 micro-tile, VALU), sync S=1 against piped S=2,
    and 1024^3 at every fill and depth with the automatic tile (VALU and
    MFMA). Each output is checked bitwise against the sync S=1 one first."""
    out = {}
    for n, cases in ((256, [("valu", "64x64", "sync", 1), ("valu", "64x64", "piped", 2)]),
                     (1024, [(c, "auto", f, S) for c in ("valu", "mfma") for f in ("sync", "piped") for S in (1, 2, 3)])):
        A = datagen.uniform_pm1_torch(datagen.SEED_A, n * n, device="cuda").view(n, n)
        B = datagen.uniform_pm1_torch(datagen.SEED_B, n * n, device="cuda").view(n, n)
        C = torch.empty((n, n), device="cuda")
        flop = 2.0 * n ** 3
        row, ref = {}, {}
        for compute, tile, fill, S in cases:
            f = lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute, tile=tile)
            f()
            torch.cuda.synchronize()
            if compute not in ref:
                ref[compute] = C.clone()
            elif not torch.equal(C.view(torch.int32), ref[compute].view(torch.int32)):
                raise SystemExit(f"bench: {n}^3 {compute} {fill} S={S} differs from sync S=1")
            t = timed_launches(f, repeats=REPEATS)
            row[f"{compute}_{tile}_{fill}_S{S}"] = {
                "ms": round(t["ms_median"], 5), "ms_min": round(t["ms_min"], 5),
                "gflops": round(flop / (t["ms_median"] * 1e-3) / 1e9, 1),
                "pct_peak": round(100 * flop / (t["ms_median"] * 1e-3) / 1e12 / 157.3, 2)}
        for key, v in row.items():
            base = row[key.rsplit("_", 2)[0] + "_sync_S1"]
            if "_piped_" in key:
                v["speedup_vs_sync_S1"] = round(base["ms"] / v["ms"], 3)
                v["time_ratio_piped_over_sync_S1"] = round(v["ms"] / base["ms"], 3)
        if with_oracle:
            row["oracle"] = oracle_rate(A, B)
        out[str(n)] = row
    return out


CONFIG5 = (("ragged_4099x3001x1537", 4099, 3001, 1537), ("tall_skinny_16384x64x4096", 16384, 64, 4096))
CONFIG5_VARIANTS = (("sync", 1), ("sync", 2), ("sync", 3), ("piped", 1), ("piped", 2), ("piped", 3))


def config5_table(m, datagen, torch, with_oracle=True):
    """The ragged 4099x3001x1537 GEMM (lda = 1537, ldb = ldc = 3001: every
    row misaligned for 16-byte loads, so 4-byte loads and zero-filled edge
    tiles) and the tall-skinny 16384x64x4096 GEMM, on seeded U[-1,1) inputs
    with the automatic tile: GFLOP/s and share of the fp32 peak per compute
    tile, fill and ring depth, each variant bit-identical to the first (sync
    S=1) before it is timed; speedups against sync S=1; the oracle's rate on
    the same inputs."""
    out = {}
    for name, M, N, K in CONFIG5:
        A = datagen.uniform_pm1_torch(datagen.SEED_A, M * K, device="cuda").view(M, K)
        B = datagen.uniform_pm1_torch(datagen.SEED_B, K * N, device="cuda").view(K, N)
        C = torch.empty((M, N), device="cuda")
        flop = 2.0 * M * N * K
        row = {}
        for compute in ("valu", "mfma"):
            plan = m.plan(M, N, K, compute=compute, stages=2, fill="piped")
            gate = Gate(torch, f"{name} {compute}")
            for fill, S in CONFIG5_VARIANTS:
                run = lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute)
                gate.check(run, C, f"{fill} S={S}")
                t = timed_launches(run, repeats=REPEATS)
                row[f"{compute}_{fill}_S{S}"] = {
                    "ms": round(t["ms_median"], 5), "ms_min": round(t["ms_min"], 5),
                    "gflops": round(flop / (t["ms_median"] * 1e-3) / 1e9, 1),
                    "pct_peak": round(100 * flop / (t["ms_median"] * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 2)}
            base = row[f"{compute}_sync_S1"]["ms"]
            for fill, S in CONFIG5_VARIANTS:
                v = row[f"{compute}_{fill}_S{S}"]
                if (fill, S) != ("sync", 1):
                    v["speedup_vs_sync_S1"] = round(base / v["ms"], 3)
                    v["time_ratio_over_sync_S1"] = round(v["ms"] / base, 3)
            row[f"{compute}_plan"] = {k: plan[k] for k in ("tile", "bm", "bn", "blocks", "load_bytes")}
        if with_oracle:
            row["oracle"] = oracle_rate(A, B)
        out[name] = row
        del A, B, C
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_timing(Ad, Bd, datagen, full=False):
    """The oracle on the host: the CPU model and thread count, one-thread
    runs at 256^3 and 1024^3 on the seeded uniform inputs, and (with `full`)
    one run over every row of the timed problem on all threads."""
    import oracle
    lib = oracle.load()
    threads = oracle.num_threads(lib)
    out = {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "threads": threads}
    oracle.set_threads(1, lib)
    try:
        for n in (256, 1024):
            A = datagen.matrix("uniform", datagen.SEED_A, n, n)
            B = datagen.matrix("uniform", datagen.SEED_B, n, n)
            dt, fl = oracle.timed_gemm_rows(A, B, n, lib=lib)
            out[f"one_thread_{n}"] = {"s": round(dt, 3), "gflops": round(fl / dt / 1e9, 3)}
    finally:
        oracle.set_threads(threads, lib)
    if full:
        A_host, B_host = Ad.cpu().numpy(), Bd.cpu().numpy()
        dt, fl = oracle.timed_gemm_rows(A_host, B_host, A_host.shape[0], lib=lib)
        out[f"all_threads_full_{A_host.shape[0]}"] = {"s": round(dt, 2), "gflops": round(fl / dt / 1e9, 3)}
    return out


if __name__ == "__main__":
    main()
