#!/usr/bin/env python3
"""Benchmark: one rank's share of the overlapped AllGather+GEMM on one MI355X.

One step is one ag_gemm call in overlap mode on the W=8 bf16 workload (A: 8 shards x 512 rows,
4096 x 8192; W_local 8192 x 3584; 128-row chunks arriving in ring order): call setup, the
producer's put + signal of the 28 remote chunks (by default copy jobs inside the persistent
kernel; --producer sdma uses the copy engines), tile claims in arrival order, flag waits, the
MFMA main loop and the bf16 epilogue, and the join. Inputs are resident in HBM before timing.

Printed (one JSON line): overlapped TFLOP/s (value), % of the bf16 MFMA peak, the overlap
figures R = T_ovl / T_gemm and eta = (T_serial - T_ovl) / min(T_copy, T_gemm) from the same
kernels in the other modes (per-call stream times with the modes interleaved call by call; the
t_*_us fields are the modes timed one after another, which the board's clock drift skews), the
dominant kernel's roofline (its own duration from timing events on the stream it runs on), and
the CPU oracle's rate on the same workload as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "overlapped AG+GEMM TFLOP/s on 1 MI355X (% MFMA peak) + overlap efficiency"
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0
# counter records (profiles/traffic_<record>.txt) of each workload's overlapped launch
TRAFFIC_RECORDS = {"ag_w8_4096x3584x8192_bf16": "gemm_kernel_256x224_bf16_ag_w8_4096x3584x8192_overlap"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the W=8 bf16 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modes", default="overlap,gemm_only,copy_only,serial,sdma",
                    help="modes to time; the overlapped steps always run (profiling runs use"
                         " 'overlap' alone so that every consumer-kernel launch is a timed step);"
                         " 'sdma' also times the overlap with the copy-engine producer")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the timed steps, run one plain device copy of this many MiB (a"
                         " known-size kernel that HBM byte counters are scaled against)")
    ap.add_argument("--producer", default="cu", choices=["cu", "sdma"],
                    help="producer of the timed steps: copy jobs inside the kernel (cu) or the"
                         " copy engines (sdma)")
    return ap.parse_args()


def time_mode(w, mode, order, steps, warmup):
    """Mean wall time per call (us) of `steps` back-to-back calls, synchronised on both sides."""
    import torch
    for _ in range(warmup):
        w.run(mode, order=order)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        w.run(mode, order=order)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps * 1e6
    st = w.status()
    if st[0]:
        raise RuntimeError(f"{mode}: a chunk wait gave up (flag {st[1]})")
    return dt


def measured_traffic(name):
    """HBM bytes per launch from the committed counter record for this workload's overlapped
    launch, or None when there is none or the kernel source changed since it was taken."""
    import hashlib
    rec = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(rec):
        return None
    kv = dict(line.strip().split("=", 1) for line in open(rec) if "=" in line and not line.startswith("#"))
    src = b"".join(open(os.path.join(ROOT, "allgather_gemm_persistent_amd", "csrc", f), "rb").read()
                   for f in ("kernels.hip", "kernels.h", "pipeline.h"))
    if hashlib.sha256(src).hexdigest() != kv.get("kernel_source_sha256"):
        return None
    return int(kv["traffic_bytes"])


def cpu_baseline(cfg, data):
    """The CPU oracle on the whole workload (float64, numpy/BLAS threads)."""
    from threadpoolctl import threadpool_info

    from allgather_gemm_persistent_amd import inputs
    from oracle import agg_oracle as O
    shards = [inputs.raw_bits(s) for s in data["shards"]]
    b = inputs.raw_bits(data["b"])
    t0 = time.perf_counter()
    O.ag_gemm_ref(shards, b, cfg.dtype, data["scale_a"], data["scale_b"])
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [os.cpu_count() or 1])
    return {"value": round(cfg.flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole workload ({cfg.m}x{cfg.n}x{cfg.k}, {cfg.flops / 1e9:.1f} GFLOP):"
                      f" exact decode + float64 matmul, {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (one rank's share of the collective on one MI355X); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    from allgather_gemm_persistent_amd import binding as B
    from allgather_gemm_persistent_amd import configs
    from allgather_gemm_persistent_amd.workload import AgWorkload

    name = args.workload or configs.HEADLINE
    cfg = configs.CONFIGS[name]
    assert cfg.op == "ag", "the benchmark measures AllGather+GEMM workloads"
    data = configs.make_ag_data(cfg)
    w = AgWorkload(cfg.world, cfg.rank, data["shards"], data["b"], cfg.chunk_rows, cfg.dtype,
                   data["scale_a"], data["scale_b"])
    order = cfg.order()
    peak = PEAK_FP8_TFLOPS if cfg.dtype == "fp8" else PEAK_BF16_TFLOPS
    B.agg_ctx_set_producer(w.ctx, args.producer)
    # the calls go to a stream of their own (as in a framework that runs its work off the legacy
    # null stream, whose implicit synchronisation costs every call some microseconds)
    bench_stream = torch.cuda.Stream()
    torch.cuda.set_stream(bench_stream)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    try:
        B.agg_ctx_set_timing(w.ctx, True)
        # the timed steps: overlapped calls
        for _ in range(args.warmup):
            w.run("overlap", order=order)
        torch.cuda.synchronize()
        B.agg_ctx_set_timing(w.ctx, True)          # clears the ring: only timed launches count
        t0 = time.perf_counter()
        for _ in range(args.steps):
            w.run("overlap", order=order)
        torch.cuda.synchronize()
        t_ovl = (time.perf_counter() - t0) / args.steps * 1e6
        st = w.status()
        if st[0]:
            raise RuntimeError(f"overlap: a chunk wait gave up (flag {st[1]})")
        kms = B.agg_ctx_kernel_times(w.ctx, args.steps)
        k_ovl_us = statistics.mean(kms) * 1e3
        # the same kernels in the other modes
        modes = set(args.modes.split(","))
        t_gemm = t_copy = t_serial = k_gemm_us = None
        if "gemm_only" in modes:
            B.agg_ctx_set_timing(w.ctx, True)
            t_gemm = time_mode(w, "gemm_only", order, args.steps, args.warmup)
            k_gemm_us = statistics.mean(B.agg_ctx_kernel_times(w.ctx, args.steps)) * 1e3
        if "copy_only" in modes:
            t_copy = time_mode(w, "copy_only", order, args.steps, args.warmup)
        if "serial" in modes:
            t_serial = time_mode(w, "serial", order, args.steps, args.warmup)
        # every mode again, interleaved call by call, so that all see the same clock and
        # temperature (the clock drops as the board heats within a run, so modes timed one after
        # another are not comparable): per-call stream time from events around each call, and
        # the consumer kernels' own durations
        k_int = s_int = None
        inter = [m for m in ("overlap", "gemm_only", "copy_only", "serial") if m == "overlap" or m in modes]
        if "gemm_only" in modes:
            B.agg_ctx_set_timing(w.ctx, True)
            seq, ev = [], []
            for _ in range(args.steps):
                for m in inter:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(bench_stream)
                    w.run(m, order=order)
                    e1.record(bench_stream)
                    ev.append((m, e0, e1))
                    seq.append(m)          # every mode times one consumer launch per call
            torch.cuda.synchronize()
            ks = B.agg_ctx_kernel_times(w.ctx, len(seq))
            k_int = {m: statistics.median([k * 1e3 for k, q in zip(ks, seq) if q == m])
                     for m in ("overlap", "gemm_only")}
            s_int = {m: statistics.median([a.elapsed_time(b) * 1e3 for q, a, b in ev if q == m])
                     for m in inter}
        other = {"cu": "sdma", "sdma": "cu"}[args.producer]
        t_ovl_other = None
        if other in modes:
            B.agg_ctx_set_producer(w.ctx, other)
            t_ovl_other = time_mode(w, "overlap", order, args.steps, args.warmup)
            B.agg_ctx_set_producer(w.ctx, args.producer)
    finally:
        B.agg_ctx_set_timing(w.ctx, False)
        w.close()

    flops = cfg.flops
    value = flops / (t_ovl * 1e-6) / 1e12
    achieved = flops / (k_ovl_us * 1e-6) / 1e12

    def rnd(x, d=1):
        return None if x is None else round(x, d)
    # R and eta from the interleaved per-call times (same clock for every mode)
    R = eta = None
    if s_int and "gemm_only" in s_int:
        R = s_int["overlap"] / s_int["gemm_only"]
        if "copy_only" in s_int and "serial" in s_int:
            eta = (s_int["serial"] - s_int["overlap"]) / min(s_int["copy_only"], s_int["gemm_only"])
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_ovl / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": f"{name}: AllGather+GEMM one rank's share, W={cfg.world}, "
                               f"A {cfg.m}x{cfg.k} ({cfg.world} shards x {cfg.m_shard} rows), "
                               f"W_local {cfg.k}x{cfg.n}, chunk_rows={cfg.chunk_rows}, "
                               f"{cfg.order_kind} arrival, {cfg.dtype}, fp32 accumulate, bf16 out",
                   "m": cfg.m, "n": cfg.n, "k": cfg.k, "world": cfg.world,
                   "chunk_rows": cfg.chunk_rows},
        "pct_mfma_peak": round(100 * value / peak, 2),
        "overlap": {"t_ovl_us": round(t_ovl, 1), "t_gemm_us": rnd(t_gemm),
                    "t_copy_us": rnd(t_copy), "t_serial_us": rnd(t_serial),
                    "R": rnd(R, 3), "eta": rnd(eta, 3),
                    "interleaved_call_us": ({m: rnd(v) for m, v in s_int.items()} if s_int else None),
                    "interleaved_kernel_us": ({"overlap": rnd(k_int["overlap"]),
                                               "gemm_only": rnd(k_int["gemm_only"]),
                                               "R": rnd(k_int["overlap"] / k_int["gemm_only"], 3)}
                                              if k_int else None),
                    "gemm_only_tflops": rnd(flops / (t_gemm * 1e-6) / 1e12) if t_gemm else None,
                    "gemm_only_kernel_us": rnd(k_gemm_us),
                    "producer": args.producer,
                    f"t_ovl_{other}_producer_us": rnd(t_ovl_other),
                    f"R_{other}_producer": rnd(t_ovl_other / t_gemm, 3)
                    if (t_ovl_other and t_gemm) else None},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(TRAFFIC_RECORDS.get(name, "")),
                     "traffic_unit": "bytes per launch",
                     "kernel": "agg::gemm_kernel (overlap launch)",
                     "kernel_us": round(k_ovl_us, 1),
                     "gemm_only_frac": rnd(flops / (k_gemm_us * 1e-6) / 1e12 / peak, 4)
                     if k_gemm_us else None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, data)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
