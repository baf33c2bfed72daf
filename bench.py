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
dominant kernel's roofline (its own duration from timing events that every n-th timed launch
carries on the stream it runs on, n = min(8, K // 8) or 1 (at least K / 256): the events cost each launch that
carries them some microseconds, so the timed steps sample), and the CPU oracle's rate on the same
workload as a baseline.

`configs` holds one block per workload (the two AllGather+GEMM sizes, ReduceScatter, decode, fp8,
decode GEMM+AllReduce, the FFN chain, AllToAll+GEMM): the same four modes interleaved call by
call (50 calls per mode for the MFMA-bound workloads, 1000 for the latency- and HBM-bound ones;
medians, with p10 / p90), each call preceded (outside its timed span) by a 512 MiB write and a read of the same
512 MiB, which evict the caches (every operand byte then comes from HBM) and leave them holding
clean lines, so that the timed call is not charged for writing back the flush's own data; R, eta and the roofline of the bare and the overlapped kernel against
the bound that applies (MFMA bf16 or fp8, HBM bytes, or launch latency); the overlap with the
copy kernel as producer (R_copy_kernel), and with pull off where pulling applies.

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
# what bounds each workload's kernel: MFMA (flops against the dtype's peak), HBM (bytes against
# 8 TB/s) or launch latency (a handful of tiles on 256 CUs)
BOUND = {"ag_w2_256x256x512_bf16": "latency", "ag_w8_4096x3584x8192_bf16": "mfma",
         "rs_w8_8192x8192x3584_bf16": "mfma", "ag_w8_128x3584x8192_bf16_decode": "hbm",
         "ag_w8_8192x7168x8192_fp8": "mfma", "ar_w8_128x8192x3584_bf16_decode": "hbm",
         "ffn_w8_4096x8192x3584_bf16": "mfma", "a2a_w8_5120x3584x8192_bf16": "mfma"}
# workloads where pulling remote rows is possible: also timed with pull off (flag-gated push)
PULL_VARIANTS = {"ag_w2_256x256x512_bf16", "ag_w8_128x3584x8192_bf16_decode"}
FLUSH_BYTES = 512 << 20


def cache_flush():
    """The flush before each timed call of a block: a 512 MiB write, which evicts every operand
    from the L2s and the 256 MB MALL, then a read of the same bytes, which evicts the write's
    dirty lines in turn (their write-back happens here, not in the timed call) and leaves clean
    ones. Returns flush(i)."""
    import torch
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    words = buf.view(torch.int32)

    def flush(i):
        buf.fill_(i & 0xFF)
        words.sum(dtype=torch.int64)
    return flush


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the board needs some tens of ms of load to reach"
                         " its operating clock)")
    ap.add_argument("--workload", default=None, help="workload name (default: the W=8 bf16 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modes", default="overlap,gemm_only,copy_only,serial,sdma",
                    help="modes to time; the overlapped steps always run (profiling runs use"
                         " 'overlap' alone so that every consumer-kernel launch is an overlapped step);"
                         " 'sdma' also times the overlap with the copy-engine producer")
    ap.add_argument("--configs", default="all",
                    help="per-workload blocks to measure: 'all', 'none', or a comma list of names")
    ap.add_argument("--config-reps", type=int, default=None,
                    help="interleaved calls per mode per block (default: 50 for MFMA-bound workloads,"
                         " 1000 for latency- and HBM-bound ones)")
    ap.add_argument("--block-modes", default="all",
                    help="profiling: the variants a block times ('all' or a comma list such as"
                         " 'gemm_only,overlap')")
    ap.add_argument("--skip-headline", action="store_true",
                    help="profiling: time only the blocks and print them (not a benchmark line)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the timed steps, run one plain device copy of this many MiB (a"
                         " known-size kernel that HBM byte counters are scaled against)")
    ap.add_argument("--producer", default="cu", choices=["cu", "sdma", "kernel"],
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


def rnd(x, d=1):
    return None if x is None else round(x, d)


# ------------------------------------------------------------------------ per-workload blocks

def make_workload(name):
    """(cfg, workload object, algorithmic bytes of the bare kernel, bytes the copy moves, flops)."""
    from allgather_gemm_persistent_amd import configs
    from allgather_gemm_persistent_amd.workload import (A2aWorkload, AgWorkload, ArWorkload, FfnWorkload,
                                                        RsWorkload)
    cfg = configs.CONFIGS[name]
    if cfg.op == "a2a":
        d = configs.make_a2a_data(cfg)
        w = A2aWorkload(cfg.world, cfg.rank, d["blocks"], d["counts"], d["b"], cfg.chunk_rows, cfg.dtype,
                        d["scale_a"], d["scale_b"])
        el = 1 if cfg.dtype == "fp8" else 2
        rows = sum(d["counts"])
        # the rows that hold tokens: read once, their products written; the weight read once
        bare = rows * cfg.k * el + cfg.k * cfg.n * el + rows * cfg.n * 2
        copy = (rows - d["counts"][cfg.rank]) * cfg.k * el
        return cfg, w, bare, copy, 2 * rows * cfg.k * cfg.n
    if cfg.op == "ag":
        d = configs.make_ag_data(cfg)
        w = AgWorkload(cfg.world, cfg.rank, d["shards"], d["b"], cfg.chunk_rows, cfg.dtype,
                       d["scale_a"], d["scale_b"])
        el = 1 if cfg.dtype == "fp8" else 2
        bare = cfg.m * cfg.k * el + cfg.k * cfg.n * el + cfg.m * cfg.n * 2
        copy = (cfg.world - 1) * cfg.m_shard * cfg.k * el
    elif cfg.op == "rs":
        d = configs.make_rs_data(cfg)
        w = RsWorkload(cfg.world, cfg.rank, d["a"], d["b"], d["peers"], cfg.chunk_rows)
        mb = cfg.m_block
        # A, B, the sent partial blocks, the incoming blocks read, the reduced block written
        bare = cfg.m * cfg.k * 2 + cfg.k * cfg.n * 2 + (cfg.world - 1) * mb * cfg.n * 4 * 2 + mb * cfg.n * 4
        copy = (cfg.world - 1) * mb * cfg.n * 4
    elif cfg.op == "ar":
        d = configs.make_ar_data(cfg)
        w = ArWorkload(cfg.world, cfg.rank, d["a"], d["b"], d["peers"], cfg.chunk_rows)
        # A, B, the partial sent, the incoming partials read, the reduced output written
        bare = cfg.m * cfg.k * 2 + cfg.k * cfg.n * 2 + cfg.m * cfg.n * 4 * (cfg.world - 1 + 2)
        copy = (cfg.world - 1) * cfg.m * cfg.n * 4
    elif cfg.op == "ffn":
        d = configs.make_ffn_data(cfg)
        w = FfnWorkload(cfg.world, cfg.rank, d["shards"], d["w1"], d["w2"], d["peers"], cfg.chunk_rows,
                        cfg.rs_chunk_rows)
        m, mb = cfg.m, cfg.m_shard
        # X, W1, h written and read, W2, the sent blocks, the incoming blocks read, the reduced block
        bare = (m * cfg.k1 * 2 + cfg.k1 * cfg.n1 * 2 + 2 * m * cfg.n1 * 2 + cfg.n1 * cfg.n2 * 2
                + (cfg.world - 1) * mb * cfg.n2 * 4 * 2 + mb * cfg.n2 * 4)
        copy = (cfg.world - 1) * mb * (cfg.k1 * 2 + cfg.n2 * 4)
    else:
        raise ValueError(cfg.op)
    return cfg, w, bare, copy, cfg.flops


def block_reps(name, reps=None):
    """Calls per mode in a workload's block: as given, else 50 for an MFMA-bound workload (long
    calls, small spread) and 1000 for a latency- or HBM-bound one (calls of tens of us)."""
    if reps is not None:
        return reps
    return 50 if BOUND[name] == "mfma" else 1000


def measure_block(name, reps, flush, only="all"):
    """Interleaved, cache-flushed timing of one workload's modes; returns the JSON block."""
    import torch

    from allgather_gemm_persistent_amd import binding as B
    cfg, w, bare_bytes, copy_bytes, flops = make_workload(name)
    ffn = cfg.op == "ffn"
    # (label, mode, pull setting or chain fusion, timed kernel launches per call)
    variants = [("overlap", "overlap", "auto", 1), ("gemm_only", "gemm_only", "auto", 1),
                ("copy_only", "copy_only", "auto", 1), ("serial", "serial", "auto", 1)]
    if name in PULL_VARIANTS:
        variants.append(("overlap_push", "overlap", "off", 1))
    if ffn:
        variants.append(("overlap_unfused", "overlap", "unfused", 2))
        variants.append(("gemm_only_unfused", "gemm_only", "unfused", 2))
    # the copy kernel beside the GEMM kernel (AGG_PRODUCER_KERNEL; the call falls back to copy
    # jobs inside the kernel where the GEMM kernel leaves it too few registers)
    variants.append(("overlap_copy_kernel", "overlap", "kernel", 1))
    variants.append(("copy_only_copy_kernel", "copy_only", "kernel", 0))
    if only != "all":
        variants = [v for v in variants if v[0] in only.split(",")]
        # on request only (traces): the copy engines as producer (AGG_PRODUCER_SDMA: one
        # hipMemcpyAsync and one stream write of the flag per chunk, beside the GEMM kernel).
        # Not in the timed blocks: its calls last milliseconds with the compute units nearly
        # idle, the board lowers its clock meanwhile, and the calls after it run slow.
        if "overlap_sdma" in only.split(","):
            variants.append(("overlap_sdma", "overlap", "sdma", 1))
    has_pull = cfg.op == "ag"
    ran = {}

    def setup(setting):
        B.agg_ctx_set_producer(w.ctx, setting if setting in ("kernel", "sdma") else "cu")
        if has_pull:
            B.agg_ctx_set_pull(w.ctx, "off" if setting == "off" else "auto")
        if ffn:
            B.agg_ctx_set_chain_fused(w.ctx, setting != "unfused")

    def run(mode):
        if ffn:
            w.run(mode, order=cfg.order(), rs_order=cfg.rs_order())
        else:
            w.run(mode, order=cfg.order())
    stream = torch.cuda.current_stream()
    try:
        for _ in range(3):                               # warm-up of every variant
            for label, mode, setting, _ in variants:
                setup(setting)
                run(mode)
                ran[label] = B.agg_ctx_last_producer(w.ctx)
        # a copy-only call times no launch under the copy kernel, one where the call fell back to
        # the in-kernel producer (its copy-only launch of the persistent kernel)
        variants = [(lb, md, st, (1 if ran.get(lb) == "cu" else 0) if lb == "copy_only_copy_kernel" else n)
                    for lb, md, st, n in variants]
        torch.cuda.synchronize()
        # the ctx keeps the durations of its last 256 launches: time the reps in batches that fit
        per_rep = sum(n for *_, n in variants)
        batch = max(1, 256 // max(per_rep, 1))
        ev, per_call = [], []                            # per call: (label, kernel ms)
        for b0 in range(0, reps, batch):
            B.agg_ctx_set_timing(w.ctx, True)            # clears the ring
            seq = []
            for i in range(b0, min(reps, b0 + batch)):
                for label, mode, setting, launches in variants:
                    setup(setting)
                    flush(i)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    run(mode)
                    e1.record(stream)
                    ev.append((label, e0, e1))
                    seq.append((label, launches))        # the timed kernel launches of the call
            torch.cuda.synchronize()
            n_launch = sum(n for _, n in seq)
            ks = B.agg_ctx_kernel_times(w.ctx, 256)
            ks = ks[len(ks) - n_launch:]
            j = 0
            for label, n in seq:                         # a call's kernel time: its launches' sum
                per_call.append((label, sum(ks[j:j + n])))
                j += n
        st = w.status()
        if st[0]:
            raise RuntimeError(f"{name}: a chunk wait gave up (flag {st[1]})")
        if ffn:
            bm, bn = 256, 256
        else:
            bm, bn = B.agg_tile_shape({"ag": 0, "a2a": 0, "rs": 1, "ar": 2}[cfg.op], cfg.dtype, cfg.m, cfg.n,
                                      cfg.k)
    finally:
        B.agg_ctx_set_timing(w.ctx, False)
        w.close()
    labels = [v[0] for v in variants]
    call_all = {lb: [a.elapsed_time(b) * 1e3 for q, a, b in ev if q == lb] for lb in labels}
    call = {lb: statistics.median(v) for lb, v in call_all.items()}
    if only != "all":
        return {"call_us": call, "kernel_us": None}
    kern_all = {lb: [k * 1e3 for q, k in per_call if q == lb] for lb in labels}
    kern = {lb: statistics.median(v) for lb, v in kern_all.items()}

    def spread(v):
        """[p10, p90] of a list of times"""
        if len(v) < 2:
            return [rnd(v[0], 2)] * 2 if v else None
        q = statistics.quantiles(v, n=10, method="inclusive")
        return [rnd(q[0], 2), rnd(q[8], 2)]
    R = call["overlap"] / call["gemm_only"]
    eta = (call["serial"] - call["overlap"]) / min(call["copy_only"], call["gemm_only"])
    bound = BOUND[name]

    def roof(kernel_us, bytes_):
        if bound == "mfma":
            peak = PEAK_FP8_TFLOPS if cfg.dtype == "fp8" else PEAK_BF16_TFLOPS
            a = flops / (kernel_us * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": rnd(a), "peak": peak, "unit": "TFLOP/s", "frac": rnd(a / peak, 4)}
        if bound == "hbm":
            a = bytes_ / (kernel_us * 1e-6) / 1e9
            return {"bound": "hbm", "achieved": rnd(a), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": rnd(a / PEAK_HBM_GBS, 4), "bytes": bytes_}
        return {"bound": "latency", "achieved": rnd(kernel_us, 2), "peak": None, "unit": "us", "frac": None}

    block = {
        "op": cfg.op, "dtype": cfg.dtype, "m": cfg.m,
        **({"k1": cfg.k1, "n1": cfg.n1, "n2": cfg.n2} if ffn else {"n": cfg.n, "k": cfg.k}),
        "world": cfg.world, "chunk_rows": cfg.chunk_rows, "tile": [bm, bn], "reps": reps,
        "cache_flushed": True,
        "call_us": {lb: rnd(v, 2) for lb, v in call.items()},
        "kernel_us": {lb: rnd(v, 2) for lb, v in kern.items()},
        "call_us_p10_p90": {lb: spread(v) for lb, v in call_all.items()},
        "kernel_us_p10_p90": {lb: spread(v) for lb, v in kern_all.items()},
        "R": rnd(R, 3), "eta": rnd(eta, 3),
        "tflops_overlap": rnd(flops / (call["overlap"] * 1e-6) / 1e12, 2),
        "roofline_bare": roof(kern["gemm_only"], bare_bytes),
        # the overlapped launch also reads every remote chunk from its peer and writes it into
        # the symmetric buffer (CU producer)
        "roofline_overlap": roof(kern["overlap"], bare_bytes + 2 * copy_bytes),
    }
    if cfg.op == "a2a":
        block["token_rows"] = flops // (2 * cfg.k * cfg.n)
        block["note_a2a"] = ("flops and bytes count the rows that hold tokens; tiles that straddle a"
                             " slot's count also compute the rows past it")
    if ffn:
        block["fusion_speedup"] = rnd(call["overlap_unfused"] / call["overlap"], 3)
        block["fusion_speedup_bare"] = rnd(call["gemm_only_unfused"] / call["gemm_only"], 3)
        block["note"] = ("overlap / gemm_only: both layers in one launch over the tile dependency graph;"
                         " *_unfused: the same tiles as two launches (all of layer 1, then all of"
                         " layer 2); fusion_speedup = unfused / fused call time")
    if "overlap_copy_kernel" in call:
        block["R_copy_kernel"] = rnd(call["overlap_copy_kernel"] / call["gemm_only"], 3)
        block["copy_kernel_producer_ran"] = ran.get("overlap_copy_kernel")
    if "overlap_push" in call:
        block["R_push"] = rnd(call["overlap_push"] / call["gemm_only"], 3)
        block["roofline_overlap_push"] = roof(kern["overlap_push"], bare_bytes + 2 * copy_bytes)
        block["note"] = ("overlap = the automatic choice (pulled: tiles read remote rows from the peers'"
                         " blocks, which on one GPU cost nothing like a link); overlap_push = every"
                         " remote tile waits for its chunks' flags")
    return block


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

    if args.skip_headline:
        torch.cuda.set_stream(torch.cuda.Stream())
        flush = cache_flush()
        names = list(BOUND) if args.configs == "all" else args.configs.split(",")
        out = {n: measure_block(n, block_reps(n, args.config_reps), flush, args.block_modes) for n in names}
        print(json.dumps(out), flush=True)
        return
    name = args.workload or configs.HEADLINE
    cfg = configs.CONFIGS[name]
    assert cfg.op == "ag", "the headline measures AllGather+GEMM workloads"
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
        # clears the ring: only timed launches count; launches 0, every, 2 * every, ... carry
        # the timing events
        # (at most 256 timed launches: the ring holds the last 256)
        every = max(1, min(8, args.steps // 8), -(-args.steps // 256))
        B.agg_ctx_set_timing(w.ctx, every)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            w.run("overlap", order=order)
        torch.cuda.synchronize()
        t_ovl = (time.perf_counter() - t0) / args.steps * 1e6
        st = w.status()
        if st[0]:
            raise RuntimeError(f"overlap: a chunk wait gave up (flag {st[1]})")
        kms = B.agg_ctx_kernel_times(w.ctx, args.steps)
        assert len(kms) == min(256, (args.steps + every - 1) // every), (len(kms), args.steps, every)
        k_ovl_us = statistics.mean(kms) * 1e3
        # context: the same steps with no timing events at all (the sampled launches above
        # carry them, which costs each of those launches some microseconds)
        B.agg_ctx_set_timing(w.ctx, False)
        t_ovl_untimed = time_mode(w, "overlap", order, args.steps, 0)
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
        other = {"cu": "sdma", "sdma": "cu", "kernel": "cu"}[args.producer]
        t_ovl_other = None
        if other in modes:
            B.agg_ctx_set_producer(w.ctx, other)
            t_ovl_other = time_mode(w, "overlap", order, args.steps, args.warmup)
            B.agg_ctx_set_producer(w.ctx, args.producer)
            # the copy-engine calls leave the compute units nearly idle for milliseconds and the
            # board lowers its clock: bring it back up before the blocks
            for _ in range(args.warmup):
                w.run("overlap", order=order)
            torch.cuda.synchronize()
    finally:
        B.agg_ctx_set_timing(w.ctx, False)
        w.close()

    # per-workload blocks, each call after a cache-evicting write and read
    blocks = {}
    if args.configs != "none":
        names = list(BOUND) if args.configs == "all" else args.configs.split(",")
        names = [n for n in names if n in configs.CONFIGS]
        flush = cache_flush()
        for n in names:
            blocks[n] = measure_block(n, block_reps(n, args.config_reps), flush, args.block_modes)
            print(f"block {n}: R {blocks[n]['R']} bare {blocks[n]['kernel_us']['gemm_only']} us",
                  file=sys.stderr, flush=True)
        del flush

    flops = cfg.flops
    value = flops / (t_ovl * 1e-6) / 1e12
    achieved = flops / (k_ovl_us * 1e-6) / 1e12
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
        "overlap": {"t_ovl_us": round(t_ovl, 1),
                    "t_ovl_without_timing_events_us": rnd(t_ovl_untimed),
                    "t_gemm_us": rnd(t_gemm),
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
        "roofline": {"bound": BOUND.get(name, "mfma"), "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(TRAFFIC_RECORDS.get(name, "")),
                     "traffic_unit": "bytes per launch",
                     "kernel": "agg::gemm_kernel (overlap launch)",
                     "kernel_us": round(k_ovl_us, 1),
                     "kernel_us_timed_launches": f"every {every}th of the {args.steps} timed steps"
                     if every > 1 else f"all {args.steps} timed steps",
                     "warm_caches": True,
                     "gemm_only_frac": rnd(flops / (k_gemm_us * 1e-6) / 1e12 / peak, 4)
                     if k_gemm_us else None},
        "configs": blocks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, data)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
