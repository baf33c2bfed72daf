"""AllGather+GEMM on the GPU through the C ABI, compared with the CPU oracle.

Parity bar: bf16 |C - ref| <= 1e-2 + 1e-2 |ref|, fp8 <= 2e-2 + 2e-2 |ref| (ref = oracle on the
same dequantised values); bit-exact for the gather buffer, the flags, tile bookkeeping, and
wherever the exact product is representable (integer inputs, identity weight).
"""

import numpy as np
import pytest
import torch

from allgather_gemm_persistent_amd import binding as B
from allgather_gemm_persistent_amd import configs, inputs
from allgather_gemm_persistent_amd.workload import AgWorkload
from oracle import agg_oracle as O

from helpers import BF16_TOL, FP8_TOL, assert_close, bits_equal, raw, small_ag_data, to_f64

pytestmark = pytest.mark.gpu

TILES = [(256, 256), (256, 224), (128, 128), (128, 64), (64, 64)]
PRODUCERS = ["cu", "sdma", "kernel"]


def _oracle_c(shards, b, dtype, sa, sb):
    return O.ag_gemm_ref([raw(s) for s in shards], raw(b), dtype, sa, sb)


def _tol(dtype):
    return FP8_TOL if dtype == "fp8" else BF16_TOL


def _alloc(regs):
    return (regs + 7) // 8 * 8


def test_register_counts_and_kernel_producer_choice(gpu):
    """The copy-kernel producer runs beside the GEMM kernel only if both fit in one SIMD's 512
    registers per lane. The counts the runtime reports must include the accumulation registers
    (the 256x256 kernels hold a 256-register accumulator per lane), else the choice would put
    the copy kernel where it cannot be resident; the copy kernel itself must be small. A call
    runs the copy kernel exactly where the counts fit, and the CU producer otherwise."""
    g, c = B.agg_kernel_regs(0, "bf16", 256, 256)
    assert 256 < g <= 512 and 0 < c <= 64, (g, c)
    g, _ = B.agg_kernel_regs(1, "bf16", 256, 256)
    assert 256 < g <= 512, g
    world, ms, k, n = 2, 128, 256, 256
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=3)
    for tile in [(256, 256), (256, 224), (64, 64)]:
        w = AgWorkload(world, 0, shards, b, chunk_rows=32, tile=tile, producer="kernel")
        try:
            assert B.agg_ctx_last_producer(w.ctx) is None
            w.run("overlap")
            assert w.status() == (0, -1)
            g, c = B.agg_kernel_regs(0, "bf16", *tile)
            want = "kernel" if _alloc(g) + _alloc(c) <= 512 else "cu"
            assert B.agg_ctx_last_producer(w.ctx) == want, (tile, g, c)
            w.run("overlap", delay_us=inputs.delays_us((world - 1) * ms // 32, 5, 20))
            assert w.status() == (0, -1)
            assert B.agg_ctx_last_producer(w.ctx) == "cu"          # delays: copy jobs in-kernel
        finally:
            w.close()


@pytest.mark.parametrize("mode", ["overlap", "serial", "gemm_only"])
def test_kernel_producer_on_a_side_stream(gpu, mode):
    """On a stream of the caller's own (not the legacy default one) the consumer kernel runs on
    that stream beside the copy kernel; every op gives the bits the in-kernel producer gives."""
    from allgather_gemm_persistent_amd.workload import A2aWorkload, ArWorkload, RsWorkload
    side = torch.cuda.Stream()
    rng = 211
    shards, b, _, _ = small_ag_data(4, 96, 256, 224, "bf16", seed=rng)
    a, _ = inputs.draw({"kind": "normal", "std": 1.0}, (384, 256), "bf16", rng + 1)
    peers_rs, _ = inputs.draw({"kind": "normal", "std": 1.0}, (4, 96, 224), "f32", rng + 2)
    peers_ar, _ = inputs.draw({"kind": "normal", "std": 1.0}, (4, 384, 224), "f32", rng + 3)
    makers = {
        "ag": lambda prod: AgWorkload(4, 1, shards, b, 32, tile=(256, 224), producer=prod),
        "rs": lambda prod: RsWorkload(4, 1, a, b, peers_rs, 32, tile=(64, 64), producer=prod),
        "ar": lambda prod: ArWorkload(4, 1, a, b, peers_ar, 32, tile=(64, 64), producer=prod),
        "a2a": lambda prod: A2aWorkload(4, 1, shards, [96, 40, 0, 77], b, 32, tile=(256, 224), producer=prod),
    }
    for op, make in makers.items():
        outs = {}
        for prod in ("cu", "kernel"):
            w = make(prod)
            try:
                if mode == "gemm_only":
                    w.run("overlap")                  # gather first; then time the bare kernel
                with torch.cuda.stream(side):
                    w.run(mode, stream=side)
                torch.cuda.synchronize()
                assert w.status() == (0, -1), (op, prod, mode)
                assert B.agg_ctx_last_producer(w.ctx) == prod, (op, prod)
                res = w.c if op in ("ag", "a2a") else w.out
                outs[prod] = res.clone()
            finally:
                w.close()
        if op == "a2a":
            rows = [p * 96 + i for p, cnt in enumerate([96, 40, 0, 77]) for i in range(cnt)]
            assert bits_equal(outs["cu"][rows], outs["kernel"][rows]), (op, mode)
        else:
            assert bits_equal(outs["cu"], outs["kernel"]), (op, mode)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", TILES)
def test_identity_weight_gives_gather_bitexact(gpu, dtype, tile):
    """B = I (K = N): every output is one product with 1, so C equals the gathered A exactly
    (fp8 values are exactly representable in bf16). Catches any row/column/layout mix-up."""
    world, ms, k = 3, 96, 192
    shards, _, _, _ = small_ag_data(world, ms, k, k, dtype, seed=5)
    eye = torch.eye(k, dtype=torch.float32)
    b = eye.to(torch.bfloat16) if dtype == "bf16" else eye.to(torch.float8_e4m3fn)
    w = AgWorkload(world, 1, shards, b, chunk_rows=32, dtype=dtype, tile=tile)
    try:
        w.run("overlap", order=inputs.seeded_order(world, 1, 3, 11))
        assert w.status() == (0, -1)
        g = torch.cat([s.to(torch.float32) for s in shards]).to(torch.bfloat16)
        assert bits_equal(w.c, g)
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", TILES)
def test_integer_inputs_bitexact(gpu, dtype, tile):
    """Entries in {-2..2}: every fp32 partial sum is an exact integer (|sum| <= 4K < 2^24), so
    the kernel's output must equal the round-to-nearest-even bf16 of the exact product, bit for
    bit, whatever order the MFMA sums in."""
    world, ms, k, n = 2, 160, (520 if dtype == "bf16" else 528), (200 if dtype == "bf16" else 208)
    shards, b, _, _ = small_ag_data(world, ms, k, n, dtype, seed=9, kind="int")
    w = AgWorkload(world, 0, shards, b, chunk_rows=40, dtype=dtype, tile=tile)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        exact = _oracle_c(shards, b, dtype, 1.0, 1.0)
        want = O.encode_bf16_rne(exact)
        assert np.array_equal(raw(w.c), want)
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("mode", ["overlap", "serial"])
@pytest.mark.parametrize("producer", PRODUCERS)
def test_ragged_shapes_vs_oracle(gpu, dtype, tile, mode, producer):
    """Sizes that are not multiples of any tile: ragged rows, columns and K tail."""
    world, rank, ms, cr, k, n = 3, 1, 200, 40, 328, 264
    if dtype == "fp8":
        k, n = 336, 272     # fp8 rows of B (n bytes) are whole 16-byte chunks
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=21)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                   tile=tile, producer=producer)
    try:
        w.run(mode, order=inputs.seeded_order(world, rank, ms // cr, 3))
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), "C")
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_order_and_mode_invariance_bitexact(gpu, producer):
    """C is bit-identical for every arrival order and every mode (each tile's arithmetic does
    not depend on when its rows arrived)."""
    world, rank, ms, cr, k, n = 4, 2, 256, 64, 1024, 512
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=33)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, tile=(128, 128), producer=producer)
    try:
        cps = ms // cr
        orders = [None, inputs.ring_order(world, rank, cps)[::-1]] + \
            [inputs.seeded_order(world, rank, cps, s) for s in (1, 2, 3)]
        outs = []
        for o in orders:
            for mode in ("overlap", "serial", "gemm_only"):
                w.c.zero_()
                w.run(mode, order=o)
                outs.append(w.c.clone())
        assert w.status() == (0, -1)
        for c in outs[1:]:
            assert bits_equal(c, outs[0])
        assert_close(to_f64(outs[0]), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_gather_and_flags_bitexact(gpu, producer):
    world, rank, ms, cr, k, n = 5, 3, 96, 16, 256, 128
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=41)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, producer=producer)
    try:
        for _ in range(3):
            w.run("overlap", order=inputs.seeded_order(world, rank, ms // cr, 8))
        assert w.status() == (0, -1)
        e = B.agg_ctx_epoch(w.ctx)
        assert e == 3
        want_g = O.gather_ref([raw(s) for s in shards])
        assert np.array_equal(raw(w.gather), want_g)
        flags = w.flags.cpu().numpy().astype(np.uint32)
        cps = ms // cr
        assert (flags == e).all(), flags      # the local shard's flags too
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_trace_each_tile_once_and_flags_seen(gpu, producer):
    world, rank, ms, cr, k, n = 4, 0, 128, 32, 256, 256
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=51)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, tile=(64, 64), producer=producer)
    try:
        if producer == "cu":
            B.agg_ctx_set_pull(w.ctx, "off")        # the flag waits are what this test traces
        tiles = (world * ms // 64) * (n // 64)
        buf = torch.zeros(tiles * 8, dtype=torch.int32, device="cuda")
        B.agg_set_trace(w.ctx, buf, buf.numel() * 4)
        order = inputs.seeded_order(world, rank, ms // cr, 4)
        w.run("overlap", order=order)
        assert w.status() == (0, -1)
        rec = buf.cpu().numpy().astype(np.uint32).reshape(-1, 8)
        assert (rec[:, 4] == 1).all()                 # visited exactly once
        e = B.agg_ctx_epoch(w.ctx)
        row_order, _ = O.ag_mtile_order(world, rank, ms, cr, order, 64)
        assert B.agg_ag_row_tile_order(world, rank, ms, cr, order, 64) == row_order
        cps = ms // cr
        for mt in range(world * ms // 64):
            need_remote = any(c // cps != rank for c in O.covering_chunks(mt * 64, mt * 64 + 64, cr))
            for nt in range(n // 64):
                r = rec[mt * (n // 64) + nt]
                if need_remote:
                    assert r[3] >= e and r[3] != 0xFFFFFFFF
                else:
                    assert r[3] == 0xFFFFFFFF
        # within each claim list, positions follow the row-tile order
        for lst in np.unique(rec[:, 0]):
            sel = rec[rec[:, 0] == lst]
            assert len(np.unique(sel[:, 1])) == len(sel)
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", [(64, 64), (128, 64), (128, 128), (256, 224)])
@pytest.mark.parametrize("rank", [0, 2])
def test_pull_matches_push_bitexact(gpu, dtype, tile, rank):
    """Pulled calls (tiles read remote rows from the peers' blocks while extra workgroups fill
    the gather buffer) give the same bits as pushed and serialized calls, the same gather
    buffer and the same flags, and match the oracle."""
    world, cr, k, n = 3, 64, (320 if dtype == "bf16" else 384), (200 if dtype == "bf16" else 208)
    ms = tile[0] * 2
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=91)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                   tile=tile)
    try:
        order = inputs.seeded_order(world, rank, ms // cr, 5)
        outs = {}
        for pull, mode in (("on", "overlap"), ("off", "overlap"), ("on", "serial")):
            B.agg_ctx_set_pull(w.ctx, pull)
            w.c.zero_()
            w.gather[[r for r in range(world * ms) if r // ms != rank]] = 0
            w.run(mode, order=order)
            assert w.status() == (0, -1)
            outs[(pull, mode)] = w.c.clone()
            assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards])), (pull, mode)
            flags = w.flags.cpu().numpy().astype(np.uint32)
            e = B.agg_ctx_epoch(w.ctx)
            cps = ms // cr
            assert (flags == e).all(), (pull, mode, flags)
        ref = outs[("on", "overlap")]
        for key, c in outs.items():
            assert bits_equal(c, ref), key
        assert_close(to_f64(ref), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), "C")
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", [(64, 64), (128, 64), (128, 128)])
@pytest.mark.parametrize("world,ms,rank", [(8, 16, 0), (8, 16, 5), (3, 48, 1)])
def test_pull_by_row_groups_matches_push_bitexact(gpu, dtype, tile, world, ms, rank):
    """Shards of a multiple of 16 rows inside taller tiles (the decode shape): each 16-row load
    group of a pulled tile reads its own shard's block. Same bits, gather buffer and flags as a
    pushed call, and the oracle."""
    cr, k, n = 16, (512 if dtype == "bf16" else 1024), (200 if dtype == "bf16" else 208)
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=93)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                   tile=tile)
    try:
        order = inputs.seeded_order(world, rank, ms // cr, 7)
        outs = []
        for pull in ("on", "off"):
            B.agg_ctx_set_pull(w.ctx, pull)
            w.c.zero_()
            w.gather[[r for r in range(world * ms) if r // ms != rank]] = 0
            w.run("overlap", order=order)
            assert w.status() == (0, -1)
            outs.append(w.c.clone())
            assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards])), pull
            flags = w.flags.cpu().numpy().astype(np.uint32)
            e = B.agg_ctx_epoch(w.ctx)
            cps = ms // cr
            assert (flags == e).all(), (pull, flags)
        assert bits_equal(outs[0], outs[1])
        assert_close(to_f64(outs[0]), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), "C")
    finally:
        w.close()


def test_withheld_chunks_time_out_then_recover(gpu):
    """Flags that never reach the epoch make the waits give up (status, failed flag id) instead
    of hanging; after agg_ctx_reset the next call is correct."""
    world, rank, ms, cr, k, n = 2, 0, 128, 64, 256, 128
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=61)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr)
    try:
        B.agg_ctx_set_timeout_us(w.ctx, 20000)
        B.agg_ctx_set_epoch(w.ctx, 7)          # flags are 0 < 7: as if chunks never arrived
        w.run("gemm_only")
        status, failed = w.status()
        assert status & 1 and failed in (2, 3)
        B.agg_ctx_reset(w.ctx, torch.cuda.current_stream())
        assert w.status() == (0, -1)
        w.run("overlap")
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_stale_epoch_is_not_accepted(gpu, producer):
    """A flag holding the previous epoch does not satisfy the current call's wait."""
    world, rank, ms, cr, k, n = 2, 1, 64, 64, 128, 128
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=71)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, producer=producer)
    try:
        w.run("copy_only")                      # flags = 1
        B.agg_ctx_set_timeout_us(w.ctx, 20000)
        B.agg_ctx_reset(w.ctx, torch.cuda.current_stream())
        w.flags.fill_(4)                        # an older epoch than the next one
        B.agg_ctx_set_epoch(w.ctx, 5)
        w.run("gemm_only")                      # waits for >= 5
        status, failed = w.status()
        assert status & 1 and failed == 0
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_epoch_wraps_and_stays_correct(gpu, producer):
    world, rank, ms, cr, k, n = 3, 0, 64, 32, 128, 64
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=81)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, producer=producer)
    try:
        B.agg_ctx_set_epoch(w.ctx, 0xFFFFFFFC)
        ref = _oracle_c(shards, b, "bf16", 1, 1)
        seen = []
        for i in range(4):
            w.c.zero_()
            w.run("overlap", order=inputs.seeded_order(world, rank, ms // cr, i + 1))
            assert w.status() == (0, -1)
            assert_close(to_f64(w.c), ref, BF16_TOL, f"C call {i}")
            seen.append(B.agg_ctx_epoch(w.ctx))
        assert seen == [0xFFFFFFFD, 0xFFFFFFFE, 1, 2]
        flags = w.flags.cpu().numpy()
        assert (flags == 2).all(), flags
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_host_delays(gpu, producer):
    world, rank, ms, cr, k, n = 4, 0, 128, 32, 512, 256
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=91)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, producer=producer)
    try:
        nrem = (world - 1) * ms // cr
        w.run("overlap", delay_us=inputs.delays_us(nrem, 5, 200))
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_degenerate_sizes(gpu, producer):
    # world 1: a plain GEMM, nothing to gather
    shards, b, _, _ = small_ag_data(1, 100, 64, 72, "bf16", seed=3)
    w = AgWorkload(1, 0, shards, b, chunk_rows=10, producer=producer)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
    finally:
        w.close()
    # k = 0: C is zero
    shards = [torch.zeros(16, 0, dtype=torch.bfloat16) for _ in range(2)]
    b = torch.zeros(0, 32, dtype=torch.bfloat16)
    w = AgWorkload(2, 0, shards, b, chunk_rows=8, producer=producer)
    try:
        w.c.fill_(1.0)
        w.run("overlap")
        assert w.status() == (0, -1)
        assert (w.c.float() == 0).all()
    finally:
        w.close()
    # m_shard = 0: nothing at all
    ctx = B.agg_ctx_create(0)
    try:
        B.ag_gemm(ctx, 2, 0, 0, 64, 64, 1, "bf16", 1.0, 1.0, [0, 0], None, None, None, None)
    finally:
        B.agg_ctx_destroy(ctx)


def test_put_signal_primitive(gpu):
    src = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    flag = torch.zeros(4, dtype=torch.int32, device="cuda")
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    B.agg_put_signal(dst, src, src.numel() * 4, flag[2:], 1234, cs)
    cs.synchronize()
    assert torch.equal(dst, src) and flag.tolist() == [0, 0, 1234, 0]


@pytest.mark.parametrize("streams", [1, 3, 8])
def test_copy_stream_counts(gpu, streams):
    world, rank, ms, cr, k, n = 8, 6, 64, 16, 256, 128
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=95)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, producer="sdma")
    try:
        B.agg_ctx_set_copy_streams(w.ctx, streams)
        w.run("overlap", order=inputs.seeded_order(world, rank, ms // cr, streams))
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
        assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards]))
    finally:
        w.close()


@pytest.mark.parametrize("copy_wgs,piece_kib", [(1, 1), (3, 2), (0, 3), (0, 1024)])
@pytest.mark.parametrize("mode", ["overlap", "serial", "copy_only"])
def test_cu_producer_pieces_and_workgroups(gpu, copy_wgs, piece_kib, mode):
    """In-kernel producer: chunks cut into many pieces, copied by one, a few or every workgroup;
    the gather buffer and flags are bit-exact and C matches the oracle."""
    world, rank, ms, cr, k, n = 4, 1, 96, 24, 264, 136      # chunk = 24 x 528 B (not a piece multiple)
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=97)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, tile=(64, 64), producer="cu")
    try:
        B.agg_ctx_set_producer(w.ctx, "cu", copy_wgs, piece_kib)
        order = inputs.seeded_order(world, rank, ms // cr, 5)
        for _ in range(2):
            w.c.zero_()
            w.run(mode, order=order)
        assert w.status() == (0, -1)
        e = B.agg_ctx_epoch(w.ctx)
        assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards]))
        flags = w.flags.cpu().numpy().astype(np.uint32)
        cps = ms // cr
        assert (flags == e).all(), flags      # the local shard's flags too
        if mode != "copy_only":
            assert_close(to_f64(w.c), _oracle_c(shards, b, "bf16", 1, 1), BF16_TOL, "C")
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", [(128, 128), (128, 64), (64, 64), (256, 224)])
@pytest.mark.parametrize("ksplit", [2, 3, 16])
def test_split_k_vs_oracle(gpu, dtype, tile, ksplit):
    """Split-K: every part's K range (the last one shorter), partials summed in part order;
    C within tolerance, bit-identical on a second call, and bit-exact on integer inputs. (A
    256 x 224 tile is never split: the request is ignored and the result must not change.)"""
    world, rank, ms, cr, n = 2, 1, 96, 32, (200 if dtype == "bf16" else 208)
    k = 1000 if dtype == "bf16" else 1040          # 32 bf16 slices (last partial) / 9 fp8 slices
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=101)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                   tile=tile)
    try:
        B.agg_ctx_set_split(w.ctx, ksplit)
        order = inputs.seeded_order(world, rank, ms // cr, 7)
        w.run("overlap", order=order)
        first = w.c.clone()
        w.c.zero_()
        w.run("overlap", order=order)
        assert w.status() == (0, -1)
        assert bits_equal(w.c, first)
        assert_close(to_f64(w.c), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), "C")
    finally:
        w.close()
    # integer inputs: every partial and every sum is exact, so the split changes no bit
    shards, b, _, _ = small_ag_data(world, ms, k, n, dtype, seed=103, kind="int")
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, tile=tile)
    try:
        B.agg_ctx_set_split(w.ctx, ksplit)
        w.run("overlap")
        assert w.status() == (0, -1)
        want = O.encode_bf16_rne(_oracle_c(shards, b, dtype, 1.0, 1.0))
        assert np.array_equal(raw(w.c), want)
    finally:
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_split_k_more_parts_than_workgroups(gpu, dtype):
    """Split-K with more parts than workgroups (1024 parts of 64 x 64 tiles): the parts cannot
    all run at once, so the last part of each tile sums it alone. Same bar as above."""
    world, rank, ms, cr, n = 2, 0, 512, 128, (200 if dtype == "bf16" else 208)
    k = 1000 if dtype == "bf16" else 1040
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=107)
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                   tile=(64, 64))
    try:
        B.agg_ctx_set_split(w.ctx, 16)
        w.run("overlap")
        assert w.status() == (0, -1)
        assert_close(to_f64(w.c), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), "C")
    finally:
        w.close()
    shards, b, _, _ = small_ag_data(world, ms, k, n, dtype, seed=109, kind="int")
    w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, tile=(64, 64))
    try:
        B.agg_ctx_set_split(w.ctx, 16)
        w.run("serial")
        assert w.status() == (0, -1)
        want = O.encode_bf16_rne(_oracle_c(shards, b, dtype, 1.0, 1.0))
        assert np.array_equal(raw(w.c), want)
    finally:
        w.close()


# ---------------------------------------------------------------------- the workload configs

AG_CONFIGS = ["ag_w2_256x256x512_bf16", "ag_w8_4096x3584x8192_bf16",
              "ag_w8_128x3584x8192_bf16_decode", "ag_w8_8192x7168x8192_fp8"]
_REFS = {}


def _config_ref(name, d):
    if name not in _REFS:
        cfg = configs.CONFIGS[name]
        _REFS[name] = _oracle_c(d["shards"], d["b"], cfg.dtype, d["scale_a"], d["scale_b"])
    return _REFS[name]


def _remote_rows(w):
    ms = w.m_shard
    return [r for r in range(w.world * ms) if r // ms != w.rank]


def _check_gather_and_flags(w, d, what):
    assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in d["shards"]])), what
    e = B.agg_ctx_epoch(w.ctx)
    flags = w.flags.cpu().numpy().astype(np.uint32)
    assert (flags == e).all(), (what, e, flags)


@pytest.mark.parametrize("name", AG_CONFIGS)
def test_config_vs_oracle(gpu, name):
    """Each AllGather+GEMM workload at full size: the overlapped call (its automatic choices),
    then every other path of the same call, each after clearing C and the remote rows of the
    gather buffer: serialized, bare GEMM, the flag-gated push (pull off: every remote tile waits
    on its chunks' flags) and both producers. C matches the oracle and every run gives the same
    bits; the gather buffer is the rank-order concatenation and every flag holds the epoch."""
    cfg = configs.CONFIGS[name]
    d = configs.make_ag_data(cfg)
    w = AgWorkload(cfg.world, cfg.rank, d["shards"], d["b"], cfg.chunk_rows, cfg.dtype,
                   d["scale_a"], d["scale_b"])
    rows = _remote_rows(w)
    try:
        print(f"config {name}: overlap", flush=True)
        w.run("overlap", order=cfg.order(), delay_us=cfg.delays())
        assert w.status() == (0, -1)
        c_ovl = w.c.clone()
        assert_close(to_f64(c_ovl), _config_ref(name, d), _tol(cfg.dtype), name)
        _check_gather_and_flags(w, d, "overlap")
        runs = [("cu", "auto", "serial"), ("cu", "auto", "gemm_only"), ("cu", "off", "overlap"),
                ("sdma", "auto", "overlap"), ("sdma", "auto", "serial"), ("kernel", "auto", "overlap")]
        for producer, pull, mode in runs:
            print(f"config {name}: {producer} pull={pull} {mode}", flush=True)
            B.agg_ctx_set_producer(w.ctx, producer)
            B.agg_ctx_set_pull(w.ctx, pull)
            w.c.zero_()
            if mode != "gemm_only":
                w.gather[rows] = 0
            w.run(mode, order=cfg.order())
            assert w.status() == (0, -1), (producer, pull, mode)
            assert bits_equal(w.c, c_ovl), (producer, pull, mode)
            _check_gather_and_flags(w, d, (producer, pull, mode))
    finally:
        w.close()


def _alt_data(cfg, seed_shift):
    import dataclasses
    return configs.make_ag_data(dataclasses.replace(cfg, seed=cfg.seed + seed_shift))


@pytest.mark.parametrize("producer", PRODUCERS)
def test_stale_data_reuse_full_size(gpu, producer):
    """Fifty overlapped calls at the W=8 4096 x 3584 x 8192 bf16 size alternate two seeded
    datasets (different peer blocks, local shard and weight) over the same gather buffer, flags
    and C, none of them cleared between calls. A tile that read a row before its chunk landed,
    or skipped its wait, would reproduce the other dataset's rows. The first call of each dataset
    is compared with the oracle; every later one must repeat its bits exactly."""
    cfg = configs.CONFIGS["ag_w8_4096x3584x8192_bf16"]
    data = [configs.make_ag_data(cfg), _alt_data(cfg, 100)]
    dev = torch.device("cuda")
    peers = [[s.to(dev) if p != cfg.rank else 0 for p, s in enumerate(d["shards"])] for d in data]
    local = [d["shards"][cfg.rank].to(dev) for d in data]
    w = AgWorkload(cfg.world, cfg.rank, data[0]["shards"], data[0]["b"], cfg.chunk_rows, cfg.dtype,
                   producer=producer)
    bs = [w.device_weight(d["b"]) for d in data]
    ms = cfg.m_shard
    first = [None, None]
    try:
        order = cfg.order()
        for i in range(50):
            j = i % 2
            w.gather[cfg.rank * ms:(cfg.rank + 1) * ms].copy_(local[j])   # the caller's shard
            B.ag_gemm(w.ctx, cfg.world, cfg.rank, ms, cfg.n, cfg.k, cfg.chunk_rows, "bf16", 1.0,
                      1.0, peers[j], w.gather, w.flags, bs[j], w.c, order=order, mode="overlap",
                      stream=torch.cuda.current_stream())
            if first[j] is None:
                assert w.status() == (0, -1)
                print(f"stale-data {producer}: dataset {j} against the oracle", flush=True)
                ref = _oracle_c(data[j]["shards"], data[j]["b"], "bf16", 1.0, 1.0)
                assert_close(to_f64(w.c), ref, BF16_TOL, f"dataset {j}")
                first[j] = w.c.clone()
            else:
                assert torch.equal(w.c, first[j]), f"call {i} (dataset {j}) differs from its first result"
        assert w.status() == (0, -1)
        flags = w.flags.cpu().numpy().astype(np.uint32)
        assert (flags == B.agg_ctx_epoch(w.ctx)).all()
        assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in data[1]["shards"]]))
    finally:
        w.close()


@pytest.mark.parametrize("mode", ["overlap", "gemm_only"])
def test_kernel_times_ring(gpu, mode):
    """With timing on, every consumer-kernel launch (or every n-th) leaves one duration in the
    ctx's ring (the launch carries its own start and end events), oldest first, and the results
    are those of the untimed calls; with timing off, reading the ring is a state error."""
    world, rank, ms, cr, k, n = 4, 1, 64, 32, 256, 128
    shards, b, sa, sb = small_ag_data(world, ms, k, n, "bf16", seed=501)
    w = AgWorkload(world, rank, shards, b, cr)
    try:
        w.run(mode)
        ref = w.c.clone()
        B.agg_ctx_set_timing(w.ctx, True)
        for _ in range(3):
            w.run(mode)
        torch.cuda.synchronize()
        times = B.agg_ctx_kernel_times(w.ctx, 8)
        assert len(times) == 3 and all(0.0 < t < 1000.0 for t in times), times
        assert bits_equal(w.c, ref)
        # every third launch: launches 1, 4 and 7 of seven
        B.agg_ctx_set_timing(w.ctx, 3)
        for _ in range(7):
            w.run(mode)
        torch.cuda.synchronize()
        times = B.agg_ctx_kernel_times(w.ctx, 8)
        assert len(times) == 3 and all(0.0 < t < 1000.0 for t in times), times
        assert bits_equal(w.c, ref)
        B.agg_ctx_set_timing(w.ctx, False)
        w.run(mode)
        torch.cuda.synchronize()
        with pytest.raises(B.AggError):
            B.agg_ctx_kernel_times(w.ctx, 8)
        assert w.status() == (0, -1)
    finally:
        B.agg_ctx_set_timing(w.ctx, False)
        w.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tile", [(256, 224), (256, 256), (128, 128), (128, 64)])
@pytest.mark.parametrize("mode", ["overlap", "serial", "gemm_only"])
def test_tail_split_bit_identical(gpu, dtype, tile, mode):
    """The tail split forced on (the last row tiles of the compute order in a second launch of
    the next smaller tile shape): C within the bar against the oracle and bit-identical to the
    single launch (same rows, same per-element K order), every flag at the epoch, and, with
    timing on, one duration for the call's two launches."""
    world, rank, ms, cr, k, n = 4, 1, 128, 32, 320, 448
    if dtype == "fp8":
        k = 384
    m = world * ms
    head, tail_ts = B.agg_tail_split(tile[0], tile[1], m, n, -(-m // tile[0]), 256, "on")
    assert head >= 1 and tail_ts[0] > 0, (tile, head, tail_ts)
    shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=41)
    order = inputs.seeded_order(world, rank, ms // cr, 5)
    outs = []
    for tail in ("off", "on"):
        w = AgWorkload(world, rank, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb,
                       tile=tile)
        try:
            B.agg_ctx_set_tail(w.ctx, tail)
            if mode == "gemm_only":
                w.run("copy_only", order=order)
            B.agg_ctx_set_timing(w.ctx, True)
            w.run(mode, order=order)
            torch.cuda.synchronize()
            times = B.agg_ctx_kernel_times(w.ctx, 8)
            assert len(times) == 1 and 0.0 < times[0] < 1000.0, times
            assert w.status() == (0, -1)
            assert_close(to_f64(w.c), _oracle_c(shards, b, dtype, sa, sb), _tol(dtype), ("C", tail))
            assert (w.flags.cpu().numpy() == B.agg_ctx_epoch(w.ctx)).all(), tail
            outs.append(w.c.clone())
        finally:
            w.close()
    assert bits_equal(outs[0], outs[1]), (dtype, tile, mode)


def test_tail_split_full_size_auto(gpu):
    """The 5120-row AllToAll workload's 320 tiles of 256 x 224 split automatically (16 row tiles in
    the first launch, 8 tail row tiles of 128 x 128 in the second); its C is bit-identical to the
    single launch."""
    cfg = configs.CONFIGS["a2a_w8_5120x3584x8192_bf16"]
    d = configs.make_a2a_data(cfg)
    from allgather_gemm_persistent_amd.workload import A2aWorkload
    rows = B.agg_a2a_row_tile_order(cfg.world, cfg.rank, cfg.cap, cfg.chunk_rows, d["counts"], cfg.order(), 256)
    head, tail_ts = B.agg_tail_split(256, 224, cfg.world * cfg.cap, cfg.n, len(rows), 256, "auto")
    assert (head, tail_ts) == (16, (128, 128)), (len(rows), head, tail_ts)
    outs = []
    for tail in ("off", "auto"):
        w = A2aWorkload(cfg.world, cfg.rank, d["blocks"], d["counts"], d["b"], cfg.chunk_rows, cfg.dtype,
                        d["scale_a"], d["scale_b"])
        try:
            B.agg_ctx_set_tail(w.ctx, tail)
            w.run("overlap", order=cfg.order())
            torch.cuda.synchronize()
            assert w.status() == (0, -1)
            outs.append(w.c.clone())
        finally:
            w.close()
    assert bits_equal(outs[0], outs[1])
