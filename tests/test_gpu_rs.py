"""GEMM+ReduceScatter on the GPU through the C ABI, compared with the CPU oracle.

Bar: |x - ref| <= 1e-2 + 1e-2 |ref| for `send` and `out` (fp32 results of bf16 products);
bit-exact for the receive buffer, the flags, and for integer-valued inputs (every fp32 sum
exact); `out` bit-identical for every arrival order (fixed summation order).
"""

import numpy as np
import pytest
import torch

from allgather_gemm_persistent_amd import binding as B
from allgather_gemm_persistent_amd import configs, inputs
from allgather_gemm_persistent_amd.workload import RsWorkload
from oracle import agg_oracle as O

from helpers import BF16_TOL, assert_close, raw, to_f64

pytestmark = pytest.mark.gpu

TILES = [(256, 256), (256, 224), (128, 128), (128, 64), (64, 64)]
PRODUCERS = ["cu", "sdma", "kernel"]


def _data(world, m, k, n, seed, kind="normal"):
    if kind == "int":
        d = {"kind": "int", "lo": -2, "hi": 2}
        a, _ = inputs.draw(d, (m, k), "bf16", seed)
        b, _ = inputs.draw(d, (k, n), "bf16", seed + 1)
        peers, _ = inputs.draw({"kind": "int", "lo": -100, "hi": 100}, (world, m // world, n), "f32", seed + 2)
    else:
        a, _ = inputs.draw({"kind": "normal", "std": 1.0}, (m, k), "bf16", seed)
        b, _ = inputs.draw({"kind": "normal", "std": 0.05}, (k, n), "bf16", seed + 1)
        peers, _ = inputs.draw({"kind": "normal", "std": 1.0}, (world, m // world, n), "f32", seed + 2)
    return a, b, peers


def _ref(w, a, b, peers):
    return O.gemm_rs_ref(raw(a), raw(b), peers.numpy(), w.world, w.rank)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("mode", ["overlap", "serial"])
@pytest.mark.parametrize("producer", PRODUCERS)
def test_ragged_vs_oracle(gpu, tile, mode, producer):
    world, rank, m, k, n, cr = 3, 1, 3 * 200, 328, 264, 40
    a, b, peers = _data(world, m, k, n, seed=7)
    w = RsWorkload(world, rank, a, b, peers, cr, tile=tile, producer=producer)
    try:
        w.run(mode, order=inputs.seeded_order(world, rank, 200 // cr, 5))
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(w.send[:world - 1]), send, BF16_TOL, "send")
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
    finally:
        w.close()


@pytest.mark.parametrize("tile", [(256, 256), (64, 64)])
def test_integer_inputs_bitexact(gpu, tile):
    world, rank, m, k, n, cr = 4, 2, 4 * 96, 512, 192, 32
    a, b, peers = _data(world, m, k, n, seed=17, kind="int")
    w = RsWorkload(world, rank, a, b, peers, cr, tile=tile)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert np.array_equal(to_f64(w.send[:world - 1]), send)
        assert np.array_equal(to_f64(w.out), out)
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_order_invariance_and_bookkeeping(gpu, producer):
    world, rank, m, k, n, cr = 8, 5, 8 * 64, 256, 256, 16
    a, b, peers = _data(world, m, k, n, seed=27)
    w = RsWorkload(world, rank, a, b, peers, cr, tile=(64, 64), producer=producer)
    try:
        cpb = (m // world) // cr
        outs, sends = [], []
        for s in (None, 1, 2, 3):
            order = None if s is None else inputs.seeded_order(world, rank, cpb, s)
            for mode in ("overlap", "serial"):
                w.out.zero_()
                w.run(mode, order=order)
                outs.append(w.out.clone())
                sends.append(w.send.clone())
        assert w.status() == (0, -1)
        for o, s in zip(outs[1:], sends[1:]):
            assert torch.equal(o, outs[0]) and torch.equal(s, sends[0])
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(outs[0]), out, BF16_TOL, "out")
        e = B.agg_ctx_epoch(w.ctx)
        rf = w.flags.cpu().numpy()
        sf = w.send_flags.cpu().numpy()
        assert (rf == e).all() and (sf == e).all(), (rf, sf)   # the local block's flags too
        recv = w.recv.cpu()
        for p in range(world):
            if p != rank:
                assert torch.equal(recv[p], peers[p])
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_world_one_and_k_zero(gpu, producer):
    a, b, peers = _data(1, 96, 64, 32, seed=37)
    w = RsWorkload(1, 0, a, b, peers, 32, producer=producer)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        _, out = _ref(w, a, b, peers)
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
    finally:
        w.close()
    a = torch.zeros(64, 0, dtype=torch.bfloat16)
    b = torch.zeros(0, 32, dtype=torch.bfloat16)
    peers = inputs.draw({"kind": "normal", "std": 1.0}, (2, 32, 32), "f32", 3)[0]
    w = RsWorkload(2, 1, a, b, peers, 16, producer=producer)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        assert torch.equal(w.out.cpu(), peers[0])
    finally:
        w.close()


def test_config_c3_vs_oracle(gpu):
    """The W=8 8192 x 8192 x 3584 GEMM+ReduceScatter at full size, overlapped, against the oracle;
    then serialized and with the copy-engine producer (receive buffer cleared first): the same
    bits in `send` and `out`, the receive buffer holding every peer's block, all flags at the
    epoch."""
    cfg = configs.CONFIGS["rs_w8_8192x8192x3584_bf16"]
    d = configs.make_rs_data(cfg)
    w = RsWorkload(cfg.world, cfg.rank, d["a"], d["b"], d["peers"], cfg.chunk_rows)

    def bookkeeping(what):
        e = B.agg_ctx_epoch(w.ctx)
        assert (w.flags.cpu().numpy() == e).all(), what
        assert (w.send_flags.cpu().numpy() == e).all(), what
        recv = w.recv.cpu()
        for p in range(cfg.world):
            if p != cfg.rank:
                assert torch.equal(recv[p], d["peers"][p]), (what, p)
    try:
        print("config c3: overlap", flush=True)
        w.run("overlap", order=cfg.order())
        assert w.status() == (0, -1)
        send, out = O.gemm_rs_ref(raw(d["a"]), raw(d["b"]), d["peers"].numpy(), cfg.world, cfg.rank)
        assert_close(to_f64(w.send), send, BF16_TOL, "send")
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
        bookkeeping("overlap")
        o1, s1 = w.out.clone(), w.send.clone()
        for producer, mode in (("cu", "serial"), ("sdma", "overlap"), ("kernel", "overlap")):
            print(f"config c3: {producer} {mode}", flush=True)
            B.agg_ctx_set_producer(w.ctx, producer)
            w.out.zero_()
            w.send.zero_()
            w.recv.zero_()
            w.run(mode, order=cfg.order())
            assert w.status() == (0, -1), (producer, mode)
            assert torch.equal(w.out, o1) and torch.equal(w.send, s1), (producer, mode)
            bookkeeping((producer, mode))
    finally:
        w.close()


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("mode", ["overlap", "serial", "gemm_only"])
def test_two_ranks_fused_local_block_vs_oracle(gpu, tile, mode):
    """W = 2: the local block's tiles are half the grid, so they add the peer's partial in their
    own epilogue (through LDS) instead of leaving it to the grid-wide reduction; ragged rows,
    columns and K tail within the bar, integer inputs bit-exact."""
    world, rank, m, k, n, cr = 2, 1, 2 * 328, 328, 264, 41
    a, b, peers = _data(world, m, k, n, seed=27)
    w = RsWorkload(world, rank, a, b, peers, cr, tile=tile)
    try:
        if mode == "gemm_only":
            w.run("copy_only", order=None)
        w.run(mode)
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(w.send[:world - 1]), send, BF16_TOL, "send")
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
    finally:
        w.close()
    a, b, peers = _data(world, m, k, n, seed=29, kind="int")
    w = RsWorkload(world, rank, a, b, peers, cr, tile=tile)
    try:
        w.run(mode if mode != "gemm_only" else "overlap")
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert np.array_equal(to_f64(w.send[:world - 1]), send)
        assert np.array_equal(to_f64(w.out), out)
    finally:
        w.close()
