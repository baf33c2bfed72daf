"""GEMM+AllReduce (one-shot, reduction fused into each tile's epilogue) on the GPU through the C
ABI, compared with the CPU oracle.

Bar: |x - ref| <= 1e-2 + 1e-2 |ref| for `send` (this rank's partial) and `out` (partial plus the
peers' partials); bit-exact for the receive buffer, the flags, and for integer-valued inputs
(every fp32 sum exact); `out` bit-identical for every arrival order and mode (fixed summation
order).
"""

import numpy as np
import pytest
import torch

from allgather_gemm_persistent_amd import binding as B
from allgather_gemm_persistent_amd import configs, inputs
from allgather_gemm_persistent_amd.workload import ArWorkload
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
        peers, _ = inputs.draw({"kind": "int", "lo": -100, "hi": 100}, (world, m, n), "f32", seed + 2)
    else:
        a, _ = inputs.draw({"kind": "normal", "std": 1.0}, (m, k), "bf16", seed)
        b, _ = inputs.draw({"kind": "normal", "std": 0.05}, (k, n), "bf16", seed + 1)
        peers, _ = inputs.draw({"kind": "normal", "std": 1.0}, (world, m, n), "f32", seed + 2)
    return a, b, peers


def _ref(w, a, b, peers):
    return O.gemm_ar_ref(raw(a), raw(b), peers.numpy(), w.world, w.rank)


def _bookkeeping(w, peers, what):
    e = B.agg_ctx_epoch(w.ctx)
    assert (w.flags.cpu().numpy() == e).all(), what
    assert (w.send_flags.cpu().numpy() == e).all(), what
    recv = w.recv.cpu()
    for p in range(w.world):
        if p != w.rank:
            assert torch.equal(recv[p], peers[p]), (what, p)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("mode", ["overlap", "serial"])
@pytest.mark.parametrize("producer", PRODUCERS)
def test_ragged_vs_oracle(gpu, tile, mode, producer):
    """Sizes that are not multiples of any tile: ragged rows, columns and K tail."""
    world, rank, m, k, n, cr = 3, 1, 200, 328, 264, 40
    a, b, peers = _data(world, m, k, n, seed=307)
    w = ArWorkload(world, rank, a, b, peers, cr, tile=tile, producer=producer)
    try:
        w.run(mode, order=inputs.seeded_order(world, rank, m // cr, 5))
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(w.send), send, BF16_TOL, "send")
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
        _bookkeeping(w, peers, (tile, mode, producer))
    finally:
        w.close()


@pytest.mark.parametrize("tile", [(128, 128), (64, 64)])
def test_integer_inputs_bitexact(gpu, tile):
    world, rank, m, k, n, cr = 4, 2, 96, 512, 192, 32
    a, b, peers = _data(world, m, k, n, seed=317, kind="int")
    w = ArWorkload(world, rank, a, b, peers, cr, tile=tile)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert np.array_equal(to_f64(w.send), send)
        assert np.array_equal(to_f64(w.out), out)
    finally:
        w.close()


@pytest.mark.parametrize("producer", PRODUCERS)
def test_order_and_mode_invariance(gpu, producer):
    world, rank, m, k, n, cr = 8, 5, 128, 256, 512, 16
    a, b, peers = _data(world, m, k, n, seed=327)
    w = ArWorkload(world, rank, a, b, peers, cr, tile=(64, 64), producer=producer)
    try:
        outs = []
        for s in (None, 1, 2):
            order = None if s is None else inputs.seeded_order(world, rank, m // cr, s)
            for mode in ("overlap", "serial", "gemm_only"):
                w.out.zero_()
                if mode != "gemm_only":
                    w.recv.zero_()
                w.run(mode, order=order)
                assert w.status() == (0, -1), (s, mode)
                outs.append((w.out.clone(), w.send.clone()))
                _bookkeeping(w, peers, (s, mode))
        for o, sd in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(sd, outs[0][1])
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(outs[0][0]), out, BF16_TOL, "out")
    finally:
        w.close()


def test_world_one_and_k_zero(gpu):
    a, b, peers = _data(1, 96, 64, 32, seed=337)
    w = ArWorkload(1, 0, a, b, peers, 32)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        send, out = _ref(w, a, b, peers)
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
    finally:
        w.close()
    a = torch.zeros(32, 0, dtype=torch.bfloat16)
    b = torch.zeros(0, 32, dtype=torch.bfloat16)
    peers = inputs.draw({"kind": "normal", "std": 1.0}, (2, 32, 32), "f32", 3)[0]
    w = ArWorkload(2, 1, a, b, peers, 16)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        assert torch.equal(w.out.cpu(), peers[0]) and (w.send.cpu() == 0).all()
    finally:
        w.close()


def test_config_decode_vs_oracle(gpu):
    """The W=8 128 x 8192 x 3584 decode GEMM+AllReduce at full size, overlapped, against the
    oracle; then serialized, bare and with the copy-engine producer (receive buffer cleared
    first): the same bits in `send` and `out`, every peer's partial in the receive buffer, all
    flags at the epoch."""
    cfg = configs.CONFIGS["ar_w8_128x8192x3584_bf16_decode"]
    d = configs.make_ar_data(cfg)
    w = ArWorkload(cfg.world, cfg.rank, d["a"], d["b"], d["peers"], cfg.chunk_rows)
    try:
        print("config ar decode: overlap", flush=True)
        w.run("overlap", order=cfg.order())
        assert w.status() == (0, -1)
        send, out = O.gemm_ar_ref(raw(d["a"]), raw(d["b"]), d["peers"].numpy(), cfg.world, cfg.rank)
        assert_close(to_f64(w.send), send, BF16_TOL, "send")
        assert_close(to_f64(w.out), out, BF16_TOL, "out")
        _bookkeeping(w, d["peers"], "overlap")
        o1, s1 = w.out.clone(), w.send.clone()
        for producer, mode in (("cu", "serial"), ("cu", "gemm_only"), ("sdma", "overlap"), ("kernel", "overlap")):
            print(f"config ar decode: {producer} {mode}", flush=True)
            B.agg_ctx_set_producer(w.ctx, producer)
            w.out.zero_()
            w.send.zero_()
            if mode != "gemm_only":
                w.recv.zero_()
            w.run(mode, order=cfg.order())
            assert w.status() == (0, -1), (producer, mode)
            assert torch.equal(w.out, o1) and torch.equal(w.send, s1), (producer, mode)
            _bookkeeping(w, d["peers"], (producer, mode))
    finally:
        w.close()
