"""The FFN chain (AllGather+GEMM -> SiLU -> GEMM+ReduceScatter in one persistent kernel) on the
GPU through the C ABI, compared with the CPU oracle.

Bar: h (bf16, SiLU of the first product) and `send` / `out` (fp32, computed from that bf16 h)
within 1e-2 + 1e-2 |ref| of the oracle's, which rounds h to bf16 as well (the second layer's operand
type). The two sides round different values (fp32 accumulations against exact products), so an
element of h may land one bf16 step apart where the exact value sits next to a rounding midpoint
(about one element in a few thousand); each such step moves a 3584-term sum by one product,
~1e-4 here, far inside the bar.
Bit-exact: gather and receive buffers, every flag at the epoch, the special case W1 = 0 (h = 0,
send = 0, out = the peers' sum, exact in fp32 for integer peers), and identical bits across
arrival orders, modes, producers and fused / unfused launches.
"""

import numpy as np
import pytest
import torch

from allgather_gemm_persistent_amd import binding as B
from allgather_gemm_persistent_amd import configs, inputs
from allgather_gemm_persistent_amd.workload import FfnWorkload
from oracle import agg_oracle as O

from helpers import BF16_TOL, assert_close, raw, to_f64

pytestmark = pytest.mark.gpu


def _data(world, ms, k1, n1, n2, seed, zero_w1=False):
    a, _ = inputs.draw({"kind": "normal", "std": 1.0}, (world * ms, k1), "bf16", seed)
    w1, _ = inputs.draw({"kind": "normal", "std": 0.05}, (k1, n1), "bf16", seed + 1)
    if zero_w1:
        w1 = torch.zeros_like(w1)
        peers, _ = inputs.draw({"kind": "int", "lo": -100, "hi": 100}, (world, ms, n2), "f32", seed + 3)
    else:
        peers, _ = inputs.draw({"kind": "normal", "std": 1.0}, (world, ms, n2), "f32", seed + 3)
    w2, _ = inputs.draw({"kind": "normal", "std": 0.05}, (n1, n2), "bf16", seed + 2)
    shards = [a[p * ms:(p + 1) * ms].contiguous() for p in range(world)]
    return shards, w1, w2, peers


def _ref(w, shards, w1, w2, peers):
    return O.ffn_chain_ref([raw(s) for s in shards], raw(w1), raw(w2), peers.numpy(), w.world, w.rank)


def _bookkeeping(w, shards, peers, what):
    e = B.agg_ctx_epoch(w.ctx)
    for name in ("flags", "rs_flags", "send_flags"):
        assert (getattr(w, name).cpu().numpy() == e).all(), (what, name)
    assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards])), what
    recv = w.recv.cpu()
    for p in range(w.world):
        if p != w.rank:
            assert torch.equal(recv[p], peers[p]), (what, p)


def _compare(w, ref, what):
    h, send, out = ref
    assert_close(to_f64(w.h), h, BF16_TOL, f"h {what}")
    assert_close(to_f64(w.send[:w.world - 1]), send, BF16_TOL, f"send {what}")
    assert_close(to_f64(w.out), out, BF16_TOL, f"out {what}")


@pytest.mark.parametrize("mode", ["overlap", "serial"])
@pytest.mark.parametrize("producer", ["cu", "sdma", "kernel"])
@pytest.mark.parametrize("fused", [True, False])
def test_ragged_vs_oracle(gpu, mode, producer, fused):
    """Shard rows, both layers' columns and K not multiples of the 256 x 256 tile."""
    world, rank, ms, k1, n1, n2 = 3, 1, 200, 328, 264, 200
    shards, w1, w2, peers = _data(world, ms, k1, n1, n2, seed=401)
    w = FfnWorkload(world, rank, shards, w1, w2, peers, chunk_rows=40, rs_chunk_rows=50, producer=producer)
    try:
        B.agg_ctx_set_chain_fused(w.ctx, fused)
        w.run(mode, order=inputs.seeded_order(world, rank, ms // 40, 3),
              rs_order=inputs.seeded_order(world, rank, ms // 50, 4))
        assert w.status() == (0, -1)
        _compare(w, _ref(w, shards, w1, w2, peers), (mode, producer, fused))
        _bookkeeping(w, shards, peers, (mode, producer, fused))
    finally:
        w.close()


def test_zero_first_layer_bitexact(gpu):
    """W1 = 0: h = silu(0) = 0 exactly, so send = 0 and out = the sum of the integer peers, exact."""
    world, rank, ms, k1, n1, n2 = 4, 2, 256, 256, 512, 264
    shards, w1, w2, peers = _data(world, ms, k1, n1, n2, seed=411, zero_w1=True)
    w = FfnWorkload(world, rank, shards, w1, w2, peers, chunk_rows=64, rs_chunk_rows=128)
    try:
        w.run("overlap")
        assert w.status() == (0, -1)
        assert (w.h.float().cpu() == 0).all()
        assert (w.send.cpu() == 0).all()
        want = sum(peers[q].double() for q in range(world) if q != rank).numpy()
        assert np.array_equal(to_f64(w.out), want)
    finally:
        w.close()


@pytest.mark.parametrize("producer", ["cu", "sdma", "kernel"])
def test_orders_modes_fusion_bit_identical(gpu, producer):
    world, rank, ms, k1, n1, n2 = 8, 3, 128, 512, 512, 512
    shards, w1, w2, peers = _data(world, ms, k1, n1, n2, seed=421)
    w = FfnWorkload(world, rank, shards, w1, w2, peers, chunk_rows=32, rs_chunk_rows=64, producer=producer)
    try:
        outs = []
        for s in (None, 1, 2):
            order = None if s is None else inputs.seeded_order(world, rank, ms // 32, s)
            rs_order = None if s is None else inputs.seeded_order(world, rank, ms // 64, s + 10)
            for fused in (True, False):
                B.agg_ctx_set_chain_fused(w.ctx, fused)
                for mode in ("overlap", "serial", "gemm_only"):
                    w.out.zero_()
                    w.h.zero_()
                    w.run(mode, order=order, rs_order=rs_order)
                    assert w.status() == (0, -1), (s, fused, mode)
                    outs.append((w.h.clone(), w.send.clone(), w.out.clone()))
                    _bookkeeping(w, shards, peers, (s, fused, mode))
        for h, sd, o in outs[1:]:
            assert torch.equal(h.view(torch.int16), outs[0][0].view(torch.int16))
            assert torch.equal(sd, outs[0][1]) and torch.equal(o, outs[0][2])
        _compare(w, _ref(w, shards, w1, w2, peers), "orders")
    finally:
        w.close()


def test_config_vs_oracle(gpu):
    """The W=8 FFN chain at full size (4096 x 8192 @ 8192 x 3584, SiLU, @ 3584 x 8192, reduce-
    scattered over 8 blocks of 512 rows), fused and overlapped, against the oracle; then unfused,
    serialized and with the copy-engine producer (buffers cleared first): the same bits."""
    cfg = configs.CONFIGS["ffn_w8_4096x8192x3584_bf16"]
    d = configs.make_ffn_data(cfg)
    w = FfnWorkload(cfg.world, cfg.rank, d["shards"], d["w1"], d["w2"], d["peers"], cfg.chunk_rows,
                    cfg.rs_chunk_rows)
    rows = [r for r in range(cfg.m) if r // cfg.m_shard != cfg.rank]
    try:
        print("config ffn: fused overlap", flush=True)
        w.run("overlap", order=cfg.order(), rs_order=cfg.rs_order())
        assert w.status() == (0, -1)
        ref = O.ffn_chain_ref([raw(s) for s in d["shards"]], raw(d["w1"]), raw(d["w2"]),
                              d["peers"].numpy(), cfg.world, cfg.rank)
        _compare(w, ref, "fused overlap")
        _bookkeeping(w, d["shards"], d["peers"], "fused overlap")
        h1, s1, o1 = w.h.clone(), w.send.clone(), w.out.clone()
        for producer, fused, mode in (("cu", False, "overlap"), ("cu", True, "serial"), ("sdma", True, "overlap")):
            print(f"config ffn: {producer} fused={fused} {mode}", flush=True)
            B.agg_ctx_set_producer(w.ctx, producer)
            B.agg_ctx_set_chain_fused(w.ctx, fused)
            for t in (w.h, w.send, w.out, w.recv):
                t.zero_()
            w.gather[rows] = 0
            w.run(mode, order=cfg.order(), rs_order=cfg.rs_order())
            assert w.status() == (0, -1), (producer, fused, mode)
            assert torch.equal(w.h.view(torch.int16), h1.view(torch.int16)), (producer, fused, mode)
            assert torch.equal(w.send, s1) and torch.equal(w.out, o1), (producer, fused, mode)
            _bookkeeping(w, d["shards"], d["peers"], (producer, fused, mode))
    finally:
        w.close()
