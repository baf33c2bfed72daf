"""The five workloads: one rank's share of AllGather+GEMM / GEMM+ReduceScatter on one GPU.

Each entry states shapes, dtype, value distributions, chunk geometry, arrival order and seeds.
Readings of points the workload statements leave open (output dtype, "N(0, 0.02)" as a standard
deviation, seeds, delay magnitude, the ReduceScatter chunk size) are listed with the design notes.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import inputs


@dataclass(frozen=True)
class AgConfig:
    """AllGather+GEMM: C (W*Ms x N, bf16) = concat(shards) (W*Ms x K) @ B (K x N)."""
    name: str
    world: int
    rank: int
    m_shard: int
    k: int
    n: int
    dtype: str                  # "bf16" or "fp8" (OCP e4m3fn)
    chunk_rows: int
    a_dist: dict
    b_dist: dict
    order_kind: str             # "seeded" or "ring"
    seed: int
    with_delays: bool = False   # seeded per-chunk host delays in correctness runs
    op: str = field(default="ag")

    @property
    def m(self) -> int:
        return self.world * self.m_shard

    @property
    def chunks_per_shard(self) -> int:
        return self.m_shard // self.chunk_rows

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def order(self) -> list:
        if self.order_kind == "ring":
            return inputs.ring_order(self.world, self.rank, self.chunks_per_shard)
        return inputs.seeded_order(self.world, self.rank, self.chunks_per_shard, self.seed + 1)

    def delays(self) -> list | None:
        if not self.with_delays:
            return None
        n = (self.world - 1) * self.chunks_per_shard
        return inputs.delays_us(n, self.seed + 2, 50)


@dataclass(frozen=True)
class RsConfig:
    """GEMM+ReduceScatter: P = A (M x K) @ B (K x N) in fp32; this rank's block is reduced."""
    name: str
    world: int
    rank: int
    m: int
    k: int
    n: int
    chunk_rows: int
    a_dist: dict
    b_dist: dict
    peer_dist: dict
    order_kind: str
    seed: int
    dtype: str = "bf16"
    op: str = field(default="rs")

    @property
    def m_block(self) -> int:
        return self.m // self.world

    @property
    def chunks_per_block(self) -> int:
        return self.m_block // self.chunk_rows

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def order(self) -> list:
        if self.order_kind == "ring":
            return inputs.ring_order(self.world, self.rank, self.chunks_per_block)
        return inputs.seeded_order(self.world, self.rank, self.chunks_per_block, self.seed + 1)


@dataclass(frozen=True)
class ArConfig:
    """GEMM+AllReduce: P = A (M x K) @ B (K x N) in fp32, summed with W-1 peers' partials."""
    name: str
    world: int
    rank: int
    m: int
    k: int
    n: int
    chunk_rows: int
    a_dist: dict
    b_dist: dict
    peer_dist: dict
    order_kind: str
    seed: int
    dtype: str = "bf16"
    op: str = field(default="ar")

    @property
    def chunks_per_peer(self) -> int:
        return self.m // self.chunk_rows

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def order(self) -> list:
        if self.order_kind == "ring":
            return inputs.ring_order(self.world, self.rank, self.chunks_per_peer)
        return inputs.seeded_order(self.world, self.rank, self.chunks_per_peer, self.seed + 1)


@dataclass(frozen=True)
class FfnConfig:
    """FFN chain: h = silu(concat(shards) @ W1) (M x N1 bf16); y = h @ W2 (M x N2 fp32),
    reduce-scattered over W row blocks of Ms rows."""
    name: str
    world: int
    rank: int
    m_shard: int
    k1: int
    n1: int
    n2: int
    chunk_rows: int
    rs_chunk_rows: int
    a_dist: dict
    w1_dist: dict
    w2_dist: dict
    peer_dist: dict
    seed: int
    dtype: str = "bf16"
    op: str = field(default="ffn")

    @property
    def m(self) -> int:
        return self.world * self.m_shard

    @property
    def flops(self) -> int:
        return 2 * self.m * self.k1 * self.n1 + 2 * self.m * self.n1 * self.n2

    def order(self) -> list:
        return inputs.ring_order(self.world, self.rank, self.m_shard // self.chunk_rows)

    def rs_order(self) -> list:
        return inputs.seeded_order(self.world, self.rank, self.m_shard // self.rs_chunk_rows, self.seed + 1)


U11 = {"kind": "uniform", "lo": -1.0, "hi": 1.0}
N1 = {"kind": "normal", "std": 1.0}
N002 = {"kind": "normal", "std": 0.02}

@dataclass(frozen=True)
class A2aConfig:
    """AllToAll (dispatch) + GEMM: each of W source ranks holds `tokens` token rows (of K) and
    routes each to one rank (a seeded categorical draw with integer `weights`); this rank
    receives, from each source, the tokens routed to it (the first `cap`, the rest dropped) into
    slot p of a W*cap x K buffer, and multiplies every received row by B (K x N)."""
    name: str
    world: int
    rank: int
    tokens: int
    cap: int
    k: int
    n: int
    chunk_rows: int
    dtype: str
    a_dist: dict
    b_dist: dict
    weights: tuple
    order_kind: str
    seed: int
    op: str = field(default="a2a")

    @property
    def m(self) -> int:
        return self.world * self.cap

    @property
    def chunks_per_slot(self) -> int:
        return self.cap // self.chunk_rows

    def order(self) -> list:
        if self.order_kind == "ring":
            return inputs.ring_order(self.world, self.rank, self.chunks_per_slot)
        return inputs.seeded_order(self.world, self.rank, self.chunks_per_slot, self.seed + 1)

    def dests(self, p: int) -> list:
        """The rank each token of source p is routed to."""
        return inputs.routing(self.tokens, self.weights, self.seed + 100 + p)


CONFIGS = {
    # tiny, latency-bound; the oracle takes milliseconds
    "ag_w2_256x256x512_bf16": AgConfig(
        "ag_w2_256x256x512_bf16", world=2, rank=0, m_shard=128, k=512, n=256, dtype="bf16",
        chunk_rows=64, a_dist=U11, b_dist=U11, order_kind="seeded", seed=1010),
    # the MFMA-bound bf16 workload (the benchmark's)
    "ag_w8_4096x3584x8192_bf16": AgConfig(
        "ag_w8_4096x3584x8192_bf16", world=8, rank=0, m_shard=512, k=8192, n=3584, dtype="bf16",
        chunk_rows=128, a_dist=N1, b_dist=N002, order_kind="ring", seed=1020, with_delays=True),
    # GEMM + ReduceScatter, 7 incoming fp32 partial blocks
    "rs_w8_8192x8192x3584_bf16": RsConfig(
        "rs_w8_8192x8192x3584_bf16", world=8, rank=0, m=8192, k=3584, n=8192, chunk_rows=128,
        a_dist=N1, b_dist=N002, peer_dist=N1, order_kind="seeded", seed=1030),
    # decode-shaped, HBM-bound
    "ag_w8_128x3584x8192_bf16_decode": AgConfig(
        "ag_w8_128x3584x8192_bf16_decode", world=8, rank=0, m_shard=16, k=8192, n=3584,
        dtype="bf16", chunk_rows=16, a_dist=N1, b_dist=N002, order_kind="ring", seed=1040),
    # fp8 e4m3fn with per-tensor scales
    "ag_w8_8192x7168x8192_fp8": AgConfig(
        "ag_w8_8192x7168x8192_fp8", world=8, rank=0, m_shard=1024, k=8192, n=7168, dtype="fp8",
        chunk_rows=256, a_dist=N1, b_dist=N002, order_kind="seeded", seed=1050),
    # decode-shaped GEMM+AllReduce: the row-parallel layer after the decode AllGather+GEMM (its
    # 3584-wide per-rank activations times this rank's 3584 x 8192 weight rows), partials of the
    # whole 128 x 8192 output summed over 8 ranks
    "ar_w8_128x8192x3584_bf16_decode": ArConfig(
        "ar_w8_128x8192x3584_bf16_decode", world=8, rank=0, m=128, k=3584, n=8192, chunk_rows=16,
        a_dist=N1, b_dist=N002, peer_dist=N1, order_kind="seeded", seed=1060),
    # the two bf16 operations as one tensor-parallel FFN: the W=8 AllGather+GEMM above
    # (4096 x 8192 @ 8192 x 3584), SiLU, then GEMM+ReduceScatter with the ReduceScatter
    # workload's weight shape (3584 x 8192) on its 4096 rows
    "ffn_w8_4096x8192x3584_bf16": FfnConfig(
        "ffn_w8_4096x8192x3584_bf16", world=8, rank=0, m_shard=512, k1=8192, n1=3584, n2=8192,
        chunk_rows=128, rs_chunk_rows=128, a_dist=N1, w1_dist=N002, w2_dist=N002, peer_dist=N1,
        seed=1070),
    # AllToAll dispatch + the expert GEMM: 8 sources x 4096 tokens, top-1 routing with this
    # rank's expert drawn 10/66 of the time (~620 tokens per source against a capacity of 640,
    # so some sources fill their slot and drop the rest), hidden 8192, expert width 3584
    "a2a_w8_5120x3584x8192_bf16": A2aConfig(
        "a2a_w8_5120x3584x8192_bf16", world=8, rank=0, tokens=4096, cap=640, k=8192, n=3584,
        chunk_rows=128, dtype="bf16", a_dist=N1, b_dist=N002, weights=(10, 8, 8, 8, 8, 8, 8, 8),
        order_kind="seeded", seed=1080),
}

HEADLINE = "ag_w8_4096x3584x8192_bf16"


def make_ag_data(cfg: AgConfig):
    """Host tensors for an AllGather+GEMM workload.

    Returns dict: shards (list of W CPU tensors Ms x K, bf16 or float8_e4m3fn), b (K x N, same
    dtype), scale_a, scale_b (per-tensor fp8 scales; 1.0 for bf16). The W shards are drawn as one
    M x K tensor (seed) and split, so the gathered matrix has one per-tensor scale.
    """
    a, sa = inputs.draw(cfg.a_dist, (cfg.m, cfg.k), cfg.dtype, cfg.seed)
    b, sb = inputs.draw(cfg.b_dist, (cfg.k, cfg.n), cfg.dtype, cfg.seed + 3)
    shards = [a[p * cfg.m_shard:(p + 1) * cfg.m_shard].contiguous() for p in range(cfg.world)]
    return {"shards": shards, "b": b, "scale_a": sa, "scale_b": sb}


def make_rs_data(cfg: RsConfig):
    """Host tensors for a GEMM+ReduceScatter workload: a (M x K), b (K x N) bf16, and peers
    (W x M/W x N fp32) where slot ``rank`` is zero and unused."""
    a, _ = inputs.draw(cfg.a_dist, (cfg.m, cfg.k), cfg.dtype, cfg.seed)
    b, _ = inputs.draw(cfg.b_dist, (cfg.k, cfg.n), cfg.dtype, cfg.seed + 3)
    peers, _ = inputs.draw(cfg.peer_dist, (cfg.world, cfg.m_block, cfg.n), "f32", cfg.seed + 4)
    peers[cfg.rank].zero_()
    return {"a": a, "b": b, "peers": peers}


def make_ar_data(cfg: ArConfig):
    """Host tensors for a GEMM+AllReduce workload: a (M x K), b (K x N) bf16, and peers
    (W x M x N fp32) where slot ``rank`` is zero and unused."""
    a, _ = inputs.draw(cfg.a_dist, (cfg.m, cfg.k), cfg.dtype, cfg.seed)
    b, _ = inputs.draw(cfg.b_dist, (cfg.k, cfg.n), cfg.dtype, cfg.seed + 3)
    peers, _ = inputs.draw(cfg.peer_dist, (cfg.world, cfg.m, cfg.n), "f32", cfg.seed + 4)
    peers[cfg.rank].zero_()
    return {"a": a, "b": b, "peers": peers}


def make_ffn_data(cfg: FfnConfig):
    """Host tensors for the FFN chain: shards (W x Ms x K1 bf16), w1 (K1 x N1), w2 (N1 x N2) bf16,
    peers (W x Ms x N2 fp32, slot ``rank`` zero and unused)."""
    a, _ = inputs.draw(cfg.a_dist, (cfg.m, cfg.k1), cfg.dtype, cfg.seed)
    w1, _ = inputs.draw(cfg.w1_dist, (cfg.k1, cfg.n1), cfg.dtype, cfg.seed + 3)
    w2, _ = inputs.draw(cfg.w2_dist, (cfg.n1, cfg.n2), cfg.dtype, cfg.seed + 5)
    peers, _ = inputs.draw(cfg.peer_dist, (cfg.world, cfg.m_shard, cfg.n2), "f32", cfg.seed + 4)
    peers[cfg.rank].zero_()
    shards = [a[p * cfg.m_shard:(p + 1) * cfg.m_shard].contiguous() for p in range(cfg.world)]
    return {"shards": shards, "w1": w1, "w2": w2, "peers": peers}


def make_a2a_data(cfg: A2aConfig):
    """Host tensors for an AllToAll+GEMM workload.

    Returns dict: tokens (W CPU tensors T x K, each source's token rows), dests (W lists, each
    token's destination rank), blocks (W CPU tensors cap x K: what source p sends this rank, its
    tokens routed here in token order, the first cap of them, zero rows after), counts (rows in
    each block), b (K x N), scale_a, scale_b. All W sources' tokens are drawn as one tensor so
    that fp8 has one per-tensor scale.
    """
    a, sa = inputs.draw(cfg.a_dist, (cfg.world * cfg.tokens, cfg.k), cfg.dtype, cfg.seed)
    b, sb = inputs.draw(cfg.b_dist, (cfg.k, cfg.n), cfg.dtype, cfg.seed + 3)
    tokens = [a[p * cfg.tokens:(p + 1) * cfg.tokens].contiguous() for p in range(cfg.world)]
    dests = [cfg.dests(p) for p in range(cfg.world)]
    blocks, counts = [], []
    for p in range(cfg.world):
        d = torch.tensor(dests[p], dtype=torch.int64)
        idx = torch.nonzero(d == cfg.rank).flatten()[:cfg.cap]
        blk = torch.zeros(cfg.cap, cfg.k, dtype=torch.uint8 if cfg.dtype == "fp8" else torch.int16)
        blk = blk.view(tokens[p].dtype)
        blk[:len(idx)] = tokens[p][idx]
        blocks.append(blk)
        counts.append(int(len(idx)))
    return {"tokens": tokens, "dests": dests, "blocks": blocks, "counts": counts, "b": b,
            "scale_a": sa, "scale_b": sb}

