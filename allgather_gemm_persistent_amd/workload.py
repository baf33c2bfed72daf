"""Device buffers for one workload (AllGather, AllToAll, ReduceScatter, AllReduce, the FFN
chain) and calls through the binding. PyTorch provides device memory and streams only; every
step runs in libagg.

The emulated peers are ordinary device allocations holding each remote rank's shard (or, for
ReduceScatter, the partial block it contributes); the symmetric buffers (gather / receive) and
the flag words are what a multi-GPU build would place in peer-visible memory.
"""

from __future__ import annotations

import torch

from . import binding as B


class AgWorkload:
    """One rank's share of AllGather+GEMM with W-1 emulated peers on one GPU.

    shards: W CPU tensors (Ms x K, bf16 or float8_e4m3fn); b_kn: CPU tensor (K x N), the weight,
    passed to the library as it is (N contiguous).
    """

    def __init__(self, world, rank, shards, b_kn, chunk_rows, dtype="bf16", scale_a=1.0,
                 scale_b=1.0, device="cuda", tile=None, producer="cu"):
        self.world, self.rank, self.chunk_rows, self.dtype = world, rank, chunk_rows, dtype
        self.m_shard, self.k = shards[0].shape
        self.n = b_kn.shape[1]
        self.m = world * self.m_shard
        self.scale_a, self.scale_b = float(scale_a), float(scale_b)
        self.device = torch.device(device)
        tdt = shards[0].dtype
        self.peers = [s.to(self.device) if p != rank else None for p, s in enumerate(shards)]
        self.local = shards[rank].to(self.device)
        # zero-filled as bytes (every torch dtype, fp8 included, has a byte view)
        esize = shards[0].element_size()
        self.gather = torch.zeros(self.m, max(self.k, 1) * esize, dtype=torch.uint8,
                                  device=self.device).view(tdt)[:, :self.k]
        self.reset_local()
        cps = self.m_shard // chunk_rows if chunk_rows else 0
        self.flags = torch.zeros(max(world * cps, 1), dtype=torch.int32, device=self.device)
        self.b = self.device_weight(b_kn)
        self.c = torch.zeros(self.m, self.n, dtype=torch.bfloat16, device=self.device)
        self.copy_stream = None     # the ctx runs the copies on its own streams
        self.ctx = B.agg_ctx_create(self.device.index or 0)
        B.agg_ctx_set_producer(self.ctx, producer)
        if tile:
            B.agg_ctx_set_tile(self.ctx, *tile)

    def device_weight(self, b_kn):
        """The weight as the library takes it, on the device."""
        return b_kn.contiguous().to(self.device)

    def reset_local(self):
        """Place the local shard in its slot of the gather buffer (the caller's job)."""
        ms = self.m_shard
        self.gather[self.rank * ms:(self.rank + 1) * ms].copy_(self.local)

    def peer_ptrs(self):
        return [p if p is not None else 0 for p in self.peers]

    def run(self, mode="overlap", order=None, delay_us=None, stream=None):
        stream = stream or torch.cuda.current_stream(self.device)
        B.ag_gemm(self.ctx, self.world, self.rank, self.m_shard, self.n, self.k, self.chunk_rows,
                  self.dtype, self.scale_a, self.scale_b, self.peer_ptrs(), self.gather,
                  self.flags, self.b, self.c, order=order, delay_us=delay_us, mode=mode,
                  stream=stream, copy_stream=self.copy_stream)

    def status(self):
        return B.agg_ctx_status(self.ctx, torch.cuda.current_stream(self.device))

    def close(self):
        if self.ctx is not None:
            B.agg_ctx_destroy(self.ctx)
            self.ctx = None


class A2aWorkload(AgWorkload):
    """One rank's share of AllToAll (dispatch) + GEMM with W-1 emulated sources on one GPU.

    blocks: W CPU tensors (cap x K, bf16 or float8_e4m3fn), what each source sends this rank (its
    first counts[p] rows hold tokens); counts: W ints; b_kn: CPU tensor (K x N). The receive
    buffer is the gather buffer of the base class, slot p of `cap` rows per source.
    """

    def __init__(self, world, rank, blocks, counts, b_kn, chunk_rows, dtype="bf16", scale_a=1.0,
                 scale_b=1.0, device="cuda", tile=None, producer="cu"):
        self.counts = [int(x) for x in counts]
        super().__init__(world, rank, blocks, b_kn, chunk_rows, dtype, scale_a, scale_b, device,
                         tile, producer)
        self.cap = self.m_shard

    def reset_local(self):
        """Place the rank's own routed rows in its slot of the receive buffer."""
        ms, cnt = self.m_shard, self.counts[self.rank]
        self.gather[self.rank * ms:self.rank * ms + cnt].copy_(self.local[:cnt])

    def run(self, mode="overlap", order=None, delay_us=None, stream=None):
        stream = stream or torch.cuda.current_stream(self.device)
        B.a2a_gemm(self.ctx, self.world, self.rank, self.m_shard, self.n, self.k, self.chunk_rows,
                   self.dtype, self.scale_a, self.scale_b, self.counts, self.peer_ptrs(), self.gather,
                   self.flags, self.b, self.c, order=order, delay_us=delay_us, mode=mode,
                   stream=stream, copy_stream=self.copy_stream)

    def held_rows(self):
        """Row indices of the receive buffer (and of C) that hold tokens."""
        return [p * self.m_shard + i for p in range(self.world) for i in range(self.counts[p])]


class RsWorkload:
    """One rank's share of GEMM+ReduceScatter with W-1 emulated peers on one GPU.

    a: CPU (M x K) bf16; b_kn: CPU (K x N) bf16; peers: CPU (W x M/W x N) float32 (slot rank
    unused).
    """

    def __init__(self, world, rank, a, b_kn, peers, chunk_rows, device="cuda", tile=None,
                 producer="cu"):
        self.world, self.rank, self.chunk_rows = world, rank, chunk_rows
        self.m, self.k = a.shape
        self.n = b_kn.shape[1]
        self.mb = self.m // world
        self.device = torch.device(device)
        self.a = a.to(self.device)
        self.b = b_kn.contiguous().to(self.device)
        self.peers = [peers[p].to(self.device) if p != rank else None for p in range(world)]
        self.recv = torch.zeros(world, self.mb, self.n, dtype=torch.float32, device=self.device)
        cpb = self.mb // chunk_rows if chunk_rows else 0
        self.flags = torch.zeros(max(world * cpb, 1), dtype=torch.int32, device=self.device)
        self.send_flags = torch.zeros(max(world * cpb, 1), dtype=torch.int32, device=self.device)
        self.send = torch.zeros(max(world - 1, 1), self.mb, self.n, dtype=torch.float32,
                                device=self.device)
        self.out = torch.zeros(self.mb, self.n, dtype=torch.float32, device=self.device)
        self.copy_stream = None     # the ctx runs the copies on its own streams
        self.ctx = B.agg_ctx_create(self.device.index or 0)
        B.agg_ctx_set_producer(self.ctx, producer)
        if tile:
            B.agg_ctx_set_tile(self.ctx, *tile)

    def peer_ptrs(self):
        return [p if p is not None else 0 for p in self.peers]

    def run(self, mode="overlap", order=None, delay_us=None, stream=None):
        stream = stream or torch.cuda.current_stream(self.device)
        B.gemm_rs(self.ctx, self.world, self.rank, self.m, self.n, self.k, self.chunk_rows,
                  self.a, self.b, self.send, self.send_flags, self.peer_ptrs(), self.recv,
                  self.flags, self.out, order=order, delay_us=delay_us, mode=mode, stream=stream,
                  copy_stream=self.copy_stream)

    def status(self):
        return B.agg_ctx_status(self.ctx, torch.cuda.current_stream(self.device))

    def close(self):
        if self.ctx is not None:
            B.agg_ctx_destroy(self.ctx)
            self.ctx = None


class ArWorkload:
    """One rank's share of GEMM+AllReduce with W-1 emulated peers on one GPU.

    a: CPU (M x K) bf16; b_kn: CPU (K x N) bf16; peers: CPU (W x M x N) float32 (slot rank
    unused): the partial each peer sends.
    """

    def __init__(self, world, rank, a, b_kn, peers, chunk_rows, device="cuda", tile=None,
                 producer="cu"):
        self.world, self.rank, self.chunk_rows = world, rank, chunk_rows
        self.m, self.k = a.shape
        self.n = b_kn.shape[1]
        self.device = torch.device(device)
        self.a = a.to(self.device)
        self.b = b_kn.contiguous().to(self.device)
        self.peers = [peers[p].to(self.device) if p != rank else None for p in range(world)]
        self.recv = torch.zeros(world, self.m, self.n, dtype=torch.float32, device=self.device)
        cpb = self.m // chunk_rows if chunk_rows else 0
        self.flags = torch.zeros(max(world * cpb, 1), dtype=torch.int32, device=self.device)
        self.send_flags = torch.zeros(max(cpb, 1), dtype=torch.int32, device=self.device)
        self.send = torch.zeros(self.m, self.n, dtype=torch.float32, device=self.device)
        self.out = torch.zeros(self.m, self.n, dtype=torch.float32, device=self.device)
        self.copy_stream = None
        self.ctx = B.agg_ctx_create(self.device.index or 0)
        B.agg_ctx_set_producer(self.ctx, producer)
        if tile:
            B.agg_ctx_set_tile(self.ctx, *tile)

    def peer_ptrs(self):
        return [p if p is not None else 0 for p in self.peers]

    def run(self, mode="overlap", order=None, delay_us=None, stream=None):
        stream = stream or torch.cuda.current_stream(self.device)
        B.gemm_ar(self.ctx, self.world, self.rank, self.m, self.n, self.k, self.chunk_rows,
                  self.a, self.b, self.send, self.send_flags, self.peer_ptrs(), self.recv,
                  self.flags, self.out, order=order, delay_us=delay_us, mode=mode, stream=stream,
                  copy_stream=self.copy_stream)

    def status(self):
        return B.agg_ctx_status(self.ctx, torch.cuda.current_stream(self.device))

    def close(self):
        if self.ctx is not None:
            B.agg_ctx_destroy(self.ctx)
            self.ctx = None


class FfnWorkload:
    """One rank's share of the FFN chain (AllGather+GEMM, SiLU, GEMM+ReduceScatter) with W-1
    emulated peers on one GPU.

    shards: W CPU tensors (Ms x K1 bf16); w1: CPU (K1 x N1) bf16; w2: CPU (N1 x N2) bf16; peers:
    CPU (W x Ms x N2) float32 (slot rank unused): what each peer contributes to this rank's block.
    """

    def __init__(self, world, rank, shards, w1, w2, peers, chunk_rows, rs_chunk_rows,
                 device="cuda", producer="cu"):
        self.world, self.rank = world, rank
        self.chunk_rows, self.rs_chunk_rows = chunk_rows, rs_chunk_rows
        self.m_shard, self.k1 = shards[0].shape
        self.n1, self.n2 = w1.shape[1], w2.shape[1]
        self.m = world * self.m_shard
        self.device = torch.device(device)
        dev = self.device
        self.peers = [s.to(dev) if p != rank else None for p, s in enumerate(shards)]
        self.local = shards[rank].to(dev)
        self.gather = torch.zeros(self.m, self.k1, dtype=torch.bfloat16, device=dev)
        self.reset_local()
        cps = self.m_shard // chunk_rows
        cpb = self.m_shard // rs_chunk_rows
        self.flags = torch.zeros(max(world * cps, 1), dtype=torch.int32, device=dev)
        self.w1 = w1.contiguous().to(dev)
        self.w2 = w2.contiguous().to(dev)
        self.h = torch.zeros(self.m, self.n1, dtype=torch.bfloat16, device=dev)
        self.rs_peers = [peers[p].to(dev) if p != rank else None for p in range(world)]
        self.recv = torch.zeros(world, self.m_shard, self.n2, dtype=torch.float32, device=dev)
        self.rs_flags = torch.zeros(max(world * cpb, 1), dtype=torch.int32, device=dev)
        self.send_flags = torch.zeros(max(world * cpb, 1), dtype=torch.int32, device=dev)
        self.send = torch.zeros(max(world - 1, 1), self.m_shard, self.n2, dtype=torch.float32, device=dev)
        self.out = torch.zeros(self.m_shard, self.n2, dtype=torch.float32, device=dev)
        self.copy_stream = None
        self.ctx = B.agg_ctx_create(dev.index or 0)
        B.agg_ctx_set_producer(self.ctx, producer)

    def reset_local(self):
        ms = self.m_shard
        self.gather[self.rank * ms:(self.rank + 1) * ms].copy_(self.local)

    def run(self, mode="overlap", order=None, rs_order=None, stream=None):
        stream = stream or torch.cuda.current_stream(self.device)
        peers = [p if p is not None else 0 for p in self.peers]
        rs_peers = [p if p is not None else 0 for p in self.rs_peers]
        B.ffn_chain(self.ctx, self.world, self.rank, self.m_shard, self.k1, self.n1, self.n2,
                    self.chunk_rows, self.rs_chunk_rows, peers, self.gather, self.flags, self.w1,
                    self.h, self.w2, self.send, self.send_flags, rs_peers, self.recv,
                    self.rs_flags, self.out, order=order, rs_order=rs_order, mode=mode,
                    stream=stream, copy_stream=self.copy_stream)

    def status(self):
        return B.agg_ctx_status(self.ctx, torch.cuda.current_stream(self.device))

    def close(self):
        if self.ctx is not None:
            B.agg_ctx_destroy(self.ctx)
            self.ctx = None
