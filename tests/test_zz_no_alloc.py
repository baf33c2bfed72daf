"""ag_gemm_noalloc (the variant for callers that cannot allocate) against ag_gemm through the C
ABI: the same kernels on the device's static scratch instead of the ctx's, so C, the gather
buffer and the flags must be bit-identical to ag_gemm's on the same inputs. Two calls in a row,
the second with a smaller input, on a shape that uses split-K partials (the static array's
partial room) and on one that does not; a call whose partials exceed the room is refused."""

import numpy as np
import pytest
import torch

from allgather_gemm_persistent_amd import binding as B
from allgather_gemm_persistent_amd import inputs
from allgather_gemm_persistent_amd.workload import AgWorkload
from oracle import agg_oracle as O

from helpers import BF16_TOL, assert_close, bits_equal, raw, small_ag_data, to_f64

pytestmark = pytest.mark.gpu


def _call(w, fn, order):
    fn(w.ctx, w.world, w.rank, w.m_shard, w.n, w.k, w.chunk_rows, w.dtype, w.scale_a, w.scale_b,
       w.peer_ptrs(), w.gather, w.flags, w.b, w.c, order=order, mode="overlap",
       stream=torch.cuda.current_stream())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_ag_gemm_twice_shrinking(gpu, dtype):
    # (world, m_shard, k, n, chunk_rows): the W=8 decode shape (4 split-K parts, 7.3 MB of
    # partials in the static array), then a smaller one without split-K
    shapes = [(8, 16, 8192, 3584, 16), (3, 64, 512, 208, 32)]
    for i, (world, ms, k, n, cr) in enumerate(shapes):
        shards, b, sa, sb = small_ag_data(world, ms, k, n, dtype, seed=200 + i)
        w = AgWorkload(world, 1, shards, b, chunk_rows=cr, dtype=dtype, scale_a=sa, scale_b=sb)
        try:
            B.agg_ctx_set_pull(w.ctx, "off")
            order = inputs.seeded_order(world, 1, ms // cr, 3 + i)
            _call(w, B.ag_gemm, order)
            assert w.status() == (0, -1)
            ref_c, ref_flags = w.c.clone(), w.flags.clone()
            w.c.zero_()
            w.gather[[r for r in range(world * ms) if r // ms != 1]] = 0
            _call(w, B.ag_gemm_noalloc, order)
            assert w.status() == (0, -1), (i, dtype)
            assert bits_equal(w.c, ref_c), (i, dtype)
            assert (w.flags.cpu() == B.agg_ctx_epoch(w.ctx)).all() and not torch.equal(w.flags, ref_flags)
            assert np.array_equal(raw(w.gather), O.gather_ref([raw(s) for s in shards]))
            tol = BF16_TOL if dtype == "bf16" else (2e-2, 2e-2)
            assert_close(to_f64(w.c), O.ag_gemm_ref([raw(s) for s in shards], raw(b), dtype, sa, sb),
                         tol, f"C {i}")
        finally:
            w.close()


def test_noalloc_refuses_partials_beyond_its_scratch(gpu):
    world, ms, k, n, cr = 2, 128, 4096, 4096, 64
    shards, b, _, _ = small_ag_data(world, ms, k, n, "bf16", seed=211)
    w = AgWorkload(world, 0, shards, b, chunk_rows=cr, tile=(128, 128))
    try:
        B.agg_ctx_set_split(w.ctx, 16)       # 16 x 256 x 4096 x 4 B = 64 MiB of partials
        with pytest.raises(B.AggError) as e:
            _call(w, B.ag_gemm_noalloc, None)
        assert e.value.code == B.AGG_E_UNSUPPORTED
        B.agg_ctx_set_producer(w.ctx, "sdma")
        B.agg_ctx_set_split(w.ctx, 0)
        with pytest.raises(B.AggError) as e:
            _call(w, B.ag_gemm_noalloc, None)
        assert e.value.code == B.AGG_E_STATE
    finally:
        w.close()
