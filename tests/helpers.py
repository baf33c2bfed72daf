"""Shared helpers of the GPU tests: comparisons against the oracle and input preparation."""

import numpy as np
import torch

from allgather_gemm_persistent_amd import inputs

BF16_TOL = (1e-2, 1e-2)   # |got - ref| <= atol + rtol * |ref|
FP8_TOL = (2e-2, 2e-2)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device or host tensor (bf16 / fp32 widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(got: np.ndarray, ref: np.ndarray, tol, what=""):
    atol, rtol = tol
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), got.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {got.size} elements out of tolerance; worst at {idx}: "
            f"got {got[idx]!r} ref {ref[idx]!r}; max abs err {float(err.max()):.3g}")


def raw(t: torch.Tensor) -> np.ndarray:
    return inputs.raw_bits(t.detach().to("cpu"))


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.detach().to("cpu").contiguous().view(torch.uint8)
    b = b.detach().to("cpu").contiguous().view(torch.uint8)
    return a.shape == b.shape and torch.equal(a, b)


def small_ag_data(world, m_shard, k, n, dtype, seed, kind="normal"):
    """Random (or small-integer) shards and weight for a test-sized AllGather+GEMM."""
    if kind == "int":
        dist_a = dist_b = {"kind": "int", "lo": -2, "hi": 2}
    else:
        dist_a, dist_b = {"kind": "normal", "std": 1.0}, {"kind": "normal", "std": 0.05}
    a, sa = inputs.draw(dist_a, (world * m_shard, k), dtype, seed)
    b, sb = inputs.draw(dist_b, (k, n), dtype, seed + 7)
    shards = [a[p * m_shard:(p + 1) * m_shard].contiguous() for p in range(world)]
    return shards, b, sa, sb
