"""Seeded synthetic inputs for the workloads (gathers, reductions, token routings).

This module holds no arithmetic of the method itself (no product, no reduction, no schedule):
it only draws input tensors, arrival orders and delays from seeds, so that the HIP library and
the CPU oracle can be fed the very same bytes. It imports nothing else from the package.

* Tensor values come from a CPU ``torch.Generator`` (normal or uniform in float32), rounded to
  bfloat16 by torch, or quantised to float8 e4m3fn with one per-tensor scale
  ``s = amax|x| / 448`` and ``q = clamp(x / s, -448, 448)`` rounded by torch's cast.
* Permutations, delays and token routings come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; the constants of Vigna's public-domain
  reference version), which is stable across library versions; a Fisher-Yates shuffle draws
  ``next() % (i + 1)`` for i = n-1 down to 1.
"""

from __future__ import annotations

import numpy as np
import torch

MASK64 = (1 << 64) - 1
FP8_MAX = 448.0


class SplitMix64:
    """SplitMix64 generator: state += golden gamma; output = mix(state)."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def routing(n_tokens: int, weights, seed: int) -> list:
    """The rank each of ``n_tokens`` tokens is routed to: a categorical draw over the ranks with
    integer ``weights``, token by token from SplitMix64(seed): r = next() % sum(weights), and the
    token goes to the first rank whose cumulative weight exceeds r."""
    w = [int(x) for x in weights]
    if not w or min(w) < 0 or sum(w) == 0:
        raise ValueError("weights must be non-negative integers with a positive sum")
    total = sum(w)
    g = SplitMix64(seed)
    out = []
    for _ in range(n_tokens):
        r = g.next() % total
        acc = 0
        for e, we in enumerate(w):
            acc += we
            if r < acc:
                out.append(e)
                break
    return out


def permutation(items, seed: int) -> list:
    """Fisher-Yates shuffle of ``items`` driven by SplitMix64(seed)."""
    out = list(items)
    g = SplitMix64(seed)
    for i in range(len(out) - 1, 0, -1):
        j = g.next() % (i + 1)
        out[i], out[j] = out[j], out[i]
    return out


def delays_us(n: int, seed: int, max_us: int = 50) -> list:
    """n host-side delays in microseconds, uniform on {0, ..., max_us}."""
    g = SplitMix64(seed)
    return [g.next() % (max_us + 1) for _ in range(n)]


def remote_chunks(world: int, rank: int, chunks_per_shard: int) -> list:
    """Global ids of the chunks that do not belong to ``rank``, ascending."""
    return [p * chunks_per_shard + j for p in range(world) if p != rank
            for j in range(chunks_per_shard)]


def ring_order(world: int, rank: int, chunks_per_shard: int) -> list:
    """Ring arrival: peers rank+1, rank+2, ... (mod W); within a peer, chunks ascending."""
    return [((rank + d) % world) * chunks_per_shard + j for d in range(1, world)
            for j in range(chunks_per_shard)]


def seeded_order(world: int, rank: int, chunks_per_shard: int, seed: int) -> list:
    """A seeded random permutation of the remote chunks."""
    return permutation(remote_chunks(world, rank, chunks_per_shard), seed)


# ----------------------------------------------------------------------------------------------
# tensors (CPU); raw bit views are what both sides consume
# ----------------------------------------------------------------------------------------------

def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal_f32(shape, std: float, seed: int) -> torch.Tensor:
    """float32 samples of N(0, std^2) (std is the standard deviation)."""
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32) * std


def uniform_f32(shape, lo: float, hi: float, seed: int) -> torch.Tensor:
    """float32 samples of U[lo, hi)."""
    return torch.rand(*shape, generator=_gen(seed), dtype=torch.float32) * (hi - lo) + lo


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round a float32 tensor to bfloat16 (torch rounds to nearest even)."""
    return x.to(torch.bfloat16)


def quantize_fp8(x: torch.Tensor):
    """Per-tensor float8 e4m3fn quantisation: returns (q as torch.float8_e4m3fn, scale float).

    s = amax|x| / 448 (float32); q = clamp(x / s, -448, 448) cast to e4m3fn. Dequantised
    values are s * q.
    """
    amax = float(x.abs().max())
    s = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
    q = (x / torch.tensor(s, dtype=torch.float32)).clamp(-FP8_MAX, FP8_MAX)
    return q.to(torch.float8_e4m3fn), float(s)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """The tensor's storage as unsigned integers (uint16 for bf16, uint8 for fp8)."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn,):
        return t.view(torch.uint8).numpy()
    raise TypeError(f"raw_bits: unsupported dtype {t.dtype}")


def draw(dist: dict, shape, dtype: str, seed: int):
    """Draw a tensor from ``dist`` ({'kind': 'normal', 'std': s} or {'kind': 'uniform',
    'lo': a, 'hi': b} or {'kind': 'int', 'lo': a, 'hi': b}) and bring it to ``dtype``.

    Returns (tensor, scale): bf16 tensors have scale 1.0; fp8 tensors carry their per-tensor
    scale. 'int' draws integers uniformly in [lo, hi] (exactly representable small values).
    """
    kind = dist["kind"]
    if kind == "normal":
        x = normal_f32(shape, dist["std"], seed)
    elif kind == "uniform":
        x = uniform_f32(shape, dist["lo"], dist["hi"], seed)
    elif kind == "int":
        x = torch.randint(dist["lo"], dist["hi"] + 1, tuple(shape), generator=_gen(seed)).float()
    else:
        raise ValueError(kind)
    if dtype == "bf16":
        return to_bf16(x), 1.0
    if dtype == "fp8":
        if kind == "int":
            return x.to(torch.float8_e4m3fn), 1.0
        return quantize_fp8(x)
    if dtype == "f32":
        return x, 1.0
    raise ValueError(dtype)
