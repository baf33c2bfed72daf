"""CPU oracle for one rank's share of an overlapped AllGather+GEMM and GEMM+ReduceScatter.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only the tests,
the smoke check and the benchmark's CPU-baseline leg call it. It shares no code, header,
table or helper with the HIP library; both sides only consume the same seeded input bytes.

What it computes, and where that is stated:

* AllGather+GEMM. The page "Triton-distributed is turning communication into compiler
  territory" (cronfeed.work), section "The first move was to expose the overlap", describes an
  AllGather that moves shards into place and a GEMM that consumes them, and the overlapped
  version that cuts the data into chunks and computes on one chunk while another moves. The
  chunked schedule changes when rows arrive, never the arithmetic, so the result is the plain
  definition  C = concat(A_shard_0, ..., A_shard_{W-1}) @ B  with every element of the
  inputs decoded exactly and accumulated in fp64.
* GEMM+ReduceScatter (same section, and the page's opening, where partial products are
  summed by their owners): every rank produces a full partial product; the rows are split
  into W blocks; block p belongs to rank p; the owner's block is the sum of all W partial
  blocks. One rank's share: its own product
  P = A @ B, the W-1 non-local row blocks of P (what it sends), and its reduced block
  P[block r] + sum of the W-1 incoming partial blocks.
* GEMM+AllReduce (section "DITRON adds three levels of tiling" names AllReduce among the
  chunked collectives): every rank's partial of the same output, summed on every rank; one
  rank's share sends its partial and adds the W-1 incoming ones.
* The FFN chain (same section's task-level tiles in one persistent kernel; section "The
  performance case has a narrow, useful boundary" measures an FFN module on AMD GPUs):
  AllGather+GEMM, an elementwise activation (SiLU), then GEMM+ReduceScatter.
* AllToAll + GEMM (section "DITRON adds three levels of tiling" names AllToAll among the
  chunked collectives): every rank routes each of its tokens to one rank; the AllToAll delivers
  to a rank, from every source, the tokens routed to it (in token order, at most `cap` per
  source, the rest dropped), into one slot of `cap` rows per source; the rank's GEMM multiplies
  every delivered row by its local weight.
* The chunk / tile bookkeeping (section "DITRON adds three levels of tiling": collectives are
  broken into chunks that are paired with computation tiles, with synchronization inserted):
  which chunks a row tile needs, and the order in which row tiles become computable when the
  chunks arrive in a given order.

Number formats (not on the pages; from the formats' public definitions):
* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; the top half of a binary32.
* float8 e4m3 "fn" (OCP 8-bit floating point, E4M3): 1 sign, 4 exponent bits (bias 7), 3 fraction
  bits; exponent 0 is subnormal; no infinities; S.1111.111 is NaN; largest finite 448.

Everything here is plain numpy in float64; the matrix product is numpy's float64 matmul used as
a library step, with nothing blocked, fused or reordered around it.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16",
    "decode_e4m3fn",
    "encode_bf16_rne",
    "gather_ref",
    "ag_gemm_ref",
    "gemm_rs_ref",
    "gemm_ar_ref",
    "silu",
    "ffn_chain_ref",
    "a2a_dispatch_ref",
    "a2a_gemm_ref",
    "covering_chunks",
    "ag_mtile_order",
    "rs_mtile_order",
    "a2a_mtile_order",
]


# ----------------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (uint16), from the 1-8-7 field layout.

    normal:    (-1)^s * 2^(E-127) * (1 + f/128)
    subnormal: (-1)^s * 2^(-126)  * (f/128)          (E == 0)
    E == 255:  +-inf (f == 0) or NaN (f != 0)
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp(1.0 + f / 128.0, e - 127)
    sub = np.ldexp(f / 128.0, -126)
    val = np.where(e == 0, sub, normal)
    val = np.where(e == 255, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def decode_e4m3fn(bits) -> np.ndarray:
    """Exact float64 value of OCP float8 E4M3 ("fn") bit patterns (uint8).

    normal:    (-1)^s * 2^(E-7) * (1 + m/8)      (1 <= E <= 15, except the NaN code)
    subnormal: (-1)^s * 2^(-6)  * (m/8)          (E == 0)
    NaN:       E == 15 and m == 7 (both signs); there is no infinity.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def encode_bf16_rne(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float64 values, rounded to nearest, ties to even.

    Written from the definition, in one step from float64 (no intermediate binary32, so no
    double rounding): with e = floor(log2|x|) held at >= -126 (the subnormal range shares the
    spacing of the smallest binade), the bf16 values near |x| are the multiples of 2^(e-7);
    q = |x| / 2^(e-7) lies in [128, 256) (or [0, 128) for subnormals); the nearest integer
    (even on a tie) qi gives the bits ((e + 126) << 7) + qi. That formula also covers the carry
    qi == 256 into the next binade and a subnormal rounding up to the smallest normal.
    Results past the largest finite value become infinity. Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("encode_bf16_rne: finite inputs only")
    a = np.abs(x)
    _, ex = np.frexp(a)                      # a = m * 2^ex with m in [0.5, 1): floor(log2 a) = ex-1
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    q = np.ldexp(a, -(e - 7))                # exact: scaling by a power of two
    qf = np.floor(q)
    rem = q - qf
    qi = qf.astype(np.int64) + ((rem > 0.5) | ((rem == 0.5) & (qf.astype(np.int64) % 2 == 1)))
    bits = ((e + 126) << 7) + qi
    bits = np.where(a == 0, 0, bits)
    bits = np.minimum(bits, 0x7F80)          # overflow rounds to infinity
    sign = np.signbit(x).astype(np.int64) << 15
    return (bits | sign).astype(np.uint16)


def _decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "fp8":
        return decode_e4m3fn(raw)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------------
# AllGather + GEMM
# ----------------------------------------------------------------------------------------------

def gather_ref(shards) -> np.ndarray:
    """The gathered operand: shards concatenated along rows in rank order 0..W-1.

    Arrival order plays no part: chunks land at their shard's fixed rows (the AllGather moves
    shards "into place", page "Triton-distributed is turning communication into compiler
    territory", section "The first move was to expose the overlap").
    shards: sequence of W raw arrays of shape (Ms, K) (uint16 bf16 bits or uint8 fp8 bits).
    """
    return np.concatenate([np.asarray(s) for s in shards], axis=0)


def ag_gemm_ref(shards, b_kn, dtype: str = "bf16", scale_a: float = 1.0,
                scale_b: float = 1.0) -> np.ndarray:
    """C = concat(shards) @ B in float64 from exactly decoded inputs.

    shards: W raw arrays (Ms, K); b_kn: raw (K, N), the logical K x N weight.
    fp8 inputs are dequantised by their per-tensor scales: C = (s_a * s_b) * (A_q @ B_q),
    the scales applied in float64.
    """
    a = _decode(gather_ref(shards), dtype)
    b = _decode(np.asarray(b_kn), dtype)
    c = a @ b
    if dtype == "fp8":
        c = c * (float(scale_a) * float(scale_b))
    return c


# ----------------------------------------------------------------------------------------------
# GEMM + ReduceScatter
# ----------------------------------------------------------------------------------------------

def gemm_rs_ref(a_mk, b_kn, peers, world: int, rank: int, dtype: str = "bf16"):
    """One rank's share of GEMM+ReduceScatter, float64.

    a_mk: raw (M, K); b_kn: raw (K, N); peers: float array (W, M/W, N) whose slot p (p != rank)
    is the partial block that rank p contributes to this rank's block; slot `rank` is ignored.
    Returns (send, out):
      send: (W-1, M/W, N) — the non-local row blocks j != rank of P = A @ B, ascending j;
      out:  (M/W, N)      — P[block rank] + sum of the W-1 incoming partial blocks.
    The partials are fp32 data, read exactly (float32 -> float64 is exact).
    """
    a = _decode(np.asarray(a_mk), dtype)
    b = _decode(np.asarray(b_kn), dtype)
    p = a @ b
    m = p.shape[0]
    if m % world:
        raise ValueError("M must be a multiple of world")
    mb = m // world
    blocks = [p[j * mb:(j + 1) * mb] for j in range(world)]
    send = np.stack([blocks[j] for j in range(world) if j != rank]) if world > 1 else \
        np.zeros((0, mb, p.shape[1]))
    peers64 = np.asarray(peers, dtype=np.float64)
    out = blocks[rank].copy()
    for q in range(world):
        if q != rank:
            out = out + peers64[q]
    return send, out


# ----------------------------------------------------------------------------------------------
# GEMM + AllReduce
# ----------------------------------------------------------------------------------------------

def gemm_ar_ref(a_mk, b_kn, peers, world: int, rank: int, dtype: str = "bf16"):
    """One rank's share of GEMM+AllReduce, float64.

    The same page ("DITRON adds three levels of tiling") names AllReduce among the collectives
    the middle end cuts into chunks paired with compute tiles. Every rank holds a partial
    product of the same M x N output (the rows of its K shard times its weight rows); the
    AllReduce leaves the sum of all W partials on every rank. One rank's share in the one-shot
    form, where each rank sends its whole partial to every peer and reduces all of them itself:
      send: P = A @ B (M x N), what this rank sends to every peer;
      out:  P + the W-1 incoming partials, added in ascending rank order.
    a_mk: raw (M, K); b_kn: raw (K, N); peers: float array (W, M, N), slot `rank` ignored.
    """
    a = _decode(np.asarray(a_mk), dtype)
    b = _decode(np.asarray(b_kn), dtype)
    p = a @ b
    out = p.copy()
    peers64 = np.asarray(peers, dtype=np.float64)
    for q in range(world):
        if q != rank:
            out = out + peers64[q]
    return p, out


# ----------------------------------------------------------------------------------------------
# The FFN chain: AllGather+GEMM -> activation -> GEMM+ReduceScatter
# ----------------------------------------------------------------------------------------------

def silu(x) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + e^-x) in float64 (the activation of the Qwen3 MLP whose
    tensor-parallel FFN the pages measure on AMD GPUs). Large negative x gives -0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def ffn_chain_ref(shards, w1_kn, w2_kn, peers, world: int, rank: int, dtype: str = "bf16"):
    """One rank's share of a tensor-parallel FFN built from the two overlapped operations, float64.

    Page "Triton-distributed is turning communication into compiler territory", section "DITRON
    adds three levels of tiling" (task-level tiles scheduled as one persistent kernel) and
    section "The performance case has a narrow, useful boundary" (the FFN module on AMD GPUs):
    the column-parallel first layer gathers the activations (AllGather+GEMM), the activation is
    applied elementwise, and the row-parallel second layer's partial product is reduce-scattered.
      h    = bf16(silu(concat(shards) @ W1))           (M x N1)
      y    = h @ W2                                     (M x N2, this rank's partial)
      send = the W-1 non-local row blocks of y, ascending block index (M/W rows each)
      out  = y[block rank] + the W-1 incoming partial blocks, ascending rank order
    The activation is the second layer's operand, so it is a tensor of the operands' type: h is
    silu of the exact product rounded to bf16 (nearest, ties to even), and the second product
    uses those values.
    shards: W raw arrays (Ms, K1); w1_kn: raw (K1, N1); w2_kn: raw (N1, N2); peers: float array
    (W, M/W, N2), slot `rank` ignored. Returns (h, send, out), h as the exact values of the bf16.
    """
    g = _decode(gather_ref(shards), dtype)
    h = decode_bf16(encode_bf16_rne(silu(g @ _decode(np.asarray(w1_kn), dtype))))
    y = h @ _decode(np.asarray(w2_kn), dtype)
    m = y.shape[0]
    if m % world:
        raise ValueError("M must be a multiple of world")
    mb = m // world
    blocks = [y[j * mb:(j + 1) * mb] for j in range(world)]
    send = np.stack([blocks[j] for j in range(world) if j != rank]) if world > 1 else \
        np.zeros((0, mb, y.shape[1]))
    out = blocks[rank].copy()
    peers64 = np.asarray(peers, dtype=np.float64)
    for q in range(world):
        if q != rank:
            out = out + peers64[q]
    return h, send, out


# ----------------------------------------------------------------------------------------------
# Chunk / tile bookkeeping
# ----------------------------------------------------------------------------------------------

# ----------------------------------------------------------------------------------------------
# AllToAll (dispatch) + GEMM
# ----------------------------------------------------------------------------------------------

def a2a_dispatch_ref(tokens, dests, rank: int, cap: int):
    """The rows an AllToAll delivers to `rank`: one block per source rank.

    tokens: W raw arrays (T_p, K), the token rows source p holds; dests: W integer sequences
    (T_p,), the rank each of those tokens is routed to. Source p's block is its tokens whose
    destination is `rank`, in token order, the first `cap` of them (tokens past the capacity are
    dropped). Written token by token. Returns a list of W raw arrays (count_p, K).
    """
    out = []
    for t, d in zip(tokens, dests):
        t = np.asarray(t)
        rows = []
        for i in range(len(d)):
            if int(d[i]) == rank and len(rows) < cap:
                rows.append(i)
        out.append(t[rows] if rows else np.zeros((0, t.shape[1]), dtype=t.dtype))
    return out


def a2a_gemm_ref(blocks, b_kn, dtype: str = "bf16", scale_a: float = 1.0, scale_b: float = 1.0):
    """The GEMM on the delivered rows: every source's block times the local weight, float64.

    blocks: W raw arrays (count_p, K) (a2a_dispatch_ref); b_kn: raw (K, N). fp8 inputs are
    dequantised by their per-tensor scales as in ag_gemm_ref. Returns W arrays (count_p, N): the
    rows of C in slot p that hold a delivered row; the slot's rows past count_p hold none.
    """
    b = _decode(np.asarray(b_kn), dtype)
    out = []
    for blk in blocks:
        c = _decode(np.asarray(blk), dtype) @ b if len(blk) else np.zeros((0, b.shape[1]))
        if dtype == "fp8":
            c = c * (float(scale_a) * float(scale_b))
        out.append(c)
    return out


def covering_chunks(row_lo: int, row_hi: int, chunk_rows: int) -> list[int]:
    """Chunk indices whose rows [c*cr, (c+1)*cr) meet the half-open row range [row_lo, row_hi).

    Written as a direct test of every chunk against the range (no division tricks).
    """
    out = []
    c = 0
    while c * chunk_rows < row_hi:
        lo, hi = c * chunk_rows, (c + 1) * chunk_rows
        if lo < row_hi and hi > row_lo:
            out.append(c)
        c += 1
    return out


def ag_mtile_order(world: int, rank: int, m_shard: int, chunk_rows: int, order, bm: int):
    """Order in which the row tiles of C become computable in AllGather+GEMM.

    Rows of the gathered operand are cut into chunks of `chunk_rows` rows of one shard; global
    chunk c covers gathered rows [c*cr, (c+1)*cr) and belongs to shard c // (m_shard/cr).
    The local shard's chunks are present from the start; the remote ones arrive in `order`.
    A row tile of `bm` rows is computable once every chunk it overlaps is present, i.e. at the
    arrival position of its latest remote chunk (-1 if it needs none). Tiles are taken in
    increasing computable position, ties by tile index: local rows first, then the arrival
    order of the chunks ("compute on one chunk while another is still moving").
    Returns (tile_order, ready_pos) as lists.
    """
    m = world * m_shard
    cps = m_shard // chunk_rows
    pos = {c: i for i, c in enumerate(order)}
    n_tiles = -(-m // bm)
    ready = []
    for t in range(n_tiles):
        lo, hi = t * bm, min((t + 1) * bm, m)
        need = [pos[c] for c in covering_chunks(lo, hi, chunk_rows) if c // cps != rank]
        ready.append(max(need) if need else -1)
    tile_order = sorted(range(n_tiles), key=lambda t: (ready[t], t))
    return tile_order, ready


def rs_mtile_order(world: int, rank: int, m_block: int, chunk_rows: int, order, bm: int):
    """Order in which this rank's row tiles are computed in GEMM+ReduceScatter.

    Row blocks of P are tiled separately (a tile never spans two blocks); block j has
    ceil(m_block/bm) tiles. Non-local blocks come first, in send order rank+1, ..., rank+W-1
    (mod W), each block's tiles ascending: they need nothing from peers. The local block comes
    last: its tile i covers local rows [i*bm, ...) and needs, from every peer p != rank, the
    incoming chunks of that peer's block overlapping those rows; global chunk id
    p * (m_block/cr) + j. It is computable at the arrival position of the latest of them.
    Returns a list of (block, tile_in_block) pairs.
    """
    cpb = m_block // chunk_rows
    pos = {c: i for i, c in enumerate(order)}
    tpb = -(-m_block // bm)
    seq = []
    for d in range(1, world):
        j = (rank + d) % world
        seq.extend((j, i) for i in range(tpb))
    ready = []
    for i in range(tpb):
        lo, hi = i * bm, min((i + 1) * bm, m_block)
        need = [pos[p * cpb + c] for p in range(world) if p != rank
                for c in covering_chunks(lo, hi, chunk_rows)]
        ready.append(max(need) if need else -1)
    seq.extend((rank, i) for i in sorted(range(tpb), key=lambda i: (ready[i], i)))
    return seq


def a2a_mtile_order(world: int, rank: int, cap: int, chunk_rows: int, counts, order, bm: int):
    """Order in which the row tiles of C become computable in AllToAll+GEMM.

    The receive buffer has W slots of `cap` rows; slot p holds rows [p*cap, p*cap + counts[p]).
    Chunk c = p*(cap/cr) + j covers rows [c*cr, (c+1)*cr) and holds rows when j*cr < counts[p].
    The local slot's chunks and the chunks that hold no row are present from the start; the
    others arrive at their position in `order` (every remote chunk listed). A row tile of `bm`
    rows that holds no row is not computed at all; the others are computable at the arrival
    position of the latest chunk they cover that holds rows (-1 if none), and are taken in
    increasing position, ties by tile index. Returns the tile order as a list.
    """
    cps = cap // chunk_rows
    m = world * cap
    pos = {c: i for i, c in enumerate(order)}

    def holds(c):
        return (c % cps) * chunk_rows < counts[c // cps]
    ready = {}
    for t in range(-(-m // bm)):
        lo, hi = t * bm, min((t + 1) * bm, m)
        if not any((x - (x // cap) * cap) < counts[x // cap] for x in range(lo, hi)):
            continue
        need = [pos[c] for c in covering_chunks(lo, hi, chunk_rows) if c // cps != rank and holds(c)]
        ready[t] = max(need) if need else -1
    return sorted(ready, key=lambda t: (ready[t], t))

