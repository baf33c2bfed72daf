"""Pins of the CPU oracle to things other than itself (CPU only).

* number formats: exhaustive comparison with torch's independent casts, plus values fixed by
  the format definitions;
* the products: exact rational brute force (bf16 and e4m3fn values are dyadic rationals, so the
  exact C is computable with fractions.Fraction) and hand-derived worked examples;
* the chunk/tile bookkeeping: an event simulation of chunk arrivals, independent of the
  oracle's "latest arrival position" formulation;
* planted mistakes: plausible bugs planted in copies of the oracle must fail these pins: a
  transposed weight, shards concatenated in arrival order instead of rank order, a dropped
  peer in the ReduceScatter sum, an e4m3 decoder off by a factor of 2, a tile order blind to the
  arrival order, the AllReduce adding the rank's own slot, and the FFN chain without its
  activation or with the activation after the second product.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import agg_oracle as O
from allgather_gemm_persistent_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _bf16_bits(vals):
    return inputs.raw_bits(torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(torch.bfloat16))


def _fp8_bits(vals):
    return inputs.raw_bits(torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn))


def _bits(vals, dtype):
    return _bf16_bits(vals) if dtype == "bf16" else _fp8_bits(vals)


# ------------------------------------------------------------------ number formats

def test_decode_bf16_exhaustive_vs_torch():
    allb = np.arange(65536, dtype=np.uint16)
    mine = O.decode_bf16(allb)
    ref = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_decode_e4m3fn_exhaustive_vs_torch():
    allb = np.arange(256, dtype=np.uint8)
    mine = O.decode_e4m3fn(allb)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


@pytest.mark.parametrize("bits,val", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127), (0x3E80, 0.25), (0x4049, 3.140625),
])
def test_decode_bf16_definition_values(bits, val):
    assert O.decode_bf16(np.uint16(bits)) == val


@pytest.mark.parametrize("bits,val", [
    (0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9),
    (0xB8, -1.0), (0x30, 0.5), (0x77, 240.0),
])
def test_decode_e4m3fn_definition_values(bits, val):
    assert O.decode_e4m3fn(np.uint8(bits)) == val


def test_e4m3fn_nan_codes_and_no_inf():
    d = O.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2 and not np.isinf(d).any()
    assert np.nanmax(d) == 448.0


def test_encode_bf16_vs_torch_on_float32():
    """torch rounds binary32 -> bf16 to nearest even in one step: compare on float32 inputs."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    # add every bf16 midpoint and its neighbours (the tie cases)
    allb = np.arange(0, 0x7F80, dtype=np.uint32)
    mids = ((allb << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(0)), -mids])
    x = x[np.isfinite(x)]
    mine = O.encode_bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_encode_bf16_exact_on_float64():
    """float64 inputs: the nearer neighbour by exact rational distance, even on a tie."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-60, 60, 3000))
    enc = O.encode_bf16_rne(x)
    for xi, bi in zip(x, enc):
        v = Fraction(float(xi))
        got = Fraction(float(O.decode_bf16(bi)))
        # neighbours of the chosen value
        up = Fraction(float(O.decode_bf16(np.uint16(bi + 1))))
        dn = Fraction(float(O.decode_bf16(np.uint16(bi - 1)))) if (bi & 0x7FFF) else -got
        assert abs(v - got) <= abs(v - up) and abs(v - got) <= abs(v - dn)


def test_encode_decode_roundtrip_all_finite_bf16():
    allb = np.arange(65536, dtype=np.uint16)
    d = O.decode_bf16(allb)
    fin = np.isfinite(d)
    back = O.encode_bf16_rne(d[fin])
    assert np.array_equal(back, allb[fin])


# ------------------------------------------------------------------ products: brute force

def _exact_matmul(a_vals, b_vals):
    """Exact rational product with pure-Python loops (tiny shapes only)."""
    m, k = len(a_vals), len(a_vals[0])
    n = len(b_vals[0])
    return [[sum((a_vals[i][t] * b_vals[t][j] for t in range(k)), Fraction(0)) for j in range(n)]
            for i in range(m)]


def _frac_matrix(raw, dtype):
    dec = O.decode_bf16 if dtype == "bf16" else O.decode_e4m3fn
    vals = dec(raw)
    return [[Fraction(float(v)) for v in row] for row in vals]


def _random_raw(shape, dtype, rng):
    if dtype == "bf16":
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    else:
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * 30).to(torch.float8_e4m3fn)
    return inputs.raw_bits(x)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("world,m_shard,k,n", [(1, 2, 16, 3), (2, 1, 32, 5), (3, 2, 48, 4),
                                               (8, 1, 16, 2)])
def test_ag_gemm_vs_exact_rational(dtype, world, m_shard, k, n):
    rng = np.random.default_rng(world * 100 + k)
    shards = [_random_raw((m_shard, k), dtype, rng) for _ in range(world)]
    b = _random_raw((k, n), dtype, rng)
    sa, sb = (0.75, 0.125) if dtype == "fp8" else (1.0, 1.0)
    c = O.ag_gemm_ref(shards, b, dtype, sa, sb)
    a_frac = sum((_frac_matrix(s, dtype) for s in shards), [])
    exact = _exact_matmul(a_frac, _frac_matrix(b, dtype))
    scale = Fraction(sa) * Fraction(sb) if dtype == "fp8" else Fraction(1)
    for i in range(world * m_shard):
        for j in range(n):
            e = exact[i][j] * scale
            assert abs(Fraction(float(c[i, j])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("world,rank", [(1, 0), (2, 1), (3, 0), (4, 2)])
def test_gemm_rs_vs_exact_rational(world, rank):
    rng = np.random.default_rng(world * 10 + rank)
    mb, k, n = 2, 16, 3
    a = _random_raw((world * mb, k), "bf16", rng)
    b = _random_raw((k, n), "bf16", rng)
    peers = rng.standard_normal((world, mb, n)).astype(np.float32)
    send, out = O.gemm_rs_ref(a, b, peers, world, rank)
    p = _exact_matmul(_frac_matrix(a, "bf16"), _frac_matrix(b, "bf16"))
    others = [j for j in range(world) if j != rank]
    assert send.shape == (world - 1, mb, n)
    for s_i, j in enumerate(others):
        for i in range(mb):
            for c in range(n):
                e = p[j * mb + i][c]
                assert abs(Fraction(float(send[s_i, i, c])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)
    for i in range(mb):
        for c in range(n):
            e = p[rank * mb + i][c] + sum(Fraction(float(peers[q, i, c])) for q in others)
            assert abs(Fraction(float(out[i, c])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_gather_places_rows_by_rank_not_arrival():
    """Row-id encoded shards: gathered row i must carry id i (shard p holds ids p*Ms..)."""
    world, ms, k = 5, 3, 4
    shards = [_bf16_bits([[float(p * ms + i)] * k for i in range(ms)]) for p in range(world)]
    g = O.decode_bf16(O.gather_ref(shards))
    assert np.array_equal(g[:, 0], np.arange(world * ms, dtype=np.float64))


# ------------------------------------------------------------------ worked examples

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["ag"], ids=lambda c: c["name"])
def test_ag_worked_examples(case):
    dt = case["dtype"]
    shards = [_bits(s, dt) for s in case["shards"]]
    c = O.ag_gemm_ref(shards, _bits(case["b"], dt), dt, case["scale_a"], case["scale_b"])
    assert np.array_equal(c, np.array(case["c"], dtype=np.float64))


@pytest.mark.parametrize("case", _golden()["rs"], ids=lambda c: c["name"])
def test_rs_worked_examples(case):
    send, out = O.gemm_rs_ref(_bf16_bits(case["a"]), _bf16_bits(case["b"]),
                              np.array(case["peers"], dtype=np.float32), case["world"], case["rank"])
    assert np.array_equal(send, np.array(case["send"], dtype=np.float64))
    assert np.array_equal(out, np.array(case["out"], dtype=np.float64))


@pytest.mark.parametrize("case", _golden()["schedule"], ids=lambda c: c["name"])
def test_schedule_worked_examples(case):
    for key in case:
        if key.startswith("bm") and key[2:].isdigit():
            order, _ = O.ag_mtile_order(case["world"], case["rank"], case["m_shard"],
                                        case["chunk_rows"], case["order"], int(key[2:]))
            assert order == case[key], key


# ------------------------------------------------------------------ bookkeeping: simulation

def _simulate_ag(world, rank, ms, cr, order, bm):
    """Deliver chunks one at a time; after each delivery, emit (ascending) every row tile whose
    rows are all present and that was not emitted before."""
    m = world * ms
    present = np.zeros(m, dtype=bool)
    present[rank * ms:(rank + 1) * ms] = True
    n_tiles = -(-m // bm)
    done, seq = set(), []

    def sweep():
        for t in range(n_tiles):
            if t not in done and present[t * bm:min((t + 1) * bm, m)].all():
                done.add(t)
                seq.append(t)
    sweep()
    for c in order:
        present[c * cr:(c + 1) * cr] = True
        sweep()
    return seq


@pytest.mark.parametrize("world,rank,ms,cr,bm", [
    (2, 0, 128, 64, 64), (2, 1, 128, 64, 128), (8, 0, 512, 128, 256), (8, 3, 16, 16, 128),
    (8, 0, 1024, 256, 256), (3, 2, 10, 5, 4), (4, 1, 12, 3, 7), (8, 7, 8, 2, 3)])
@pytest.mark.parametrize("order_seed", [0, 1, 2])
def test_ag_mtile_order_vs_simulation(world, rank, ms, cr, bm, order_seed):
    cps = ms // cr
    order = inputs.seeded_order(world, rank, cps, order_seed) if order_seed else \
        inputs.ring_order(world, rank, cps)
    got, ready = O.ag_mtile_order(world, rank, ms, cr, order, bm)
    assert got == _simulate_ag(world, rank, ms, cr, order, bm)
    assert sorted(got) == list(range(-(-world * ms // bm)))


@pytest.mark.parametrize("lo,hi,cr", [(0, 1, 1), (0, 128, 64), (5, 37, 8), (63, 65, 64),
                                      (100, 356, 128), (7, 8, 3)])
def test_covering_chunks_vs_per_row(lo, hi, cr):
    assert O.covering_chunks(lo, hi, cr) == sorted({r // cr for r in range(lo, hi)})


def _simulate_rs(world, rank, mb, cr, order, bm):
    tpb = -(-mb // bm)
    seq = [((rank + d) % world, i) for d in range(1, world) for i in range(tpb)]
    cpb = mb // cr
    present = {p: np.zeros(mb, dtype=bool) for p in range(world) if p != rank}
    done = set()

    def sweep():
        for i in range(tpb):
            lo, hi = i * bm, min((i + 1) * bm, mb)
            if i not in done and all(present[p][lo:hi].all() for p in present):
                done.add(i)
                seq.append((rank, i))
    sweep()
    for c in order:
        p, j = divmod(c, cpb)
        present[p][j * cr:(j + 1) * cr] = True
        sweep()
    return seq


@pytest.mark.parametrize("world,rank,mb,cr,bm", [(8, 0, 1024, 128, 256), (2, 1, 64, 16, 32),
                                                  (4, 2, 30, 5, 8), (3, 0, 12, 12, 5)])
def test_rs_mtile_order_vs_simulation(world, rank, mb, cr, bm):
    order = inputs.seeded_order(world, rank, mb // cr, 99)
    assert O.rs_mtile_order(world, rank, mb, cr, order, bm) == _simulate_rs(world, rank, mb, cr, order, bm)


# ------------------------------------------------------------------ planted mistakes

def _ag_transposed_b(shards, b, dtype="bf16", sa=1.0, sb=1.0):
    a = O.decode_bf16(O.gather_ref(shards))
    bb = O.decode_bf16(b)
    return a @ bb.T.reshape(bb.shape) if bb.shape[0] == bb.shape[1] else a @ bb[::-1]


def _ag_arrival_concat(shards, b, dtype="bf16", sa=1.0, sb=1.0):
    a = O.decode_bf16(np.concatenate(shards[::-1], axis=0))
    return a @ O.decode_bf16(b)


def _rs_drop_last_peer(a, b, peers, world, rank, dtype="bf16"):
    send, out = O.gemm_rs_ref(a, b, peers, world, rank)
    last = max(q for q in range(world) if q != rank)
    return send, out - np.asarray(peers, dtype=np.float64)[last]


def _decode_e4m3_wrong_bias(bits):
    return O.decode_e4m3fn(bits) * 2.0


@pytest.mark.parametrize("mutant", ["transposed_b", "arrival_concat"])
def test_planted_ag_mistakes_fail_the_pins(mutant):
    fn = {"transposed_b": _ag_transposed_b, "arrival_concat": _ag_arrival_concat}[mutant]
    failed = False
    for case in _golden()["ag"]:
        if case["dtype"] != "bf16":
            continue
        shards = [_bf16_bits(s) for s in case["shards"]]
        c = fn(shards, _bf16_bits(case["b"]))
        if c.shape != np.array(case["c"]).shape or not np.array_equal(c, np.array(case["c"], dtype=np.float64)):
            failed = True
    assert failed


def test_planted_rs_mistake_fails_the_pin():
    case = _golden()["rs"][0]
    send, out = _rs_drop_last_peer(_bf16_bits(case["a"]), _bf16_bits(case["b"]),
                                   np.array(case["peers"], dtype=np.float32), case["world"], case["rank"])
    assert not np.array_equal(out, np.array(case["out"], dtype=np.float64))


def test_planted_decoder_mistake_fails_the_pin():
    allb = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    bad = _decode_e4m3_wrong_bias(allb)
    ok = ~np.isnan(ref)
    assert not np.array_equal(bad[ok], ref[ok])


def test_planted_schedule_mistake_fails_the_pin():
    """A schedule that ignores arrival order (plain ascending tiles) fails the simulation."""
    world, rank, ms, cr, bm = 8, 0, 512, 128, 256
    order = inputs.ring_order(world, rank, ms // cr)[::-1]
    naive = list(range(world * ms // bm))
    assert naive != _simulate_ag(world, rank, ms, cr, order, bm)


# ------------------------------------------------------------------ GEMM + AllReduce

@pytest.mark.parametrize("world,rank", [(1, 0), (2, 1), (4, 3), (8, 0)])
def test_gemm_ar_vs_exact_rational(world, rank):
    rng = np.random.default_rng(700 + world * 10 + rank)
    m, k, n = 3, 16, 4
    a = _random_raw((m, k), "bf16", rng)
    b = _random_raw((k, n), "bf16", rng)
    peers = rng.standard_normal((world, m, n)).astype(np.float32)
    send, out = O.gemm_ar_ref(a, b, peers, world, rank)
    p = _exact_matmul(_frac_matrix(a, "bf16"), _frac_matrix(b, "bf16"))
    for i in range(m):
        for c in range(n):
            e = p[i][c]
            assert abs(Fraction(float(send[i, c])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)
            e = e + sum(Fraction(float(peers[q, i, c])) for q in range(world) if q != rank)
            assert abs(Fraction(float(out[i, c])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("case", _golden()["ar"], ids=lambda c: c["name"])
def test_ar_worked_examples(case):
    send, out = O.gemm_ar_ref(_bf16_bits(case["a"]), _bf16_bits(case["b"]),
                              np.array(case["peers"], dtype=np.float32), case["world"], case["rank"])
    assert np.array_equal(send, np.array(case["send"], dtype=np.float64))
    assert np.array_equal(out, np.array(case["out"], dtype=np.float64))


def test_planted_ar_mistake_fails_the_pin():
    """Adding the rank's own peer slot (instead of skipping it) fails the worked example."""
    case = _golden()["ar"][0]
    peers = np.array(case["peers"], dtype=np.float64)
    send, _ = O.gemm_ar_ref(_bf16_bits(case["a"]), _bf16_bits(case["b"]), peers, case["world"], case["rank"])
    wrong = send + peers.sum(axis=0)
    assert not np.array_equal(wrong, np.array(case["out"], dtype=np.float64))


# ------------------------------------------------------------------ the activation (SiLU)

def _silu_decimal(x) -> Fraction:
    """x / (1 + e^-x) with decimal's own 60-digit exp: an implementation independent of numpy's."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        d = decimal.Decimal(Fraction(x).numerator) / decimal.Decimal(Fraction(x).denominator)
        return Fraction(d / (1 + (-d).exp()))


@pytest.mark.parametrize("x", [0.0, 1e-8, -1e-8, 0.5, -0.5, 1.0, -1.0, 2.0, -3.25, 7.5, -12.0,
                               20.0, -40.0, 88.0, -700.0])
def test_silu_vs_high_precision(x):
    got = Fraction(float(O.silu(np.float64(x))))
    want = _silu_decimal(x)
    assert abs(got - want) <= abs(want) * Fraction(1, 10 ** 15) + Fraction(1, 10 ** 300)


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4
    assert abs(float(O.silu(np.log(3.0))) - 0.75 * np.log(3.0)) <= 1e-15
    # x sigmoid(x) - (-x) sigmoid(-x) = x
    xs = np.linspace(-20, 20, 81)
    assert np.allclose(O.silu(xs) - O.silu(-xs), xs, rtol=0, atol=1e-13)
    # the large-|x| limits: silu(x) -> x, silu(-x) -> -0
    assert O.silu(800.0) == 800.0 and O.silu(-800.0) == 0.0


# ------------------------------------------------------------------ the FFN chain

def _bf16_round(x: Fraction) -> Fraction:
    """Nearest bf16 (ties to even) of an exact value, through torch's float32 -> bfloat16 cast
    (float32 first: a second rounding only on the rare values within 2^-24 of a bf16 midpoint)."""
    v = torch.tensor(float(x), dtype=torch.float32).to(torch.bfloat16).to(torch.float64).item()
    return Fraction(v)


def _ffn_exact(shards, w1, w2, peers, world, rank):
    """Exact rationals for both products, 60-digit SiLU in between, the activation rounded to bf16
    (the second layer's operand type)."""
    g = sum((_frac_matrix(s, "bf16") for s in shards), [])
    pre = _exact_matmul(g, _frac_matrix(w1, "bf16"))
    h = [[_bf16_round(_silu_decimal(v)) for v in row] for row in pre]
    y = _exact_matmul(h, _frac_matrix(w2, "bf16"))
    mb = len(y) // world
    send = [[y[j * mb + i] for i in range(mb)] for j in range(world) if j != rank]
    out = [[y[rank * mb + i][c] + sum(Fraction(float(peers[q][i][c])) for q in range(world) if q != rank)
            for c in range(len(y[0]))] for i in range(mb)]
    return h, send, out


def _close(got, want):
    return abs(Fraction(float(got)) - want) <= abs(want) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("world,rank", [(1, 0), (2, 1), (4, 2)])
def test_ffn_chain_vs_exact(world, rank):
    rng = np.random.default_rng(800 + world * 10 + rank)
    ms, k1, n1, n2 = 2, 8, 6, 3
    shards = [_random_raw((ms, k1), "bf16", rng) for _ in range(world)]
    w1 = _random_raw((k1, n1), "bf16", rng)
    w2 = _random_raw((n1, n2), "bf16", rng)
    peers = rng.standard_normal((world, ms, n2)).astype(np.float32)
    h, send, out = O.ffn_chain_ref(shards, w1, w2, peers, world, rank)
    eh, es, eo = _ffn_exact(shards, w1, w2, peers, world, rank)
    assert all(_close(h[i, j], eh[i][j]) for i in range(len(eh)) for j in range(n1))
    assert send.shape == (world - 1, ms, n2)
    assert all(_close(send[b, i, c], es[b][i][c]) for b in range(world - 1) for i in range(ms) for c in range(n2))
    assert all(_close(out[i, c], eo[i][c]) for i in range(ms) for c in range(n2))


@pytest.mark.parametrize("case", _golden()["ffn"], ids=lambda c: c["name"])
def test_ffn_worked_examples(case):
    s = 2.0 / (1.0 + np.exp(-2.0))          # silu(2) from its definition
    # h is rounded to bf16: s = 1.7616 lies between the bf16 values 225/128 and 226/128 (spacing
    # 2^-7 in [1, 2)), nearer the first; s - 2 = -0.23841 lies between -244/1024 and -245/1024
    # (spacing 2^-10 in [1/8, 1/4)), nearer the first
    hs, hm = 225 / 128, -244 / 1024
    assert abs(s - hs) < 2 ** -8 and abs((s - 2.0) - hm) < 2 ** -11
    h, send, out = O.ffn_chain_ref([_bf16_bits(x) for x in case["shards"]], _bf16_bits(case["w1"]),
                                   _bf16_bits(case["w2"]), np.array(case["peers"], dtype=np.float32),
                                   case["world"], case["rank"])
    assert np.array_equal(h, [[0.0, hs], [hm, 0.0]])
    assert np.array_equal(send, [[[hm]]])
    assert np.array_equal(out, [[hs + 0.5]])


def _ffn_no_activation(shards, w1, w2, peers, world, rank):
    g = O.decode_bf16(O.gather_ref(shards))
    y = (g @ O.decode_bf16(w1)) @ O.decode_bf16(w2)
    mb = y.shape[0] // world
    return y[rank * mb:(rank + 1) * mb] + sum(np.asarray(peers, np.float64)[q] for q in range(world) if q != rank)


def _ffn_activation_last(shards, w1, w2, peers, world, rank):
    g = O.decode_bf16(O.gather_ref(shards))
    y = O.silu((g @ O.decode_bf16(w1)) @ O.decode_bf16(w2))
    mb = y.shape[0] // world
    return y[rank * mb:(rank + 1) * mb] + sum(np.asarray(peers, np.float64)[q] for q in range(world) if q != rank)


@pytest.mark.parametrize("mutant", [_ffn_no_activation, _ffn_activation_last])
def test_planted_ffn_mistakes_fail_the_pins(mutant):
    rng = np.random.default_rng(811)
    world, rank, ms, k1, n1, n2 = 2, 1, 2, 8, 6, 3
    shards = [_random_raw((ms, k1), "bf16", rng) for _ in range(world)]
    w1 = _random_raw((k1, n1), "bf16", rng)
    w2 = _random_raw((n1, n2), "bf16", rng)
    peers = rng.standard_normal((world, ms, n2)).astype(np.float32)
    _, _, eo = _ffn_exact(shards, w1, w2, peers, world, rank)
    bad = mutant(shards, w1, w2, peers, world, rank)
    assert not all(_close(bad[i, c], eo[i][c]) for i in range(ms) for c in range(n2))


# ------------------------------------------------------------------ AllToAll (dispatch) + GEMM

def _a2a_case(world, t, k, rng, dtype="bf16"):
    tokens = [_random_raw((t, k), dtype, rng) for _ in range(world)]
    dests = [list(rng.integers(0, world, size=t)) for _ in range(world)]
    return tokens, dests


@pytest.mark.parametrize("world,rank,t,cap", [(1, 0, 5, 5), (2, 1, 6, 2), (3, 0, 7, 3), (4, 2, 9, 9)])
def test_a2a_dispatch_token_by_token(world, rank, t, cap):
    """Every source's block for a rank is its tokens routed there, in token order, the first cap.
    Checked against row ids written into the tokens themselves (token i of source p holds the
    value 16*p + i in every column), so a dropped, reordered or misrouted row shows up."""
    rng = np.random.default_rng(900 + world * 10 + rank)
    dests = [list(rng.integers(0, world, size=t)) for _ in range(world)]
    tokens = [_bf16_bits([[16 * p + i] * 2 for i in range(t)]) for p in range(world)]
    blocks = O.a2a_dispatch_ref(tokens, dests, rank, cap)
    for p in range(world):
        ids = [int(v) for v in O.decode_bf16(blocks[p])[:, 0] - 16 * p] if len(blocks[p]) else []
        routed = [i for i in range(t) if dests[p][i] == rank]
        assert ids == routed[:cap]
        assert np.array_equal(O.decode_bf16(blocks[p])[:, 1], O.decode_bf16(blocks[p])[:, 0])


def test_a2a_dispatch_delivers_every_token_once():
    """With a capacity no source exceeds, the blocks all ranks receive from one source are a
    partition of that source's tokens (each token delivered once, to its destination)."""
    rng = np.random.default_rng(931)
    world, t, k = 4, 11, 3
    tokens, dests = _a2a_case(world, t, k, rng)
    for p in range(world):
        got = np.concatenate([O.a2a_dispatch_ref(tokens, dests, r, t)[p] for r in range(world)])
        assert sorted(map(tuple, got.tolist())) == sorted(map(tuple, np.asarray(tokens[p]).tolist()))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_a2a_gemm_vs_exact_rational(dtype):
    rng = np.random.default_rng(941)
    world, rank, t, k, n, cap = 3, 1, 5, 16, 3, 2
    tokens, dests = _a2a_case(world, t, k, rng, dtype)
    blocks = O.a2a_dispatch_ref(tokens, dests, rank, cap)
    b = _random_raw((k, n), dtype, rng)
    sa, sb = (0.5, 0.25) if dtype == "fp8" else (1.0, 1.0)
    c = O.a2a_gemm_ref(blocks, b, dtype, sa, sb)
    scale = Fraction(sa) * Fraction(sb) if dtype == "fp8" else Fraction(1)
    for p in range(world):
        assert c[p].shape == (len(blocks[p]), n)
        if not len(blocks[p]):
            continue
        exact = _exact_matmul(_frac_matrix(blocks[p], dtype), _frac_matrix(b, dtype))
        for i in range(len(blocks[p])):
            for j in range(n):
                assert Fraction(float(c[p][i, j])) == exact[i][j] * scale


@pytest.mark.parametrize("case", _golden()["a2a"], ids=lambda c: c["name"])
def test_a2a_worked_examples(case):
    tokens = [_bf16_bits(x) if x else np.zeros((0, 2), np.uint16) for x in case["tokens"]]
    blocks = O.a2a_dispatch_ref(tokens, case["dests"], case["rank"], case["cap"])
    for p, want in enumerate(case["blocks"]):
        assert np.array_equal(O.decode_bf16(blocks[p]).reshape(-1, 2), np.array(want, np.float64).reshape(-1, 2))
    c = O.a2a_gemm_ref(blocks, _bf16_bits(case["b"]))
    for p, want in enumerate(case["c"]):
        assert np.array_equal(c[p].reshape(-1, 2), np.array(want, np.float64).reshape(-1, 2))


def _simulate_a2a(world, rank, cap, cr, counts, order, bm):
    """Deliver chunks one at a time (a chunk's rows, token rows or not, arrive together; rows of
    chunks without a token are there from the start); after each delivery, emit (ascending)
    every row tile that holds a token and whose rows are all present."""
    m = world * cap
    token = np.array([(x % cap) < counts[x // cap] for x in range(m)])
    present = np.zeros(m, dtype=bool)
    present[rank * cap:(rank + 1) * cap] = True
    for c in range(world * (cap // cr)):
        if not token[c * cr:(c + 1) * cr].any():
            present[c * cr:(c + 1) * cr] = True
    n_tiles = -(-m // bm)
    done, seq = set(), []

    def sweep():
        for t in range(n_tiles):
            rows = slice(t * bm, min((t + 1) * bm, m))
            if t not in done and token[rows].any() and present[rows].all():
                done.add(t)
                seq.append(t)
    sweep()
    for c in order:
        present[c * cr:(c + 1) * cr] = True
        sweep()
    return seq


@pytest.mark.parametrize("world,rank,cap,cr,bm,counts", [
    (2, 0, 8, 4, 4, [3, 5]), (3, 1, 12, 4, 8, [12, 0, 7]), (4, 3, 6, 2, 4, [1, 6, 0, 2]),
    (8, 0, 640, 128, 256, [626, 603, 606, 617, 629, 614, 640, 616]), (8, 5, 16, 4, 64, [0] * 8),
    (5, 2, 10, 5, 3, [10, 4, 5, 0, 9]), (3, 0, 9, 3, 5, [2, 9, 4])])
@pytest.mark.parametrize("order_seed", [0, 1, 2])
def test_a2a_mtile_order_vs_simulation(world, rank, cap, cr, bm, counts, order_seed):
    cps = cap // cr
    order = inputs.seeded_order(world, rank, cps, 7 + order_seed) if order_seed else \
        inputs.ring_order(world, rank, cps)
    got = O.a2a_mtile_order(world, rank, cap, cr, counts, order, bm)
    assert got == _simulate_a2a(world, rank, cap, cr, counts, order, bm)


def _a2a_ignore_cap(tokens, dests, rank, cap):
    return O.a2a_dispatch_ref(tokens, dests, rank, 10 ** 9)


def _a2a_last_cap(tokens, dests, rank, cap):
    out = []
    for t, d in zip(tokens, dests):
        rows = [i for i in range(len(d)) if int(d[i]) == rank][-cap:] if cap else []
        out.append(np.asarray(t)[rows])
    return out


def _a2a_wrong_rank(tokens, dests, rank, cap):
    return O.a2a_dispatch_ref(tokens, dests, (rank + 1) % len(tokens), cap)


@pytest.mark.parametrize("mutant", [_a2a_ignore_cap, _a2a_last_cap, _a2a_wrong_rank])
def test_planted_a2a_mistakes_fail_the_pins(mutant):
    case = _golden()["a2a"][0]
    tokens = [_bf16_bits(x) if x else np.zeros((0, 2), np.uint16) for x in case["tokens"]]
    blocks = mutant(tokens, case["dests"], case["rank"], case["cap"])
    same = all(np.array_equal(O.decode_bf16(np.asarray(blk)).reshape(-1, 2), np.array(w, np.float64).reshape(-1, 2))
               for blk, w in zip(blocks, case["blocks"]))
    assert not same


def test_planted_a2a_schedule_mistake_fails_the_pin():
    """A tile order that waits for chunks holding no token at their place in the arrival order
    (instead of counting them present) differs from the simulation."""
    world, rank, cap, cr, bm, counts = 3, 0, 8, 4, 8, [8, 8, 3]
    order = [4, 2, 3, 5]              # slot 2's empty chunk 5 comes last: it must not delay tile 2
    cps = cap // cr
    pos = {c: i for i, c in enumerate(order)}
    ready = {}
    for t in range(world * cap // bm):
        lo, hi = t * bm, (t + 1) * bm
        if any((x % cap) < counts[x // cap] for x in range(lo, hi)):
            need = [pos[c] for c in O.covering_chunks(lo, hi, cr) if c // cps != rank]
            ready[t] = max(need) if need else -1
    wrong = sorted(ready, key=lambda t: (ready[t], t))
    assert wrong != _simulate_a2a(world, rank, cap, cr, counts, order, bm)

