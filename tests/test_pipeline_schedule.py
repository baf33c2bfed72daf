"""The operand pipelines' barrier counts (csrc/pipeline.h, the constants the GEMM kernel uses)
against an independent replay of each issue order: at every slice's barrier, the data the next
reads need must have landed given the count (loads complete in issue order), and no load may
refill an LDS slot before the last read of its old contents. A count that is too large is a race
that GPU runs would only show now and then; this pins it on the CPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "allgather_gemm_persistent_amd", "csrc", "pipeline.h")

# (NI) of the four-stage tiles; (R, NL) of the pair tiles; (NLA, NIB, NHB) of the mixed tiles, as
# the kernel instantiates them (4 waves): 64x64 / 128x64 / 128x128 -> R 4, NL 4 / 6 / 8, NLP NL/2;
# 256x224 / 256x256, bf16 and fp8 -> NLA 8, NIB 4, NHB 0, NLAP 4 (a tile below 64x64 would take the
# four stages; the other values exercise the same arithmetic)
STAGE = [(2, 1), (2, 0), (3, 1), (4, 2), (4, 0), (8, 4)]                     # (NI, NH)
PAIRS = [(2, 16, 8), (4, 4, 2), (4, 4, 0), (4, 6, 3), (4, 6, 0), (4, 8, 4), (4, 8, 0), (2, 8, 4)]   # (R, NL, NLP)
MIXED = [(8, 4, 0, 4), (8, 4, 0, 0), (8, 4, 1, 4), (8, 4, 2, 4), (8, 4, 0, 2)]   # (NLA, NIB, NHB, NLAP)


@pytest.fixture(scope="module")
def counts(tmp_path_factory):
    """Compile a host program against pipeline.h and read the counts it prints."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("pipeline")
    src = d / "counts.cpp"
    lines = ['#include <cstdio>', f'#include "{HEADER}"', "int main() {", "  using namespace agg;"]
    for ni, nh in STAGE:
        lines.append(f'  std::printf("stage {ni} {nh} %d %d\\n", stage_barrier_count({ni}), '
                     f'stage_prologue_count({ni}, {nh}));')
    for r, nl, nlp in PAIRS:
        lines.append(f'  std::printf("pair {r} {nl} {nlp} %d %d %d\\n", pair_barrier_count(0, {r}, {nl}), '
                     f'pair_barrier_count(1, {r}, {nl}), pair_prologue_count({r}, {nl}, {nlp}));')
    for nla, nib, nhb, nlap in MIXED:
        lines.append(f'  std::printf("mixed {nla} {nib} {nhb} {nlap} %d %d %d %d %d\\n", '
                     + ", ".join(f"mixed_barrier_count({u}, {nla}, {nib}, {nhb}, {nlap})" for u in range(4))
                     + f", mixed_prologue_count({nla}, {nib}, {nhb}, {nlap}));")
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = d / "counts"
    subprocess.run([cxx, "-std=c++17", "-O1", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    table = {}
    for line in out.splitlines():
        f = line.split()
        if f[0] == "stage":
            table[("stage", int(f[1]), int(f[2]))] = (int(f[3]), int(f[4]))
        elif f[0] == "pair":
            table[("pair", int(f[1]), int(f[2]), int(f[3]))] = tuple(int(x) for x in f[4:])
        else:
            table[("mixed", int(f[1]), int(f[2]), int(f[3]), int(f[4]))] = tuple(int(x) for x in f[5:])
    return table


class Replay:
    """Loads of one wave in issue order, completing in that order; a barrier with count c means
    every load but the last c issued has completed."""

    def __init__(self):
        self.issued = []      # (slot, item) per load
        self.done = 0
        self.errors = []

    def issue(self, item, n):
        self.issued.extend([item] * n)

    def barrier(self, count):
        self.done = max(self.done, len(self.issued) - count)

    def landed(self, item, n):
        idx = [k for k, x in enumerate(self.issued) if x == item]
        return len(idx) == n and max(idx) < self.done


def replay_stages(ni, nh, bar, pro, slices=64):
    r = Replay()
    for q in range(3):
        r.issue(("B", q), ni)
    r.issue(("B", 3), nh)
    r.barrier(pro)
    need = lambda s: r.landed(("B", s), ni)
    if not need(0):
        r.errors.append("prologue")
    for t in range(slices):
        # before the barrier: the rest of slice t+3 into the slot slice t-1 left (read before
        # the barrier of slice t-1)
        r.issue(("B", t + 3), ni - nh)
        r.barrier(bar)
        if not need(t + 1):
            r.errors.append(("slice", t + 1))
        # after the barrier: the first loads of slice t+4 into slice t's slot (read before it)
        r.issue(("B", t + 4), nh)
    return r.errors


def replay_pairs(R, nl, nlp, bar_even, bar_odd, pro, slices=96):
    r = Replay()
    for q in range(R - 1):
        r.issue(("P", q), nl)
    r.issue(("P", R - 1), nlp)
    r.barrier(pro)
    if not r.landed(("P", 0), nl):
        r.errors.append("prologue")
    for t in range(slices):
        if t % 2 == 0:
            # into the region pair t/2-1 left: its last read was before the barrier of slice t-1
            r.issue(("P", t // 2 + R - 1), nl - nlp)
        r.barrier(bar_odd if t % 2 else bar_even)
        if not r.landed(("P", (t + 1) // 2), nl):
            r.errors.append(("pair", (t + 1) // 2, t))
        if t % 2 == 1:
            # into slice t's own region: every wave has read pair (t-1)/2 before this barrier
            r.issue(("P", (t + 1) // 2 + R - 1), nlp)
    return r.errors


def replay_mixed(nla, nib, nhb, nlap, bars, pro, slices=96):
    r = Replay()
    r.issue(("A", 0), nla)
    r.issue(("A", 1), nlap)
    for q in range(3):
        r.issue(("B", q), nib)
    r.issue(("B", 3), nhb)
    r.barrier(pro)
    if not (r.landed(("A", 0), nla) and r.landed(("B", 0), nib)):
        r.errors.append("prologue")
    for t in range(slices):
        if t % 2 == 0:
            r.issue(("A", t // 2 + 1), nla - nlap)
        r.issue(("B", t + 3), nib - nhb)
        r.barrier(bars[t % 4])
        if not r.landed(("A", (t + 1) // 2), nla):
            r.errors.append(("A", (t + 1) // 2, t))
        if not r.landed(("B", t + 1), nib):
            r.errors.append(("B", t + 1, t))
        if t % 2 == 1:
            r.issue(("A", (t + 1) // 2 + 1), nlap)
        r.issue(("B", t + 4), nhb)
    return r.errors


@pytest.mark.parametrize("ni,nh", STAGE)
def test_stage_counts(counts, ni, nh):
    bar, pro = counts[("stage", ni, nh)]
    assert replay_stages(ni, nh, bar, pro) == []
    # one more load in flight would be a race
    assert replay_stages(ni, nh, bar + 1, pro) != [] or replay_stages(ni, nh, bar, pro + 1) != []


@pytest.mark.parametrize("R,nl,nlp", PAIRS)
def test_pair_counts(counts, R, nl, nlp):
    even, odd, pro = counts[("pair", R, nl, nlp)]
    assert replay_pairs(R, nl, nlp, even, odd, pro) == []
    # the odd barriers and the prologue's wait for the last loads they may: one more in flight
    # would be a race (an even barrier needs the pair its odd predecessor already waited for)
    assert replay_pairs(R, nl, nlp, even, odd + 1, pro) != []
    assert replay_pairs(R, nl, nlp, even, odd, pro + 1) != []


@pytest.mark.parametrize("nla,nib,nhb,nlap", MIXED)
def test_mixed_counts(counts, nla, nib, nhb, nlap):
    *bars, pro = counts[("mixed", nla, nib, nhb, nlap)]
    assert replay_mixed(nla, nib, nhb, nlap, bars, pro) == []
    for u in range(4):
        worse = list(bars)
        worse[u] += 1
        assert replay_mixed(nla, nib, nhb, nlap, worse, pro) != [], u
    assert replay_mixed(nla, nib, nhb, nlap, bars, pro + 1) != []


def test_refills_follow_last_reads():
    """A refill writes an LDS slot only after every wave has passed the barrier that follows the
    last read of the slot's old contents. Pair region of pair p+R: its old pair p is last read in
    the first half of slice 2p+1, so the refill may come after the barrier of slice 2p+1 (odd
    slices issue after their barrier; even ones before theirs, i.e. after the previous slice's).
    B stage of slice s+4: slice s is last read before the barrier of slice s."""
    for R in (2, 4):
        for t in range(200):
            if t % 2 == 0:
                old = t // 2 + R - 1 - R
                assert old < 0 or 2 * old + 1 <= t - 1
            else:
                old = (t + 1) // 2 + R - 1 - R
                assert old < 0 or 2 * old + 1 <= t
    for t in range(200):
        assert (t + 3) - 4 <= t - 1      # before the barrier of slice t: slice t-1's stage
        assert (t + 4) - 4 <= t          # after it: slice t's stage
