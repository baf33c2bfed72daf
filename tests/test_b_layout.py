"""The K x N weight operand's path through LDS (csrc/pipeline.h, the functions the GEMM kernel
uses): direct-to-LDS loads fill each slice's B block, and transposing LDS reads turn its
N-contiguous rows into the K-packed MFMA fragments.

Replayed on the CPU for every block width the kernels are instantiated with (64, 128 and 256
columns, bf16 and fp8):
  * the loads cover every (K row, 16-byte column chunk) of the block exactly once;
  * the per-lane read addresses the kernel forms (base + step * r + 16 * (c0 ^ swizzle)) equal the
    layout's own offsets, and, put through the lane permutation of ds_read_b64_tr_b16 / _b8 as
    measured on the GPU, deliver to every lane exactly the (K row, column) elements the 16x16x32
    bf16 or 32x32x64 fp8 MFMA operand layout asks of it;
  * each half wave of 32 lanes reads 32 distinct 8-byte slots of the 64 four-byte banks.
A planted mistake (the swizzle left out, an untransposed read) must fail the replay.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "allgather_gemm_persistent_amd", "csrc", "pipeline.h")
CASES = [(bnp, el) for el in (2, 1) for bnp in (64, 128, 256)]


@pytest.fixture(scope="module")
def tables(tmp_path_factory):
    """Compile a host program against pipeline.h and read its load and read tables."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("blayout")
    src = d / "tab.cpp"
    src.write_text(f'''#include <cstdio>
#include "{HEADER}"
using namespace agg;
int main() {{
  const int cases[6][2] = {{{{64, 2}}, {{128, 2}}, {{256, 2}}, {{64, 1}}, {{128, 1}}, {{256, 1}}}};
  for (auto& c : cases) {{
    const int bnp = c[0], el = c[1], P = bnp * el / 16;
    for (int q = 0; q < 4 * bnp; ++q) std::printf("L %d %d %d %d %d\\n", bnp, el, q, b_load_row(q, P), b_load_chunk(q, P, el));
    const int reads = el == 2 ? 2 : 4;
    for (int c0 = 0; c0 < P; c0 += 2)
      for (int r = 0; r < reads; ++r)
        for (int lane = 0; lane < 64; ++lane)
          std::printf("R %d %d %d %d %d %d %d\\n", bnp, el, c0, r, lane, b_read_offset(lane, r, c0, P, el),
                      b_read_base(lane, P, el) + r * b_read_step(P, el) + 16 * (c0 ^ b_read_swizzle(lane, P, el)));
  }}
  return 0;
}}
''')
    exe = d / "tab"
    subprocess.run([cxx, "-std=c++17", "-O1", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    loads, reads = {}, {}
    for line in out.splitlines():
        f = line.split()
        v = [int(x) for x in f[1:]]
        if f[0] == "L":
            loads.setdefault((v[0], v[1]), {})[v[2]] = (v[3], v[4])
        else:
            reads.setdefault((v[0], v[1]), {})[(v[2], v[3], v[4])] = (v[5], v[6])
    return loads, reads


def tr_source(lane, e, el, transposed=False):
    """(source lane, element) of element e of `lane` after a transposing read, as measured;
    transposed=True plants the mistake of a plain (untransposed) read."""
    if transposed:
        return lane, e
    g = 16 * (lane // 16)
    if el == 2:
        return g + (lane % 16) // 4 + 4 * e, lane % 4
    return g + (lane % 16) // 8 + 2 * e, lane % 8


def replay(loads, reads, bnp, el, transposed=False, drop_swizzle=False):
    """Returns a list of problems (empty when the layout is right)."""
    P, rows = bnp * el // 16, 64 // el
    per = 16 // el                          # elements per 16-byte chunk
    problems = []
    lds = {}
    for q, (k, c) in loads.items():
        lds[q] = (k, c)
    if sorted(lds.values()) != [(k, c) for k in range(rows) for c in range(P)]:
        problems.append("loads do not cover every (row, chunk) once")
    n_reads = 2 if el == 2 else 4
    for c0 in range(0, P, 2):
        for r in range(n_reads):
            addr = {}
            for lane in range(64):
                off, formed = reads[(c0, r, lane)]
                if drop_swizzle:
                    k = (8 * (lane >> 4) + 4 * r + ((lane & 15) >> 2)) if el == 2 else \
                        (32 * (lane >> 5) + 8 * r + ((lane & 15) >> 1))
                    ch = ((lane & 3) >> 1) if el == 2 else ((lane >> 4) & 1)
                    off = formed = 16 * (k * P + c0 + ch) + 8 * (lane & 1)
                if off != formed:
                    problems.append(f"read offset formed differently at c0={c0} r={r} lane={lane}")
                addr[lane] = off
            # what each lane's 8 bytes hold: (row, column) per element
            held = {}
            for lane, a in addr.items():
                k, c = lds[a // 16]
                first = c * per + (a % 16) // el
                held[lane] = [(k, first + e) for e in range(8 // el)]
            for lane in range(64):
                for e in range(8 // el):
                    s, se = tr_source(lane, e, el, transposed)
                    got = held[s][se]
                    if el == 2:
                        want = (8 * (lane // 16) + 4 * r + e, c0 * per + lane % 16)
                    else:
                        want = (32 * (lane // 32) + 8 * r + e, c0 * per + lane % 32)
                    if got != want:
                        problems.append(f"c0={c0} r={r} lane={lane} e={e}: got {got} want {want}")
            for half in (range(32), range(32, 64)):
                slots = {(addr[l] % 256) // 8 for l in half}
                if len(slots) != 32:
                    problems.append(f"bank conflict at c0={c0} r={r} ({len(slots)} slots)")
    return problems


@pytest.mark.parametrize("bnp,el", CASES)
def test_b_layout_delivers_mfma_fragments(tables, bnp, el):
    loads, reads = tables
    problems = replay(loads[(bnp, el)], reads[(bnp, el)], bnp, el)
    assert not problems, problems[:5]


@pytest.mark.parametrize("bnp,el", [(256, 2), (128, 1)])
def test_b_layout_replay_catches_planted_mistakes(tables, bnp, el):
    loads, reads = tables
    assert replay(loads[(bnp, el)], reads[(bnp, el)], bnp, el, transposed=True)
    assert any("bank conflict" in p for p in
               replay(loads[(bnp, el)], reads[(bnp, el)], bnp, el, drop_swizzle=True))
