// Barrier counts of the GEMM kernel's operand pipelines: how many of a wave's direct-to-LDS loads
// may still be in flight at the barrier of each slice (the s_waitcnt vmcnt of the barrier), so
// that every load of the data the next slice reads has landed. Plain constexpr arithmetic, used by
// the kernel for its template arguments and by a host-side test that replays each issue order.
#pragma once

namespace agg {

// Four 64-byte stages, NI loads per wave per slice: slice t issues, before its barrier, loads
// NI/2.. of slice t+3 and, after it, loads 0..NI/2-1 of slice t+4; the prologue issues slices 0..2
// and the first half of slice 3.
constexpr int stage_barrier_count(int NI) { return 2 * NI; }
constexpr int stage_prologue_count(int NI) { return 2 * NI + NI / 2; }

// R regions of 128-byte slice pairs, NL loads per wave per pair: an even slice t issues, before
// its barrier, the second half of pair t/2+R-1; an odd slice t, after its barrier, the first half
// of pair (t+1)/2+R-1; the prologue issues pairs 0..R-2 and the first half of pair R-1. An odd
// slice's barrier needs pair (t+1)/2 whole; an even slice's, pair t/2.
constexpr int pair_barrier_count(int u, int R, int NL) { return (u & 1) ? (R - 2) * NL : (R - 1) * NL; }
constexpr int pair_prologue_count(int R, int NL) { return (R - 2) * NL + NL / 2; }

// Mixed (big bf16 tiles): A rows in two regions of slice pairs (NLA loads per pair), B rows in four
// 64-byte stages (NIB loads per slice, NHB of them after the barrier). Issue order per wave: the
// prologue's A pair 0, first half of A pair 1, B slices 0..2, first NHB loads of B slice 3; then
// slice s issues before its barrier the second half of A pair s/2+1 (even s) and the last NIB-NHB
// loads of B slice s+3, and after it the first half of A pair (s+1)/2+1 (odd s) and the first NHB
// loads of B slice s+4. Returns how many loads follow the later of the last load of A pair
// (t+1)/2 and of B slice t+1 at the barrier of slice t (t = -1: the prologue's barrier).
constexpr int mixed_loads_after(int t, int NLA, int NIB, int NHB) {
  const int pa_need = t < 0 ? 0 : (t + 1) / 2;
  const int sb_need = t + 1;
  int n = NLA, last = pa_need == 0 ? n : 0;     // A pair 0
  n += NLA / 2;                                 // first half of A pair 1
  for (int q = 0; q < 3; ++q) {                 // B slices 0..2
    n += NIB;
    if (sb_need == q && n > last) last = n;
  }
  n += NHB;                                     // first loads of B slice 3
  for (int s = 0; s <= t; ++s) {
    if (s % 2 == 0) {
      n += NLA - NLA / 2;
      if (pa_need == s / 2 + 1 && n > last) last = n;
    }
    n += NIB - NHB;
    if (sb_need == s + 3 && n > last) last = n;
    if (s < t) {
      if (s % 2 == 1) n += NLA / 2;
      n += NHB;
    }
  }
  return n - last;
}

// The barrier count of trip slice u (four slices per trip): the fewest loads that follow the needed
// ones at that slice over the first trips (the prologue's order differs from the steady state's).
constexpr int mixed_barrier_count(int u, int NLA, int NIB, int NHB) {
  int m = mixed_loads_after(u, NLA, NIB, NHB);
  for (int k = 1; k < 4; ++k) {
    const int v = mixed_loads_after(u + 4 * k, NLA, NIB, NHB);
    m = v < m ? v : m;
  }
  return m;
}

constexpr int mixed_prologue_count(int NLA, int NIB, int NHB) { return mixed_loads_after(-1, NLA, NIB, NHB); }

}  // namespace agg
