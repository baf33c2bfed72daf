// Barrier counts of the GEMM kernel's operand pipelines: how many of a wave's direct-to-LDS loads
// may still be in flight at the barrier of each slice (the s_waitcnt vmcnt of the barrier), so
// that every load of the data the next slice reads has landed. Plain constexpr arithmetic, used by
// the kernel for its template arguments and by a host-side test that replays each issue order.
#pragma once

namespace agg {

// Bytes of LDS that direct-to-LDS loads may fill: their LDS address (M0) is taken to wrap at
// 128 KiB on gfx950 (layouts that reached past it gave wrong results), so every operand stage of
// the GEMM kernel lies below this bound.
constexpr int kLdsDmaLimit = 128 * 1024;

// Four 64-byte stages, NI loads per wave per slice: slice t issues, before its barrier, loads
// NH.. of slice t+3 and, after it, loads 0..NH-1 of slice t+4; the prologue issues slices 0..2 and
// the first NH loads of slice 3. At a slice's barrier 2*NI loads follow the last one of slice t+1,
// whatever NH is.
constexpr int stage_barrier_count(int NI) { return 2 * NI; }
constexpr int stage_prologue_count(int NI, int NH) { return 2 * NI + NH; }

// R regions of 128-byte slice pairs, NL loads per wave per pair: an even slice t issues, before
// its barrier, loads NLP.. of pair t/2+R-1; an odd slice t, after its barrier, loads 0..NLP-1 of
// pair (t+1)/2+R-1; the prologue issues pairs 0..R-2 and the first NLP loads of pair R-1. An odd
// slice's barrier needs pair (t+1)/2 whole; an even slice's, pair t/2 (counts independent of NLP).
constexpr int pair_barrier_count(int u, int R, int NL) { return (u & 1) ? (R - 2) * NL : (R - 1) * NL; }
constexpr int pair_prologue_count(int R, int NL, int NLP) { return (R - 2) * NL + NLP; }

// Mixed (the big tiles, bf16 and fp8): A rows in two regions of slice pairs (NLA loads per pair),
// B rows in four 64-byte stages (NIB loads per slice). Issue order per wave: the prologue's A pair
// 0, the first NLAP loads of A pair 1, B slices 0..2, the first NHB loads of B slice 3; then slice
// s issues before its barrier the other NLA-NLAP loads of A pair s/2+1 (even s) and the last
// NIB-NHB loads of B slice s+3, and after it the first NLAP loads of A pair (s+1)/2+1 (odd s) and
// the first NHB loads of B slice s+4. Returns how many loads follow the later of the last load of
// A pair (t+1)/2 and of B slice t+1 at the barrier of slice t (t = -1: the prologue's barrier).
constexpr int mixed_loads_after(int t, int NLA, int NIB, int NHB, int NLAP) {
  const int pa_need = t < 0 ? 0 : (t + 1) / 2;
  const int sb_need = t + 1;
  int n = NLA, last = pa_need == 0 ? n : 0;     // A pair 0
  n += NLAP;                                    // first loads of A pair 1
  for (int q = 0; q < 3; ++q) {                 // B slices 0..2
    n += NIB;
    if (sb_need == q && n > last) last = n;
  }
  n += NHB;                                     // first loads of B slice 3
  for (int s = 0; s <= t; ++s) {
    if (s % 2 == 0) {
      n += NLA - NLAP;
      if (pa_need == s / 2 + 1 && n > last) last = n;
    }
    n += NIB - NHB;
    if (sb_need == s + 3 && n > last) last = n;
    if (s < t) {
      if (s % 2 == 1) n += NLAP;
      n += NHB;
    }
  }
  return n - last;
}

// The barrier count of trip slice u (four slices per trip): the fewest loads that follow the needed
// ones at that slice over the first trips (the prologue's order differs from the steady state's).
constexpr int mixed_barrier_count(int u, int NLA, int NIB, int NHB, int NLAP) {
  int m = mixed_loads_after(u, NLA, NIB, NHB, NLAP);
  for (int k = 1; k < 4; ++k) {
    const int v = mixed_loads_after(u + 4 * k, NLA, NIB, NHB, NLAP);
    m = v < m ? v : m;
  }
  return m;
}

constexpr int mixed_prologue_count(int NLA, int NIB, int NHB, int NLAP) {
  return mixed_loads_after(-1, NLA, NIB, NHB, NLAP);
}

}  // namespace agg

namespace agg {

// ---- the B operand (K x N, N contiguous) in LDS
//
// One 64-byte K slice of a tile's B columns is a block of 64/elem K rows, each BNP*elem bytes (BNP
// = the tile's columns rounded up to 64), i.e. P = BNP*elem/16 chunks of 16 bytes per row and
// 4*BNP chunks in all. Chunk c of row k sits at chunk position k*P + (c ^ b_swizzle(k, P, elem)),
// so direct-to-LDS load lanes that fill consecutive positions fetch whole row segments (every
// request a full line for rows of 128 bytes and more).
//
// The MFMA operand needs K-packed fragments (a lane holds consecutive K of one column); gfx950's
// transposing LDS reads build them from N-contiguous rows. Within each 16-lane group g of the
// wave, ds_read_b64_tr_b16 gives lane l element e = element l%4 of the 8 bytes read by lane
// 16g + (l%16)/4 + 4e, and ds_read_b64_tr_b8 gives lane l byte e = byte l%8 of the 8 bytes read by
// lane 16g + (l%16)/8 + 2e (both measured on the GPU with every lane reading a distinct address).
// So for the bf16 16x16x32 fragment (lane l: column l%16, K 8*(l/16) .. +7), read r of two has lane
// s fetch K row 8*(s/16) + 4r + (s%16)/4, columns 4*(s%4) .. +3; for the fp8 32x32x64 fragment
// (lane l: column l%32, K 32*(l/32) .. +31), read r of four has lane s fetch K row
// 32*(s/32) + 8r + (s%16)/2, columns 16*((s/16)%2) + 8*(s%2) .. +7. A half wave then reads 8 rows
// x 32 bytes; the swizzle puts those rows on distinct 32-byte bank groups of the 256-byte bank
// line (64 banks of 4 bytes).
constexpr int b_swizzle(int k, int P, int elem) {
  if (elem == 2) {      // half wave: rows 4r + a and 8 + 4r + a, a = 0..3
    if (P >= 16) return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
    return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));    // P == 8: two rows per bank line
  }
  // fp8, half wave: rows 8r .. 8r + 7
  if (P >= 16) return 2 * (k & 7);
  if (P == 8) return 2 * ((k >> 1) & 3);
  return 2 * ((k >> 2) & 1);                               // P == 4: four rows per bank line
}

// The B load that fills chunk position q of a slice's block: its K row and its column chunk.
constexpr int b_load_row(int q, int P) { return q / P; }
constexpr int b_load_chunk(int q, int P, int elem) { return (q % P) ^ b_swizzle(q / P, P, elem); }

// Transposing reads of a B fragment: lane `lane`'s K row for read r (0..1 bf16, 0..3 fp8), the
// chunk it reads relative to the fragment's first chunk (0 or 1), the 8-byte half, and the
// swizzle of its rows (the same for every r).
constexpr int b_read_row(int lane, int r, int elem) {
  return elem == 2 ? 8 * (lane >> 4) + 4 * r + ((lane & 15) >> 2)
                   : 32 * (lane >> 5) + 8 * r + ((lane & 15) >> 1);
}
constexpr int b_read_chunk(int lane, int elem) { return elem == 2 ? (lane & 3) >> 1 : (lane >> 4) & 1; }
constexpr int b_read_half(int lane, int elem) { return elem == 2 ? lane & 1 : lane & 1; }
constexpr int b_read_swizzle(int lane, int P, int elem) { return b_swizzle(b_read_row(lane, 0, elem), P, elem); }
// What the kernel computes once per lane: the offset of read 0 for a fragment at chunk 0 before
// the swizzle, and the step from read r to read r + 1 (4 rows bf16, 8 rows fp8). For an even c0
// the offset of read r is b_read_base + r * b_read_step + 16 * (c0 ^ b_read_swizzle).
constexpr int b_read_base(int lane, int P, int elem) {
  return 16 * (b_read_row(lane, 0, elem) * P + b_read_chunk(lane, elem)) + 8 * b_read_half(lane, elem);
}
constexpr int b_read_step(int P, int elem) { return 16 * (elem == 2 ? 4 : 8) * P; }
// LDS byte offset, inside the slice's B block, of read r of lane `lane` for the fragment whose
// columns start at chunk `c0` (even)
constexpr int b_read_offset(int lane, int r, int c0, int P, int elem) {
  return 16 * (b_read_row(lane, r, elem) * P + ((c0 + b_read_chunk(lane, elem)) ^ b_read_swizzle(lane, P, elem))) +
         8 * b_read_half(lane, elem);
}

}  // namespace agg
