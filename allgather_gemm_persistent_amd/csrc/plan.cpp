// Host-side planning: argument checks, tile shape choice and row-tile orders.
//
// The row-tile order is the chunk/tile pairing of the page "Triton-distributed is turning
// communication into compiler territory", section "DITRON adds three levels of tiling"
// (collectives broken into chunks that are paired with computation tiles), applied to the
// overlap of section "The first move was to expose the overlap": tiles whose rows are all local
// go first, then each tile as soon as the latest chunk it overlaps has arrived.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <numeric>

#include "../../include/agg.h"

namespace agg {

namespace {
thread_local std::string g_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

const std::vector<TileShape>& tile_shapes() {
  static const std::vector<TileShape> shapes = {
      {256, 256}, {256, 224}, {128, 128}, {128, 64}, {64, 64}};
  return shapes;
}

int choose_list_cols(int lists, int n_row_tiles, int n_col_tiles, int bm, int bn, int workers) {
  int best = 1;
  int64_t best_rows = -1;
  workers = std::max(workers, 1);
  for (int lc = 1; lc <= lists; lc *= 2) {
    if (lists % lc) continue;
    const int lr = lists / lc;
    if (lc > n_col_tiles || lr > std::max(n_row_tiles, 1)) continue;
    const int64_t nx = (n_col_tiles + lc - 1) / lc;            // column tiles per list
    const int64_t ny = (n_row_tiles + lr - 1) / lr;            // row tiles per list
    const int64_t cols = std::min<int64_t>(nx, workers);
    const int64_t rows = std::min<int64_t>((workers + nx - 1) / nx, ny);
    const int64_t touched = rows * bm + cols * bn;
    if (best_rows < 0 || touched < best_rows) {
      best_rows = touched;
      best = lc;
    }
  }
  return best;
}

int slice_bytes(int) { return 64; }

KSplit choose_ksplit(int op, int dtype, int64_t tiles, int64_t k, int units) {
  KSplit r{1, 0};
  const int64_t kbytes = k * (dtype == AGG_FP8_E4M3 ? 1 : 2);
  const int64_t nk = (kbytes + slice_bytes(dtype) - 1) / slice_bytes(dtype);
  r.kps = int(std::max<int64_t>(nk, 1));
  // split only an AllGather+GEMM whose tiles leave more than half the units idle, and only so
  // far that every part keeps at least 16 slices
  if (op != 0 || tiles <= 0 || tiles * 2 > units || tiles > kMaxSplitTiles) return r;
  int64_t s = std::min<int64_t>({int64_t(units) / tiles, nk / 16, int64_t(kAutoKSplit)});
  if (s < 2) return r;
  int64_t kps = (nk + s - 1) / s;
  kps += kps & 1;                         // parts start on whole slice pairs
  r.kps = int(kps);
  r.ksplit = int((nk + kps - 1) / kps);   // no empty part
  return r;
}

// Relative MFMA efficiency of each shape (operand bytes per flop fall as the tile grows; the
// 128 x 128 weight from bare launches of the 5120-row AllToAll workload, where its 4.4 waves
// ran 14% slower than two waves of 256 x 256 tiles).
static double tile_eff(const TileShape& s) {
  if (s.bm == 256 && s.bn == 256) return 1.0;
  if (s.bm == 256) return 0.98;
  if (s.bm == 128 && s.bn == 128) return 0.6;
  if (s.bm == 128) return 0.5;
  return 0.35;
}

static_assert(kTailAuto == AGG_TAIL_AUTO && kTailOff == AGG_TAIL_OFF && kTailOn == AGG_TAIL_ON, "tail modes");

TailSplit tail_split(TileShape ts, int64_t m, int64_t n, int n_rows, int units, int mode) {
  TailSplit r{0, {0, 0}};
  if (mode == kTailOff || n_rows < 2 || n <= 0 || m <= 0 || units < 1) return r;
  // the next smaller shape whose rows divide the big tile's
  TileShape t2{0, 0};
  if (ts.bm == 256) t2 = {128, 128};
  else if (ts.bm == 128 && ts.bn == 128) t2 = {128, 64};
  else if (ts.bm == 128 && ts.bn == 64) t2 = {64, 64};
  if (t2.bm == 0) return r;
  const int64_t nct = (n + ts.bn - 1) / ts.bn;
  const int64_t tiles = int64_t(n_rows) * nct;
  // the head: whole row tiles that fill whole waves
  int64_t head = (tiles / units) * units / nct;
  if (mode == kTailOn) head = std::min<int64_t>(std::max<int64_t>(head, 1), n_rows - 1);
  if (head < 1 || head >= n_rows) return r;
  // the tail's rows at the smaller shape (every sub-tile of a tail row tile, clipped at m)
  const int64_t sub = ts.bm / t2.bm;
  const int64_t tail_rows = std::min<int64_t>((n_rows - head) * sub, (m + t2.bm - 1) / t2.bm);
  const int64_t tiles2 = tail_rows * ((n + t2.bn - 1) / t2.bn);
  if (mode == kTailAuto) {
    // in waves of big tiles: the split pays when its second launch (plus ~5% for the launch
    // itself) takes less than the big tiles' last wave
    const double ratio = (double(t2.bm) * t2.bn / tile_eff(t2)) / (double(ts.bm) * ts.bn / tile_eff(ts));
    const double unsplit = double((tiles + units - 1) / units);
    const double split = double((head * nct + units - 1) / units) + double((tiles2 + units - 1) / units) * ratio + 0.05;
    if (split >= unsplit) return r;
  }
  r.head_rows = int(head);
  r.tail = t2;
  return r;
}

TileShape choose_tile(int op, int dtype, int64_t m, int64_t n, int64_t k) {
  auto eff = tile_eff;
  const int64_t kUnits = 256;  // compute units of one MI355X, one workgroup each
  TileShape best = tile_shapes().back();
  double best_cost = 1e300;
  int64_t best_tiles = 0;
  for (const TileShape& s : tile_shapes()) {
    int64_t tiles = ((m + s.bm - 1) / s.bm) * ((n + s.bn - 1) / s.bn);
    // a split-K call spreads each tile's K over ksplit workgroups (plus a reduction)
    const KSplit ks = s.bm * s.bn <= kMaxSplitTileArea ? choose_ksplit(op, dtype, tiles, k, int(kUnits))
                                                       : KSplit{1, 0};
    int64_t items = tiles * ks.ksplit;
    int64_t waves = std::max<int64_t>(1, (items + kUnits - 1) / kUnits);
    double cost = double(waves) * s.bm * s.bn / eff(s) / ks.ksplit * (ks.ksplit > 1 ? 1.1 : 1.0);
    if (cost < best_cost * (1 - 1e-9) || (std::fabs(cost - best_cost) <= 1e-9 * cost && tiles > best_tiles)) {
      best = s;
      best_cost = cost;
      best_tiles = tiles;
    }
  }
  return best;
}

std::vector<int32_t> ring_order(int world, int rank, int chunks_per_shard) {
  std::vector<int32_t> out;
  out.reserve(size_t(world - 1) * chunks_per_shard);
  for (int d = 1; d < world; ++d) {
    int p = (rank + d) % world;
    for (int j = 0; j < chunks_per_shard; ++j) out.push_back(p * chunks_per_shard + j);
  }
  return out;
}

int check_order(int world, int rank, int chunks_per_shard, const int32_t* order, int n_order) {
  const int64_t expect = int64_t(world - 1) * chunks_per_shard;
  if (n_order != expect)
    return fail(AGG_E_ARG, "order has %d entries, expected %lld remote chunks", n_order,
                (long long)expect);
  std::vector<char> seen(size_t(world) * chunks_per_shard, 0);
  for (int i = 0; i < n_order; ++i) {
    int32_t c = order[i];
    if (c < 0 || c >= world * chunks_per_shard)
      return fail(AGG_E_ARG, "order[%d] = %d is not a chunk id", i, c);
    if (c / chunks_per_shard == rank)
      return fail(AGG_E_ARG, "order[%d] = %d is a local chunk", i, c);
    if (seen[c]) return fail(AGG_E_ARG, "order[%d] = %d repeats a chunk", i, c);
    seen[c] = 1;
  }
  return AGG_OK;
}

std::vector<int32_t> ag_row_tile_order(int world, int rank, int64_t m_shard, int chunk_rows,
                                       const std::vector<int32_t>& order, int bm, const int32_t* counts) {
  const int64_t m = int64_t(world) * m_shard;
  const int64_t cps = m_shard / chunk_rows;
  const int64_t n_chunks = int64_t(world) * cps;
  std::vector<int64_t> pos(size_t(n_chunks), -1);
  for (size_t i = 0; i < order.size(); ++i) pos[size_t(order[i])] = int64_t(i);
  // with counts: chunk c holds rows when its first row lies below its slot's count
  auto holds = [&](int64_t c) { return !counts || (c % cps) * chunk_rows < counts[c / cps]; };
  // with counts: rows [lo, hi) hold a row when some slot they meet has rows there
  auto has_rows = [&](int64_t lo, int64_t hi) {
    if (!counts) return true;
    for (int64_t p = lo / m_shard; p <= (hi - 1) / m_shard; ++p)
      if (std::max(lo, p * m_shard) < p * m_shard + counts[p]) return true;
    return false;
  };
  const int64_t tiles = (m + bm - 1) / bm;
  std::vector<int64_t> ready(size_t(tiles), -1);
  std::vector<int32_t> idx;
  idx.reserve(size_t(tiles));
  for (int64_t t = 0; t < tiles; ++t) {
    int64_t lo = t * bm, hi = std::min(m, lo + bm);
    if (!has_rows(lo, hi)) continue;
    idx.push_back(int32_t(t));
    for (int64_t c = lo / chunk_rows; c <= (hi - 1) / chunk_rows; ++c)
      if (c / cps != rank && holds(c)) ready[size_t(t)] = std::max(ready[size_t(t)], pos[size_t(c)]);
  }
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return ready[size_t(a)] < ready[size_t(b)]; });
  return idx;
}

std::vector<int32_t> rs_row_tile_order(int world, int rank, int64_t m, int chunk_rows,
                                       const std::vector<int32_t>& order, int bm) {
  const int64_t mb = m / world;
  const int64_t cpb = mb / chunk_rows;
  const int64_t tpb = (mb + bm - 1) / bm;
  std::vector<int32_t> seq;
  seq.reserve(size_t(world * tpb));
  for (int d = 1; d < world; ++d) {
    int j = (rank + d) % world;
    for (int64_t i = 0; i < tpb; ++i) seq.push_back(int32_t(j * tpb + i));
  }
  std::vector<int64_t> pos(size_t(world * cpb), -1);
  for (size_t i = 0; i < order.size(); ++i) pos[size_t(order[i])] = int64_t(i);
  std::vector<int64_t> ready(size_t(tpb), -1);
  for (int64_t i = 0; i < tpb; ++i) {
    int64_t lo = i * bm, hi = std::min(mb, lo + bm);
    for (int p = 0; p < world; ++p) {
      if (p == rank) continue;
      for (int64_t q = lo / chunk_rows; q <= (hi - 1) / chunk_rows; ++q)
        ready[size_t(i)] = std::max(ready[size_t(i)], pos[size_t(p * cpb + q)]);
    }
  }
  std::vector<int32_t> local(static_cast<size_t>(tpb));
  std::iota(local.begin(), local.end(), 0);
  std::stable_sort(local.begin(), local.end(),
                   [&](int32_t a, int32_t b) { return ready[size_t(a)] < ready[size_t(b)]; });
  for (int32_t i : local) seq.push_back(int32_t(rank * tpb + i));
  return seq;
}

}  // namespace agg

// ------------------------------------------------------------------------------------------
// C entry points that need no device
// ------------------------------------------------------------------------------------------

using namespace agg;

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int elem_bytes(int dtype) { return dtype == AGG_FP8_E4M3 ? 1 : 2; }

bool uses_copy_stream(int mode) { return mode == AGG_OVERLAP || mode == AGG_SERIAL || mode == AGG_COPY_ONLY; }

}  // namespace

extern "C" const char* agg_last_error(void) { return g_error.c_str(); }

extern "C" int agg_tile_shape(int op, int dtype, int64_t m, int64_t n, int64_t k, int* bm, int* bn) {
  if (!bm || !bn) return fail(AGG_E_ARG, "agg_tile_shape: NULL output");
  TileShape s = choose_tile(op, dtype, m, n, k);
  *bm = s.bm;
  *bn = s.bn;
  return AGG_OK;
}

extern "C" int agg_tail_split(int bm, int bn, int64_t m, int64_t n, int n_row_tiles, int units, int mode,
                              int* head_rows, int* tail_bm, int* tail_bn) {
  clear_error();
  if (!head_rows || !tail_bm || !tail_bn) return fail(AGG_E_ARG, "agg_tail_split: NULL output");
  if (mode != kTailAuto && mode != kTailOff && mode != kTailOn) return fail(AGG_E_ARG, "unknown tail mode %d", mode);
  const TailSplit t = tail_split(TileShape{bm, bn}, m, n, n_row_tiles, units, mode);
  *head_rows = t.head_rows;
  *tail_bm = t.tail.bm;
  *tail_bn = t.tail.bn;
  return AGG_OK;
}

extern "C" int agg_check_ag_args(int world, int rank, int64_t m_shard, int64_t n, int64_t k,
                                 int chunk_rows, int dtype, float scale_a, float scale_b,
                                 const void* const* peer_src, const void* gather, const void* flags,
                                 const void* b, const void* c, const int32_t* order, int n_order,
                                 int mode, agg_stream stream, agg_stream copy_stream) {
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD) return fail(AGG_E_ARG, "world %d not in [1, %d]", world, AGG_MAX_WORLD);
  if (rank < 0 || rank >= world) return fail(AGG_E_ARG, "rank %d not in [0, %d)", rank, world);
  if (m_shard < 0 || n < 0 || k < 0) return fail(AGG_E_ARG, "negative size");
  if (dtype != AGG_BF16 && dtype != AGG_FP8_E4M3) return fail(AGG_E_ARG, "unknown dtype %d", dtype);
  if (mode < AGG_OVERLAP || mode > AGG_COPY_ONLY) return fail(AGG_E_ARG, "unknown mode %d", mode);
  if (chunk_rows < 1) return fail(AGG_E_ARG, "chunk_rows %d < 1", chunk_rows);
  if (m_shard % chunk_rows) return fail(AGG_E_ARG, "chunk_rows %d does not divide m_shard %lld", chunk_rows, (long long)m_shard);
  const int64_t cps = m_shard / chunk_rows;
  if (world * cps > AGG_MAX_CHUNKS) return fail(AGG_E_UNSUPPORTED, "%lld chunks exceed %d", (long long)(world * cps), AGG_MAX_CHUNKS);
  const int eb = elem_bytes(dtype);
  if ((k * eb) % 16) return fail(AGG_E_ARG, "k * %d bytes = %lld is not a multiple of 16", eb, (long long)(k * eb));
  if ((n * 2) % 16) return fail(AGG_E_ARG, "n * 2 bytes = %lld is not a multiple of 16", (long long)(n * 2));
  if ((n * eb) % 16) return fail(AGG_E_ARG, "a row of b, n * %d bytes = %lld, is not a multiple of 16", eb, (long long)(n * eb));
  if (k > (int64_t(1) << 30) || n > (int64_t(1) << 30) || world * m_shard > (int64_t(1) << 30))
    return fail(AGG_E_UNSUPPORTED, "dimension beyond 2^30");
  if (world * m_shard * k * eb >= (int64_t(1) << 31) || n * k * eb >= (int64_t(1) << 31))
    return fail(AGG_E_UNSUPPORTED, "an operand reaches 2 GiB (the kernel addresses operands with 31-bit offsets)");
  if (dtype == AGG_FP8_E4M3 && !(std::isfinite(scale_a) && std::isfinite(scale_b) && scale_a > 0 && scale_b > 0))
    return fail(AGG_E_ARG, "fp8 scales must be finite and > 0 (got %g, %g)", scale_a, scale_b);
  if (uses_copy_stream(mode) && copy_stream && stream == copy_stream)
    return fail(AGG_E_ARG, "stream and copy_stream must differ");
  const int64_t m = world * m_shard;
  const bool empty = (m == 0);
  if (!empty) {
    if (k > 0 && (!gather || misaligned(gather))) return fail(AGG_E_ARG, "gather is NULL or not 16-byte aligned");
    if (world > 1 && (!flags || (reinterpret_cast<uintptr_t>(flags) & 3u))) return fail(AGG_E_ARG, "flags is NULL or not 4-byte aligned");
    if (mode != AGG_COPY_ONLY && n > 0) {
      if (k > 0 && (!b || misaligned(b))) return fail(AGG_E_ARG, "b is NULL or not 16-byte aligned");
      if (!c || misaligned(c)) return fail(AGG_E_ARG, "c is NULL or not 16-byte aligned");
    }
    if (world > 1 && mode != AGG_GEMM_ONLY && k > 0) {
      if (!peer_src) return fail(AGG_E_ARG, "peer_src is NULL");
      for (int p = 0; p < world; ++p)
        if (p != rank && (!peer_src[p] || misaligned(peer_src[p])))
          return fail(AGG_E_ARG, "peer_src[%d] is NULL or not 16-byte aligned", p);
    }
  }
  if (order == nullptr) {
    if (n_order != 0) return fail(AGG_E_ARG, "order is NULL but n_order = %d", n_order);
  } else if (int rc = check_order(world, rank, int(cps), order, n_order)) {
    return rc;
  }
  if (!empty) {
    TileShape s = choose_tile(0, dtype, m, n, k);
    if ((m + s.bm - 1) / s.bm > AGG_MAX_ROW_TILES)
      return fail(AGG_E_UNSUPPORTED, "%lld row tiles exceed %d", (long long)((m + s.bm - 1) / s.bm), AGG_MAX_ROW_TILES);
  }
  return AGG_OK;
}

extern "C" int agg_check_a2a_args(int world, int rank, int64_t cap, int64_t n, int64_t k,
                                  int chunk_rows, int dtype, float scale_a, float scale_b,
                                  const int32_t* counts, const void* const* peer_src, const void* recv,
                                  const void* flags, const void* b, const void* c, const int32_t* order,
                                  int n_order, int mode, agg_stream stream, agg_stream copy_stream) {
  if (int rc = agg_check_ag_args(world, rank, cap, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
                                 recv, flags, b, c, order, n_order, mode, stream, copy_stream))
    return rc;
  if (!counts) return fail(AGG_E_ARG, "counts is NULL");
  for (int p = 0; p < world; ++p)
    if (counts[p] < 0 || counts[p] > cap)
      return fail(AGG_E_ARG, "counts[%d] = %d not in [0, cap = %lld]", p, counts[p], (long long)cap);
  return AGG_OK;
}

extern "C" int agg_check_rs_args(int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                                 const void* a, const void* b, const void* send, const void* send_flags,
                                 const float* const* peer_src, const void* recv, const void* flags,
                                 const void* out, const int32_t* order, int n_order, int mode,
                                 agg_stream stream, agg_stream copy_stream) {
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD) return fail(AGG_E_ARG, "world %d not in [1, %d]", world, AGG_MAX_WORLD);
  if (rank < 0 || rank >= world) return fail(AGG_E_ARG, "rank %d not in [0, %d)", rank, world);
  if (m < 0 || n < 0 || k < 0) return fail(AGG_E_ARG, "negative size");
  if (mode < AGG_OVERLAP || mode > AGG_COPY_ONLY) return fail(AGG_E_ARG, "unknown mode %d", mode);
  if (m % world) return fail(AGG_E_ARG, "m %lld is not a multiple of world %d", (long long)m, world);
  if (chunk_rows < 1) return fail(AGG_E_ARG, "chunk_rows %d < 1", chunk_rows);
  const int64_t mb = m / world;
  if (mb % chunk_rows) return fail(AGG_E_ARG, "chunk_rows %d does not divide m/world %lld", chunk_rows, (long long)mb);
  const int64_t cpb = mb / chunk_rows;
  if (world * cpb > AGG_MAX_CHUNKS) return fail(AGG_E_UNSUPPORTED, "%lld chunks exceed %d", (long long)(world * cpb), AGG_MAX_CHUNKS);
  if ((k * 2) % 16) return fail(AGG_E_ARG, "k * 2 bytes = %lld is not a multiple of 16", (long long)(k * 2));
  if ((n * 2) % 16) return fail(AGG_E_ARG, "a row of b, n * 2 bytes = %lld, is not a multiple of 16", (long long)(n * 2));
  if (k > (int64_t(1) << 30) || n > (int64_t(1) << 30) || m > (int64_t(1) << 30))
    return fail(AGG_E_UNSUPPORTED, "dimension beyond 2^30");
  if (m * k * 2 >= (int64_t(1) << 31) || n * k * 2 >= (int64_t(1) << 31))
    return fail(AGG_E_UNSUPPORTED, "an operand reaches 2 GiB (the kernel addresses operands with 31-bit offsets)");
  if (m * n * 4 >= (int64_t(1) << 31))
    return fail(AGG_E_UNSUPPORTED, "the receive buffer reaches 2 GiB (31-bit offsets)");
  if (uses_copy_stream(mode) && copy_stream && stream == copy_stream)
    return fail(AGG_E_ARG, "stream and copy_stream must differ");
  if (mb > 0 && n > 0) {
    if (mode != AGG_COPY_ONLY) {
      if (k > 0 && (!a || misaligned(a))) return fail(AGG_E_ARG, "a is NULL or not 16-byte aligned");
      if (k > 0 && (!b || misaligned(b))) return fail(AGG_E_ARG, "b is NULL or not 16-byte aligned");
      if (world > 1 && (!send || misaligned(send))) return fail(AGG_E_ARG, "send is NULL or not 16-byte aligned");
      if (world > 1 && (!send_flags || (reinterpret_cast<uintptr_t>(send_flags) & 3u))) return fail(AGG_E_ARG, "send_flags is NULL or not 4-byte aligned");
      if (!out || misaligned(out)) return fail(AGG_E_ARG, "out is NULL or not 16-byte aligned");
    }
    if (world > 1) {
      if (!recv || misaligned(recv)) return fail(AGG_E_ARG, "recv is NULL or not 16-byte aligned");
      if (!flags || (reinterpret_cast<uintptr_t>(flags) & 3u)) return fail(AGG_E_ARG, "flags is NULL or not 4-byte aligned");
      if (mode != AGG_GEMM_ONLY) {
        if (!peer_src) return fail(AGG_E_ARG, "peer_src is NULL");
        for (int p = 0; p < world; ++p)
          if (p != rank && (!peer_src[p] || misaligned(peer_src[p])))
            return fail(AGG_E_ARG, "peer_src[%d] is NULL or not 16-byte aligned", p);
      }
    }
  }
  if (order == nullptr) {
    if (n_order != 0) return fail(AGG_E_ARG, "order is NULL but n_order = %d", n_order);
  } else if (int rc = check_order(world, rank, int(cpb), order, n_order)) {
    return rc;
  }
  if (mb > 0) {
    TileShape s = choose_tile(1, AGG_BF16, m, n, k);
    if (world * ((mb + s.bm - 1) / s.bm) > AGG_MAX_ROW_TILES)
      return fail(AGG_E_UNSUPPORTED, "row tiles exceed %d", AGG_MAX_ROW_TILES);
  }
  return AGG_OK;
}

extern "C" int agg_ag_row_tile_order(int world, int rank, int64_t m_shard, int chunk_rows,
                                     const int32_t* order, int n_order, int bm, int32_t* out_tiles,
                                     int max_tiles, int* n_tiles) {
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD || rank < 0 || rank >= world || m_shard < 0 ||
      chunk_rows < 1 || m_shard % chunk_rows || bm < 1 || !n_tiles)
    return fail(AGG_E_ARG, "agg_ag_row_tile_order: invalid geometry");
  const int cps = int(m_shard / chunk_rows);
  std::vector<int32_t> ord;
  if (order) {
    if (int rc = check_order(world, rank, cps, order, n_order)) return rc;
    ord.assign(order, order + n_order);
  } else {
    ord = ring_order(world, rank, cps);
  }
  std::vector<int32_t> t = ag_row_tile_order(world, rank, m_shard, chunk_rows, ord, bm);
  *n_tiles = int(t.size());
  if (int(t.size()) > max_tiles || (!out_tiles && !t.empty()))
    return fail(AGG_E_ARG, "agg_ag_row_tile_order: needs %d entries", int(t.size()));
  std::copy(t.begin(), t.end(), out_tiles);
  return AGG_OK;
}

extern "C" int agg_a2a_row_tile_order(int world, int rank, int64_t cap, int chunk_rows,
                                      const int32_t* counts, const int32_t* order, int n_order, int bm,
                                      int32_t* out_tiles, int max_tiles, int* n_tiles) {
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD || rank < 0 || rank >= world || cap < 0 ||
      chunk_rows < 1 || cap % chunk_rows || bm < 1 || !n_tiles || !counts)
    return fail(AGG_E_ARG, "agg_a2a_row_tile_order: invalid geometry");
  for (int p = 0; p < world; ++p)
    if (counts[p] < 0 || counts[p] > cap) return fail(AGG_E_ARG, "counts[%d] = %d not in [0, cap]", p, counts[p]);
  const int cps = int(cap / chunk_rows);
  std::vector<int32_t> ord;
  if (order) {
    if (int rc = check_order(world, rank, cps, order, n_order)) return rc;
    ord.assign(order, order + n_order);
  } else {
    ord = ring_order(world, rank, cps);
  }
  std::vector<int32_t> t = ag_row_tile_order(world, rank, cap, chunk_rows, ord, bm, counts);
  *n_tiles = int(t.size());
  if (int(t.size()) > max_tiles || (!out_tiles && !t.empty()))
    return fail(AGG_E_ARG, "agg_a2a_row_tile_order: needs %d entries", int(t.size()));
  std::copy(t.begin(), t.end(), out_tiles);
  return AGG_OK;
}

extern "C" int agg_rs_row_tile_order(int world, int rank, int64_t m, int chunk_rows,
                                     const int32_t* order, int n_order, int bm, int32_t* out_tiles,
                                     int max_tiles, int* n_tiles) {
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD || rank < 0 || rank >= world || m < 0 || m % world ||
      chunk_rows < 1 || (m / world) % chunk_rows || bm < 1 || !n_tiles)
    return fail(AGG_E_ARG, "agg_rs_row_tile_order: invalid geometry");
  const int cpb = int((m / world) / chunk_rows);
  std::vector<int32_t> ord;
  if (order) {
    if (int rc = check_order(world, rank, cpb, order, n_order)) return rc;
    ord.assign(order, order + n_order);
  } else {
    ord = ring_order(world, rank, cpb);
  }
  std::vector<int32_t> t = rs_row_tile_order(world, rank, m, chunk_rows, ord, bm);
  *n_tiles = int(t.size());
  if (int(t.size()) > max_tiles || (!out_tiles && !t.empty()))
    return fail(AGG_E_ARG, "agg_rs_row_tile_order: needs %d entries", int(t.size()));
  std::copy(t.begin(), t.end(), out_tiles);
  return AGG_OK;
}

extern "C" int agg_check_ar_args(int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                                 const void* a, const void* b, const void* send, const void* send_flags,
                                 const float* const* peer_src, const void* recv, const void* flags,
                                 const void* out, const int32_t* order, int n_order, int mode,
                                 agg_stream stream, agg_stream copy_stream) {
  using namespace agg;
  clear_error();
  if (world < 1 || world > AGG_MAX_WORLD) return fail(AGG_E_ARG, "world %d not in [1, %d]", world, AGG_MAX_WORLD);
  if (rank < 0 || rank >= world) return fail(AGG_E_ARG, "rank %d not in [0, %d)", rank, world);
  if (m < 0 || n < 0 || k < 0) return fail(AGG_E_ARG, "negative size");
  if (mode < AGG_OVERLAP || mode > AGG_COPY_ONLY) return fail(AGG_E_ARG, "unknown mode %d", mode);
  if (chunk_rows < 1) return fail(AGG_E_ARG, "chunk_rows %d < 1", chunk_rows);
  if (m % chunk_rows) return fail(AGG_E_ARG, "chunk_rows %d does not divide m %lld", chunk_rows, (long long)m);
  const int64_t cpb = m / chunk_rows;
  if (world * cpb > AGG_MAX_CHUNKS) return fail(AGG_E_UNSUPPORTED, "%lld chunks exceed %d", (long long)(world * cpb), AGG_MAX_CHUNKS);
  if ((k * 2) % 16) return fail(AGG_E_ARG, "k * 2 bytes = %lld is not a multiple of 16", (long long)(k * 2));
  if ((n * 2) % 16) return fail(AGG_E_ARG, "a row of b, n * 2 bytes = %lld, is not a multiple of 16", (long long)(n * 2));
  if (k > (int64_t(1) << 30) || n > (int64_t(1) << 30) || m > (int64_t(1) << 30))
    return fail(AGG_E_UNSUPPORTED, "dimension beyond 2^30");
  if (m * k * 2 >= (int64_t(1) << 31) || n * k * 2 >= (int64_t(1) << 31))
    return fail(AGG_E_UNSUPPORTED, "an operand reaches 2 GiB (the kernel addresses operands with 31-bit offsets)");
  if (world * m * n * 4 >= (int64_t(1) << 31))
    return fail(AGG_E_UNSUPPORTED, "the receive buffer reaches 2 GiB (31-bit offsets)");
  if (uses_copy_stream(mode) && copy_stream && stream == copy_stream)
    return fail(AGG_E_ARG, "stream and copy_stream must differ");
  if (m > 0 && n > 0) {
    if (mode != AGG_COPY_ONLY) {
      if (k > 0 && (!a || misaligned(a))) return fail(AGG_E_ARG, "a is NULL or not 16-byte aligned");
      if (k > 0 && (!b || misaligned(b))) return fail(AGG_E_ARG, "b is NULL or not 16-byte aligned");
      if (!send || misaligned(send)) return fail(AGG_E_ARG, "send is NULL or not 16-byte aligned");
      if (world > 1 && (!send_flags || (reinterpret_cast<uintptr_t>(send_flags) & 3u))) return fail(AGG_E_ARG, "send_flags is NULL or not 4-byte aligned");
      if (!out || misaligned(out)) return fail(AGG_E_ARG, "out is NULL or not 16-byte aligned");
    }
    if (world > 1) {
      if (!recv || misaligned(recv)) return fail(AGG_E_ARG, "recv is NULL or not 16-byte aligned");
      if (!flags || (reinterpret_cast<uintptr_t>(flags) & 3u)) return fail(AGG_E_ARG, "flags is NULL or not 4-byte aligned");
      if (mode != AGG_GEMM_ONLY) {
        if (!peer_src) return fail(AGG_E_ARG, "peer_src is NULL");
        for (int p = 0; p < world; ++p)
          if (p != rank && (!peer_src[p] || misaligned(peer_src[p])))
            return fail(AGG_E_ARG, "peer_src[%d] is NULL or not 16-byte aligned", p);
      }
    }
  }
  if (order == nullptr) {
    if (n_order != 0) return fail(AGG_E_ARG, "order is NULL but n_order = %d", n_order);
  } else if (int rc = check_order(world, rank, int(cpb), order, n_order)) {
    return rc;
  }
  if (m > 0) {
    TileShape s = choose_tile(2, AGG_BF16, m, n, k);
    if ((m + s.bm - 1) / s.bm > AGG_MAX_ROW_TILES) return fail(AGG_E_UNSUPPORTED, "row tiles exceed %d", AGG_MAX_ROW_TILES);
  }
  return AGG_OK;
}
