// Host-side planning shared by the C entry points: argument checks, tile shapes, row-tile
// orders, and the thread-local error text. Plain C++17, no HIP: it also builds with g++ alone.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace agg {

// Thread-local error text behind agg_last_error(); returns `code` for chaining.
int fail(int code, const char* fmt, ...);
void clear_error();

struct TileShape {
  int bm, bn;
};

// Output tile shape for one call. op: 0 = AllGather+GEMM, 1 = GEMM+ReduceScatter.
TileShape choose_tile(int op, int dtype, int64_t m, int64_t n, int64_t k);

// K slice of the kernel's main loop in bytes (64 for both operand types).
int slice_bytes(int dtype);

// Split-K: with fewer output tiles than half the compute units and a long K, each tile's K
// range is cut into `ksplit` parts computed by different workgroups (AllGather+GEMM only). The
// parts hold `kps` K slices each (the last one may hold fewer); every part is non-empty.
struct KSplit {
  int ksplit, kps;
};
KSplit choose_ksplit(int op, int dtype, int64_t tiles, int64_t k, int units);
// split-K exists for tiles of at most this many elements (128 x 128)
constexpr int kMaxSplitTileArea = 128 * 128;
constexpr int kMaxKSplit = 16;      // parts a caller may force
constexpr int kAutoKSplit = 4;      // parts chosen automatically (the reduction costs a pass per part)
constexpr int kMaxSplitTiles = 1024;   // tiles of a split-K call (one arrival counter each)

// Split of the claim lists (one per XCD) into list_rows x list_cols: list x takes the row tiles
// at compute positions x / list_cols, + list_rows, + 2 * list_rows, ... and the column tiles of
// block x % list_cols. Picks the split whose first wave of tiles on one XCD (`workers` tiles in
// flight) touches the fewest distinct A and B rows per K step, so the XCD's L2 holds them.
int choose_list_cols(int lists, int n_row_tiles, int n_col_tiles, int bm, int bn, int workers);

// Tail split of an AllGather+GEMM call whose tiles spill into a last, partly filled wave: the
// first `head_rows` row tiles of the compute order (whole waves of `ts` tiles) run in one launch,
// the remaining row tiles, cut into the smaller shape `tail`, in a second launch right after
// it. head_rows == 0: no split. mode: kTailAuto (split when a tile-time model says the second
// launch beats the last wave), kTailOff, kTailOn (split whenever a smaller shape exists and
// there are two row tiles or more).
constexpr int kTailAuto = 0, kTailOff = 1, kTailOn = 2;
struct TailSplit {
  int head_rows;
  TileShape tail;
};
TailSplit tail_split(TileShape ts, int64_t m, int64_t n, int n_rows, int units, int mode);

// Every candidate tile shape the kernels are instantiated for.
const std::vector<TileShape>& tile_shapes();

// Row tiles of the AllGather+GEMM output in computable order (see agg.h). With `counts`
// (AllToAll: slot p holds only its first counts[p] rows), chunks that hold no row count as
// present from the start and row tiles that hold no row are left out.
std::vector<int32_t> ag_row_tile_order(int world, int rank, int64_t m_shard, int chunk_rows,
                                       const std::vector<int32_t>& order, int bm,
                                       const int32_t* counts = nullptr);

// Row tiles (block * tiles_per_block + tile) of GEMM+ReduceScatter in compute order.
std::vector<int32_t> rs_row_tile_order(int world, int rank, int64_t m, int chunk_rows,
                                       const std::vector<int32_t>& order, int bm);

// Ring arrival order of the remote chunks: peers rank+1, rank+2, ... (mod world), chunks
// ascending within a peer.
std::vector<int32_t> ring_order(int world, int rank, int chunks_per_shard);

// Checks that `order` holds each remote chunk id exactly once. Returns AGG_OK or AGG_E_ARG.
int check_order(int world, int rank, int chunks_per_shard, const int32_t* order, int n_order);

}  // namespace agg
