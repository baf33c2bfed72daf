// Device-side interface of libagg: the argument block of the persistent GEMM kernel, the
// layout of the ctx's device scratch, and the launch functions (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/agg.h"

namespace agg {

// ctx scratch, in uint32 words
constexpr int kScrLists = 0;       // claim-list counters, one per XCD (<= 16)
constexpr int kScrDone = 16;       // workgroups that finished the current launch
constexpr int kScrStatus = 17;     // bit 0: a flag wait gave up
constexpr int kScrFailed = 18;     // first flag index that timed out (0xFFFFFFFF = none)
constexpr int kScrCopyNext = 19;   // in-kernel producer: next copy job
constexpr int kScrCopyT0 = 20;     // in-kernel producer: wall clock of the first job (delays)
constexpr int kScrRedNext = 21;    // ReduceScatter: next row group of the local block to reduce
constexpr int kScrCopyDone = 22;   // copy kernel: workgroups that finished the current launch
constexpr int kScrRsCount = 64;    // ReduceScatter per-send-chunk completion counters
constexpr int kScrPieces = kScrRsCount + AGG_MAX_CHUNKS;   // per-chunk copied-piece counters
constexpr int kScrOrder = kScrPieces + AGG_MAX_CHUNKS;     // arrival order (chunk ids)
constexpr int kScrDelay = kScrOrder + AGG_MAX_CHUNKS;      // cumulative producer delays (ticks)
constexpr int kScrRowOrder = kScrDelay + AGG_MAX_CHUNKS;   // row tiles in compute order
constexpr int kScrSplit = kScrRowOrder + AGG_MAX_ROW_TILES; // split-K: parts done per tile
constexpr int kScrLocal = kScrSplit + 1024;  // RS: local tiles stored, per row tile of the block
constexpr int kScrWords = kScrLocal + AGG_MAX_ROW_TILES;
constexpr int kMaxLists = 16;

enum Epilogue { kEpiAllGather = 0, kEpiReduceScatter = 1, kEpiAllReduce = 2, kEpiFfn = 3 };

// One set of copy jobs of the in-kernel producer: job i*pieces + q of the set moves piece q of the
// i-th arriving chunk from its peer's block into the symmetric buffer; the job completing a chunk
// releases its flag.
struct CopySet {
  const uint8_t* peer[AGG_MAX_WORLD];   // per-peer source blocks (emulated peers)
  uint8_t* sym;                         // symmetric buffer (gather / receive)
  uint32_t* put_flags;                  // flags the producer releases
  int64_t chunk_bytes, piece_bytes;
  int64_t valid_bytes[AGG_MAX_WORLD];   // bytes of each peer's slot that hold rows (AllToAll:
                                        // counts[p] rows; otherwise the whole slot)
  uint32_t jobs;                        // chunks x pieces of this set
  int pieces;                           // pieces per chunk
  int cps;                              // chunks per peer block
  int order_off;                        // its arrival order: scratch[kScrOrder + order_off + i]
  int piece_off;                        // its piece counters: scratch[kScrPieces + piece_off + chunk]
};

struct GemmArgs {
  const uint8_t* a;         // AG: gather buffer M x K; RS: A, M x K
  const uint8_t* b;         // K x N (N contiguous)
  uint16_t* c;              // AG output, M x N bfloat16
  float* send;              // RS: (world-1) x Mb x N; AR: M x N (the partial every peer gets)
  float* out;               // RS: Mb x N; AR: M x N
  const float* recv;        // RS: world x Mb x N; AR: world x M x N
  const uint32_t* flags;    // flags the tiles wait on (AG gather flags / RS, AR receive flags)
  uint32_t* send_flags;     // RS: world x Mb/cr; AR: M/cr
  uint32_t* scratch;        // ctx scratch (kScr*)
  uint32_t* trace;          // optional per-tile trace, 8 words per tile
  int64_t M, N, K;          // K in elements
  int64_t m_block;          // RS: rows per block (Mb)
  int world, rank;
  int chunk_rows, cps;      // rows per chunk, chunks per shard (AG) / per block (RS)
  int n_row_tiles;          // row tiles this launch computes (AG: up to ceil(M/BM); RS: world *
                            //   tiles_per_block), listed from scratch[kScrRowOrder + row_base]
  int row_base;             // AG: where this launch's row-tile order starts (a tail launch's
                            //   rows follow the head launch's in the same table)
  int n_col_tiles;          // ceil(N/BN) * ksplit: claimable columns (each tile's K parts)
  int ksplit;               // K parts per tile (1: no split); part p covers K slices
  int kps;                  //   [p*kps, min((p+1)*kps, slices)) of the main loop's slices
  float* ws;                // split-K partial products, ksplit x M x N fp32
  int split_together;       // split-K with every part of every tile in its own workgroup at
                            //   once: the parts sum the tile together, a row range each
  int tpb;                  // RS: row tiles per block
  int fuse_local;           // RS: the local block's tiles add the peers' partials themselves
                            //   (else every workgroup reduces the local block after the tiles)
  int n_lists;              // claim lists (one per XCD)
  int list_cols;            // lists split as (n_lists / list_cols) row groups x list_cols column blocks
  uint32_t epoch;           // flags >= epoch mean "arrived"
  float scale;              // fp8: scale_a * scale_b; bf16: 1
  uint64_t timeout_ticks;   // in wall-clock (s_memrealtime) ticks
  uint32_t trace_tiles;     // capacity of `trace` in tiles (0 = off)
  // (the row tiles in compute order are in scratch, kScrRowOrder + row_base)
  // in-kernel producer: the jobs of set 0, then those of set 1 (the FFN chain's receive chunks)
  CopySet cs[2];
  uint32_t copy_jobs;                   // 0: no copies in this launch; else cs[0].jobs + cs[1].jobs
  int copy_wgs;                         // workgroups that take copy jobs first (<= grid)
  int copy_delays;                      // nonzero: honour set 0's cumulative delays in scratch
  // AG pull: tiles read remote rows straight from the peers' blocks (no chunk wait); the copy
  // jobs (which still fill the gather buffer and release the flags) go to the last copy_wgs
  // workgroups, which claim tiles only after copying
  int pull;
  // AG push with copiers to spare (small gathers): the copy jobs go to the last copy_wgs
  // workgroups, which take no tile before copying, so no tile's start waits behind a copy of
  // its own workgroup; the tiles still wait for their chunks' flags
  int copiers_last;
  // nonzero: remote chunks may land while this launch runs (an overlapped call); a tile that
  // reads remote rows then acquires after its chunk waits. Otherwise every row a tile reads was
  // written before the launch began, which the launch's own start makes visible.
  int concurrent_producer;
  // flags this launch sets to the epoch at its start (workgroup 0): the local shard's chunks
  // (present from the call's start; a launch that carries the copy jobs marks them) and, for
  // ReduceScatter tile launches, the local block's send flags (nothing is sent for that block)
  uint32_t* mark_flags[3];
  int mark_count[3];
  // FFN chain (kEpiFfn): the fields above describe phase 2, a GEMM+ReduceScatter whose A is h
  // (K = the first layer's N); phase 1, AllGather+GEMM tiles whose epilogue writes
  // silu(product) into h as bf16, uses these. Tasks: phase 1's tiles (row tiles in scratch
  // kScrRowOrder[0 .. n_row_tiles1)) then phase 2's (kScrRowOrder[n_row_tiles1 ..]), claimed in
  // that order from one counter.
  const uint8_t* a1;                    // gather buffer M x K1
  const uint8_t* b1;                    // K1 x N1
  uint16_t* h;                          // M x N1 bfloat16
  const uint32_t* flags1;               // gather flags
  int64_t K1, N1;
  int chunk_rows1, cps1;
  int n_row_tiles1, n_col_tiles1;
};

// Launch the persistent kernel instantiated for (bm, bn, dtype, epilogue) with `grid`
// workgroups of 256 threads on `stream`; non-null events t0 / t1 receive the launch's start and
// end. Returns hipErrorInvalidValue for a shape that has no instantiation.
hipError_t launch_gemm(const GemmArgs& args, int bm, int bn, int dtype, int epilogue, int grid,
                       hipStream_t stream, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// Workgroups of the (bm, bn, dtype, epilogue) kernel that fit on one CU at once (0 for a shape
// without an instantiation).
int max_blocks_per_cu(int bm, int bn, int dtype, int epilogue);

// The producer as a kernel of its own (one wave per workgroup, `grid` workgroups, few registers),
// run beside the GEMM kernel in the register and wave slots it leaves free: args.cs / copy_jobs /
// epoch / scratch / mark_flags[0..1] as for the in-kernel producer.
hipError_t launch_copy(const GemmArgs& args, int grid, hipStream_t stream);

// Registers per lane of a GEMM kernel instance and of the copy kernel as the runtime reports
// them (hipFuncGetAttributes), or -1.
int kernel_regs(int bm, int bn, int dtype, int epilogue);
int copy_kernel_regs();

// Fill `words` uint32 at `dst` with `value` (a kernel, not a memset node).
hipError_t launch_fill_u32(uint32_t* dst, size_t words, uint32_t value, hipStream_t stream);

}  // namespace agg
