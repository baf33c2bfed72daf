// libagg host runtime: the ctx, the producers (put + signal) and the C entry points ag_gemm,
// ag_gemm_noalloc, gemm_rs, gemm_ar, ffn_chain and agg_put_signal.
//
// Method: page "Triton-distributed is turning communication into compiler territory", section
// "The first move was to expose the overlap": chunked transfers and computation proceed together
// instead of one after the other; the primitives are symmetric memory, remote data access,
// signaling and asynchronous tasks. Section "DITRON adds three levels of tiling": device-level
// tiles are data movements mapped onto DMA engines; collectives are chunked and paired with
// computation tiles with synchronization inserted.
//
// One chunk's "remote access" is a copy (hipMemcpyDeviceToDeviceNoCU) from the emulated peer's
// memory into the symmetric gather buffer; its "signal" is hipStreamWriteValue32 of the call's
// epoch into the chunk's flag word on the same stream, so stream order puts the flag after the
// data.
//
// This producer needs a few free compute units. A kernel trace of it shows the chunk copies
// (2 MiB each) on the copy engines, at about 51 GB/s per copy, but every stream write as a
// runtime kernel (__amd_rocclr_streamOpsWrite), and memsets and host-to-device copies are
// runtime kernels too. Under a grid that holds every CU those kernels never start, so the
// consumer would wait for them until its timeout. In overlap mode the persistent grid therefore
// leaves `reserved_cus` CUs to the producer (default 32, four per XCD: workgroups are dealt
// round-robin over the XCDs and one fills a CU; 8 and 16 free CUs were measured to still starve
// it); every other mode uses all CUs.
//
// The CU producer needs none of that: copy workgroups inside the persistent kernel take the chunk
// copies as jobs (arrival order, a chunk cut into pieces), the workgroup that completes a chunk
// releases its flag, and copy workgroups turn to tiles when the jobs run out. Its arrival order
// and delays sit in the ctx scratch, uploaded only when they change. The kernel producer runs the
// same jobs in a kernel of its own (one-wave workgroups) on one copy stream, resident beside the
// persistent kernel where the registers allow it.
//
// Chunks are spread over several copy streams (chunk i of the arrival order on stream i mod S),
// each stream feeding its own SDMA engine the way W-1 peers feed separate links; every stream
// keeps the arrival order, so chunks land in that order in groups of S.
//
// Every stream the ctx launches work on (the consumer kernel's and the copy streams) is created
// with a CU mask (all CUs), which gives it a hardware queue of its own. A shared queue deadlocks
// the overlap: the runtime may hand a stream write that follows an SDMA copy to the hardware only
// after the copy finishes, and if another stream has meanwhile put a barrier that waits for the
// persistent kernel into the same queue (the caller joining the kernel, say), the late write
// sits behind that barrier while the kernel waits for the write.
//
// Flags only grow within an epoch cycle (1 .. 0xFFFFFFFE); when the epoch would pass the end of
// the cycle the ctx zero-fills every flags buffer bound to it and starts again at 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "plan.h"

using namespace agg;

namespace {

constexpr uint32_t kEpochLast = 0xFFFFFFFEu;   // 0xFFFFFFFF means "no flag" in traces
constexpr int kMaxCopyStreams = 8;
constexpr int kDefaultCopyStreams = 4;
constexpr int kDefaultReservedCus = 32;
// AGG_PULL_AUTO pulls gathers of at most this many remote bytes (latency-bound transfers)
constexpr int64_t kPullMaxBytes = int64_t(4) << 20;
constexpr int kTimingRing = 256;          // launches whose kernel duration is kept

enum FlagSlot { kFlagsAg = 0, kFlagsRsRecv = 1, kFlagsRsSend = 2, kFlagsArRecv = 3, kFlagsArSend = 4, kFlagSlots = 5 };

// The no-allocation entry point's scratch: the kernel's counters, status and tables
// (kScrWords words, rounded up to 256 bytes) followed by room for split-K partials.
constexpr size_t kStaticWords = (size_t(kScrWords) + 63) / 64 * 64;
constexpr size_t kStaticWsBytes = size_t(8) << 20;
constexpr size_t kStaticBytes = kStaticWords * 4 + kStaticWsBytes;
constexpr int kMaxDevices = 64;

}  // namespace

// One copy per GPU, held until the process ends. Host code never passes this name to a kernel
// or a copy (on the host it is only a stand-in for the symbol): it uses the device address
// hipGetSymbolAddress returned for the current device at set-up (static_scratch_setup).
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticBytes];

namespace {

// Per device: the address of `scratch` on that device, and the tables it holds as last uploaded.
struct StaticScratch {
  uint32_t* words = nullptr;
  std::vector<uint32_t> up[3];
};
std::mutex g_static_mu;
StaticScratch g_static[kMaxDevices];

}  // namespace

struct agg_ctx {
  int device = 0;
  int cus = 0;
  int lists = 8;                    // claim lists: one per XCD of an MI355X
  int list_cols = 0;                // column blocks of the list grid (0: chosen per call)
  uint32_t* scratch = nullptr;      // kScrWords words
  uint32_t epoch = 0;
  uint64_t timeout_us = 2000000;
  double ticks_per_us = 100.0;
  int force_bm = 0, force_bn = 0;   // 0: automatic tile shape
  int n_copy = kDefaultCopyStreams;
  int reserved_cus = kDefaultReservedCus;   // CUs the overlapped grid leaves to the producer
  hipStream_t ks = nullptr;                           // consumer kernel stream (own HW queue)
  hipStream_t cstream[kMaxCopyStreams] = {};          // copy streams (own HW queues), lazily made
  hipEvent_t ev_fork = nullptr, ev_kernel = nullptr, ev_user = nullptr;
  hipEvent_t ev_copy[kMaxCopyStreams] = {};
  uint32_t* trace = nullptr;
  size_t trace_bytes = 0;
  int timing_every = 0;                     // record a timing event pair around every n-th
                                            // launch (0: none)
  hipEvent_t ev_t0[kTimingRing] = {}, ev_t1[kTimingRing] = {};
  uint64_t calls = 0;                       // launches since timing was switched on
  uint64_t launches = 0;                    // launches recorded since timing was switched on
  uint32_t* bound[kFlagSlots] = {};
  size_t bound_words[kFlagSlots] = {};
  int force_split = 0;                       // 0: split-K chosen per call
  bool chain_fused = true;                   // ffn_chain: both layers in one launch
  int tail = AGG_TAIL_AUTO;                  // ag_gemm / a2a_gemm: tail split of the last wave
  float* ws = nullptr;                       // split-K partials (grown on demand)
  size_t ws_bytes = 0;
  int producer = AGG_PRODUCER_CU;
  int last_producer = -1;        // the producer the last call ran (AGG_PRODUCER_*)
  int copy_wgs = 0;                          // 0: every workgroup takes copy jobs first
  int pull = AGG_PULL_AUTO;                  // AllGather+GEMM pull mode (overlapped CU calls)
  int64_t piece_bytes = 0;                   // 0: chosen per call
  // tables the kernel reads from scratch, as last uploaded: row tiles in compute order, arrival
  // order, cumulative delays (kScrRowOrder / kScrOrder / kScrDelay)
  std::vector<uint32_t> up[3];
  uint32_t* up_host = nullptr;               // pinned staging for the three tables
  bool used_static = false;                  // ag_gemm_noalloc ran on this ctx (its status and
                                             //   counters are in the device's static scratch)
  hipEvent_t ev_upload = nullptr;
  bool upload_pending = false;
};

namespace {

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(AGG_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

int elem_bytes(int dtype) { return dtype == AGG_FP8_E4M3 ? 1 : 2; }

hipStream_t S(agg_stream s) { return reinterpret_cast<hipStream_t>(s); }

void busy_wait_us(uint32_t us) {
  if (!us) return;
  auto end = std::chrono::steady_clock::now() + std::chrono::microseconds(us);
  while (std::chrono::steady_clock::now() < end) {
  }
}

int bind_flags(agg_ctx* ctx, int slot, uint32_t* p, size_t words) {
  if (!p || words == 0) return AGG_OK;
  if (ctx->bound[slot] == nullptr) {
    ctx->bound[slot] = p;
    ctx->bound_words[slot] = words;
    return AGG_OK;
  }
  if (ctx->bound[slot] != p)
    return fail(AGG_E_STATE, "a different flags buffer is bound to this ctx; call agg_ctx_reset first");
  ctx->bound_words[slot] = std::max(ctx->bound_words[slot], words);
  return AGG_OK;
}

// Advance the epoch for a producing call; at the end of a cycle zero-fill the bound flags on
// `stream` first (earlier producers were joined into `stream`, so this is ordered after them).
int next_epoch(agg_ctx* ctx, hipStream_t stream, uint32_t* out) {
  if (ctx->epoch >= kEpochLast) {
    for (int s = 0; s < kFlagSlots; ++s)
      if (ctx->bound[s]) HIP_TRY(launch_fill_u32(ctx->bound[s], ctx->bound_words[s], 0u, stream));
    ctx->epoch = 0;
  }
  ctx->epoch += 1;
  *out = ctx->epoch;
  return AGG_OK;
}

int put_signal(void* dst, const void* src, size_t bytes, uint32_t* flag, uint32_t value, hipStream_t cs) {
  if (bytes) HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDeviceNoCU, cs));
  HIP_TRY(hipStreamWriteValue32(cs, flag, value, 0));
  return AGG_OK;
}

// Chunk q of peer p: rows [q*cr, (q+1)*cr) of peer p's block, landing at rows
// p*slot_rows + q*cr of the symmetric buffer.
struct ChunkCopy {
  const uint8_t* const* src;   // [world] per-peer base
  uint8_t* dst;                // symmetric buffer base
  int64_t slot_rows, cr, row_bytes;
  int cps;
  const int32_t* valid_rows = nullptr;   // AllToAll: rows of each peer's slot that hold data
};

// Bytes of chunk q of peer p that hold rows: the whole chunk, or (AllToAll) the part of it
// below the peer's count.
int64_t held_bytes(const ChunkCopy& cc, int p, int q) {
  const int64_t rows = cc.valid_rows ? std::min<int64_t>(std::max<int64_t>(cc.valid_rows[p] - q * cc.cr, 0), cc.cr)
                                     : cc.cr;
  return rows * cc.row_bytes;
}

hipError_t make_own_queue_stream(agg_ctx* ctx, hipStream_t* out) {
  std::vector<uint32_t> mask(size_t((ctx->cus + 31) / 32), 0xFFFFFFFFu);
  return hipExtStreamCreateWithCUMask(out, uint32_t(mask.size()), mask.data());
}

// The ctx copy streams a call uses (created on first use).
int copy_streams(agg_ctx* ctx, size_t chunks, std::vector<hipStream_t>& out) {
  const int n = int(std::max<size_t>(1, std::min<size_t>(size_t(ctx->n_copy), chunks)));
  out.clear();
  for (int i = 0; i < n; ++i) {
    if (!ctx->cstream[i]) HIP_TRY(make_own_queue_stream(ctx, &ctx->cstream[i]));
    out.push_back(ctx->cstream[i]);
  }
  return AGG_OK;
}

int produce(const ChunkCopy& cc, uint32_t* flags, const std::vector<int32_t>& order,
            const uint32_t* delay_us, uint32_t epoch, const std::vector<hipStream_t>& streams,
            int rank) {
  const size_t bytes = size_t(cc.cr * cc.row_bytes);
  // the local shard's chunks are in place from the start: their flags are raised first
  for (int q = 0; q < cc.cps; ++q)
    HIP_TRY(hipStreamWriteValue32(streams[0], flags + size_t(rank) * cc.cps + q, epoch, 0));
  for (size_t i = 0; i < order.size(); ++i) {
    const int c = order[i];
    const int p = c / cc.cps, q = c % cc.cps;
    if (delay_us) busy_wait_us(delay_us[i]);
    const uint8_t* src = cc.src[p] + size_t(q) * bytes;
    uint8_t* dst = cc.dst + size_t(p * cc.slot_rows + q * cc.cr) * size_t(cc.row_bytes);
    if (int rc = put_signal(dst, src, size_t(held_bytes(cc, p, q)), flags + c, epoch, streams[i % streams.size()]))
      return rc;
  }
  return AGG_OK;
}

TileShape tile_for(agg_ctx* ctx, int op, int dtype, int64_t m, int64_t n, int64_t k) {
  if (ctx->force_bm) return TileShape{ctx->force_bm, ctx->force_bn};
  return choose_tile(op, dtype, m, n, k);
}

// Workgroups of the persistent grid: one per CU (a workgroup fills a CU), minus the CUs left to
// the producer when chunks arrive while the kernel runs.
int grid_for(agg_ctx* ctx, int64_t tiles, bool overlapped) {
  int64_t units = ctx->cus - (overlapped ? ctx->reserved_cus : 0);
  int64_t g = std::min<int64_t>(std::max<int64_t>(units, 1), tiles);
  return int(std::max<int64_t>(g, 1));
}

// Stream choreography shared by ag_gemm and gemm_rs. `launch` enqueues the consumer kernel on
// ctx->ks, `put_all` the producer's copies and flags on the copy streams.
//   OVERLAP:   stream -> {ks, copy streams}; kernel and chunks run together; all -> stream
//   SERIAL:    stream -> copy streams; all chunks; copy streams -> ks; kernel; ks -> stream
//   GEMM_ONLY: stream -> ks; kernel; ks -> stream
//   COPY_ONLY: stream -> copy streams; all chunks; copy streams -> stream
// A non-NULL user copy stream `us` is joined too: the copies start after earlier work on it, and
// later work on it starts after the copies.
template <typename Launch, typename Put>
int schedule(agg_ctx* ctx, int mode, hipStream_t s, hipStream_t us,
             const std::vector<hipStream_t>& cstreams, bool kernel, Launch launch, bool chunks,
             Put put_all, hipStream_t ks) {
  HIP_TRY(hipEventRecord(ctx->ev_fork, s));
  if (chunks) {
    if (us) HIP_TRY(hipEventRecord(ctx->ev_user, us));
    for (hipStream_t c : cstreams) {
      HIP_TRY(hipStreamWaitEvent(c, ctx->ev_fork, 0));
      if (us) HIP_TRY(hipStreamWaitEvent(c, ctx->ev_user, 0));
    }
  }
  auto join_copies = [&](hipStream_t into) -> int {
    for (size_t j = 0; j < cstreams.size(); ++j) {
      HIP_TRY(hipEventRecord(ctx->ev_copy[j], cstreams[j]));
      HIP_TRY(hipStreamWaitEvent(into, ctx->ev_copy[j], 0));
      if (us) HIP_TRY(hipStreamWaitEvent(us, ctx->ev_copy[j], 0));
    }
    return AGG_OK;
  };
  if (mode == AGG_OVERLAP) {
    // the kernel on the caller's stream: the copies go first, so that nothing enqueued later
    // can hold them behind the kernel that waits for them
    if (chunks && ks == s)
      if (int rc = put_all()) return rc;
    if (kernel) {
      if (ks != s) HIP_TRY(hipStreamWaitEvent(ks, ctx->ev_fork, 0));
      if (int rc = launch()) return rc;
    }
    if (chunks) {
      if (ks != s)
        if (int rc = put_all()) return rc;
      if (int rc = join_copies(s)) return rc;
    }
  } else {
    if (chunks) {
      if (int rc = put_all()) return rc;
      if (int rc = join_copies(kernel ? ks : s)) return rc;
    }
    if (kernel) {
      if (ks != s) HIP_TRY(hipStreamWaitEvent(ks, ctx->ev_fork, 0));
      if (int rc = launch()) return rc;
    }
  }
  if (kernel && ks != s) {
    HIP_TRY(hipEventRecord(ctx->ev_kernel, ks));
    HIP_TRY(hipStreamWaitEvent(s, ctx->ev_kernel, 0));
  }
  return AGG_OK;
}

// Enqueue the consumer kernel: launch(t0, t1) with the ring's next timing event pair when timing
// is on and this launch is one of the sampled ones (the launch itself records the kernel's start
// and end in them: no marker packets on the stream), or with null events.
template <typename F>
int timed_launch(agg_ctx* ctx, F launch) {
  if (!ctx->timing_every || ctx->calls++ % uint64_t(ctx->timing_every) != 0) {
    HIP_TRY(launch(nullptr, nullptr));
    return AGG_OK;
  }
  const int slot = int(ctx->launches % kTimingRing);
  HIP_TRY(launch(ctx->ev_t0[slot], ctx->ev_t1[slot]));
  ++ctx->launches;
  return AGG_OK;
}

// The scratch a call's kernels use: the ctx's own (counters and tables allocated at creation,
// split-K partials grown on demand) or, for ag_gemm_noalloc, the device's static array (fixed
// room for partials, nothing allocated).
struct Scratch {
  uint32_t* words;              // kScrWords counters, status and tables
  std::vector<uint32_t>* up;    // the three tables the words hold, as last uploaded
  bool fixed;                   // true: partials only in the static array's fixed room
};

Scratch own_scratch(agg_ctx* ctx) { return Scratch{ctx->scratch, ctx->up, false}; }

// The split-K partial buffer, grown to `bytes` when needed (a synchronising reallocation: the
// previous buffer may still be read by enqueued work).
int ensure_ws(agg_ctx* ctx, size_t bytes) {
  if (bytes <= ctx->ws_bytes) return AGG_OK;
  if (ctx->ws) {
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipFree(ctx->ws));
    ctx->ws = nullptr;
    ctx->ws_bytes = 0;
  }
  HIP_TRY(hipMalloc(reinterpret_cast<void**>(&ctx->ws), bytes));
  ctx->ws_bytes = bytes;
  return AGG_OK;
}

// K split of one AllGather+GEMM call (the ctx may force one; tiles above 128 x 128 never split).
KSplit ksplit_for(agg_ctx* ctx, TileShape ts, int dtype, int64_t tiles, int64_t k) {
  KSplit ks = choose_ksplit(0, dtype, tiles, k, ctx->cus);
  if (ts.bm * ts.bn > kMaxSplitTileArea) {
    ks.ksplit = 1;
    const int64_t kb = k * (dtype == AGG_FP8_E4M3 ? 1 : 2);
    ks.kps = int(std::max<int64_t>(1, (kb + slice_bytes(dtype) - 1) / slice_bytes(dtype)));
  } else if (ctx->force_split > 0) {
    const int64_t kb = k * (dtype == AGG_FP8_E4M3 ? 1 : 2);
    const int64_t nk = std::max<int64_t>(1, (kb + slice_bytes(dtype) - 1) / slice_bytes(dtype));
    const int64_t s = std::min<int64_t>(ctx->force_split, nk);
    ks.kps = int((nk + s - 1) / s);
    ks.kps += ks.kps & 1;                   // parts start on whole slice pairs
    ks.ksplit = int((nk + ks.kps - 1) / ks.kps);
  }
  return ks;
}

void fill_common(agg_ctx* ctx, GemmArgs& g, TileShape ts, int grid) {
  g.n_lists = std::min(ctx->lists, kMaxLists);
  g.list_cols = ctx->list_cols > 0 && g.n_lists % ctx->list_cols == 0
                    ? ctx->list_cols
                    : choose_list_cols(g.n_lists, g.n_row_tiles, g.n_col_tiles, ts.bm, ts.bn,
                                       (grid + g.n_lists - 1) / g.n_lists);
  g.timeout_ticks = uint64_t(double(ctx->timeout_us) * ctx->ticks_per_us);
}

// The tables the kernel reads from scratch: 0 = row tiles in compute order, 1 = arrival order of
// the remote chunks, 2 = cumulative producer delays in wall-clock ticks.
constexpr int kTabWords[3] = {AGG_MAX_ROW_TILES, AGG_MAX_CHUNKS, AGG_MAX_CHUNKS};
constexpr int kTabScratch[3] = {kScrRowOrder, kScrOrder, kScrDelay};
constexpr int kTabHost[3] = {0, AGG_MAX_ROW_TILES, AGG_MAX_ROW_TILES + AGG_MAX_CHUNKS};
constexpr int kTabHostWords = AGG_MAX_ROW_TILES + 2 * AGG_MAX_CHUNKS;

// Copy table `t` into scratch on stream `s`, unless scratch already holds exactly `v`. The
// pinned staging area is reused only after the previous upload has been consumed.
int upload_table(agg_ctx* ctx, const Scratch& sp, hipStream_t s, int t, const std::vector<uint32_t>& v) {
  if (v.empty() || v == sp.up[t]) return AGG_OK;
  if (v.size() > size_t(kTabWords[t])) return fail(AGG_E_UNSUPPORTED, "table %d: %zu entries exceed %d", t, v.size(), kTabWords[t]);
  if (ctx->upload_pending) {
    HIP_TRY(hipEventSynchronize(ctx->ev_upload));
    ctx->upload_pending = false;
  }
  std::memcpy(ctx->up_host + kTabHost[t], v.data(), v.size() * sizeof(uint32_t));
  HIP_TRY(hipMemcpyAsync(sp.words + kTabScratch[t], ctx->up_host + kTabHost[t],
                         v.size() * sizeof(uint32_t), hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(ctx->ev_upload, s));
  ctx->upload_pending = true;
  sp.up[t] = v;
  return AGG_OK;
}

int upload_rows(agg_ctx* ctx, const Scratch& sp, hipStream_t s, const std::vector<int32_t>& rows) {
  return upload_table(ctx, sp, s, 0, std::vector<uint32_t>(rows.begin(), rows.end()));
}

// Arrival order and cumulative delays (wall-clock ticks) for the CU producer.
int upload_schedule(agg_ctx* ctx, const Scratch& sp, hipStream_t s, const std::vector<int32_t>& ord,
                    const uint32_t* delay_us) {
  if (int rc = upload_table(ctx, sp, s, 1, std::vector<uint32_t>(ord.begin(), ord.end()))) return rc;
  if (!delay_us) return AGG_OK;
  std::vector<uint32_t> d(ord.size());
  double sum = 0;
  for (size_t i = 0; i < ord.size(); ++i) {
    sum += double(delay_us[i]) * ctx->ticks_per_us;
    d[i] = uint32_t(std::min(sum, 4.0e9));
  }
  return upload_table(ctx, sp, s, 2, d);
}

// One set of copies of the producer: its chunk geometry, the flags it releases and how many
// chunks arrive (in the order uploaded for it).
struct CopyPlan {
  ChunkCopy cc;
  uint32_t* flags;
  size_t n_order;
};

// Copy-job fields of the kernel arguments for the CU producer: set s's jobs follow set s-1's, its
// arrival order follows theirs in the uploaded table, and its piece counters start at s * 2048.
void fill_copies(agg_ctx* ctx, GemmArgs& g, const CopyPlan* sets, int nsets, bool delays, int world,
                 int grid, int pull_copiers, int64_t min_piece = 65536) {
  // automatic piece size: as many pieces per chunk as keep every job in one round of the
  // copying workgroups (so no workgroup copies twice while others idle), in whole 4 KiB pages,
  // at least min_piece: for the persistent kernel's 256-thread copiers, when tiles wait for the
  // chunks, 64 KiB, one round of their copy loop (256 threads x 16 vectors of 16 bytes), so a
  // smaller piece saves no time and adds a counted piece to its chunk (pushed small gathers:
  // 64 KiB pieces took the 256-row call's launch from 13.4 to 12.7 us and the decode gather's
  // from 46.2 to 45.5 against 16 KiB); 16 KiB for pulled calls and the copy kernel
  const int copiers = pull_copiers > 0 ? pull_copiers
                      : ctx->copy_wgs > 0 ? std::min(ctx->copy_wgs, grid) : grid;
  size_t chunks = 0;
  for (int s = 0; s < nsets; ++s) chunks += sets[s].n_order;
  const int64_t per_chunk = std::max<int64_t>(1, int64_t(copiers) / std::max<int64_t>(int64_t(chunks), 1));
  g.copy_jobs = 0;
  int order_off = 0;
  for (int s = 0; s < 2; ++s) {
    CopySet& cs = g.cs[s];
    std::memset(&cs, 0, sizeof cs);
    if (s >= nsets) continue;
    const CopyPlan& pl = sets[s];
    for (int p = 0; p < world; ++p) {
      cs.peer[p] = pl.cc.src[p];
      cs.valid_bytes[p] = (pl.cc.valid_rows ? pl.cc.valid_rows[p] : pl.cc.slot_rows) * pl.cc.row_bytes;
    }
    cs.sym = pl.cc.dst;
    cs.put_flags = pl.flags;
    cs.chunk_bytes = pl.cc.cr * pl.cc.row_bytes;
    const int64_t autop =
        std::max<int64_t>(((cs.chunk_bytes + per_chunk - 1) / per_chunk + 4095) / 4096 * 4096, min_piece);
    const int64_t piece = std::max<int64_t>(16, (ctx->piece_bytes > 0 ? ctx->piece_bytes : autop) / 16 * 16);
    cs.piece_bytes = std::min<int64_t>(cs.chunk_bytes, piece);
    cs.pieces = cs.piece_bytes > 0 ? int((cs.chunk_bytes + cs.piece_bytes - 1) / cs.piece_bytes) : 1;
    if (cs.piece_bytes == 0) cs.piece_bytes = 16;   // empty chunks (k = 0): one empty piece each
    cs.jobs = uint32_t(pl.n_order) * uint32_t(cs.pieces);
    cs.cps = pl.cc.cps;
    cs.order_off = order_off;
    cs.piece_off = s * (AGG_MAX_CHUNKS / 2);
    order_off += int(pl.n_order);
    g.copy_jobs += cs.jobs;
  }
  // default: every workgroup copies first. A grid of one tile per workgroup finishes at the last
  // tile's start plus one tile time, and the copy ends soonest with every workgroup on it.
  g.copy_wgs = copiers;
  g.copy_delays = delays ? 1 : 0;
}

void attach_trace(agg_ctx* ctx, GemmArgs& g, int64_t tiles) {
  if (ctx->trace && ctx->trace_bytes / 32 >= size_t(tiles)) {
    g.trace = ctx->trace;
    g.trace_tiles = uint32_t(tiles);
  }
}

// Flags a launch raises to the epoch at its start: the local slot of the flags each producer set
// releases (a launch with copy jobs) and, ReduceScatter, the local slot of the send flags (a
// launch with tiles).
struct Marks {
  uint32_t* copy_flags[2] = {nullptr, nullptr};
  int copy_count[2] = {0, 0};
  uint32_t* tile_flags = nullptr;
  int tile_count = 0;
};

// One launch of the persistent kernel under the CU producer: `copies` adds the copy jobs,
// `tiles_on` keeps the GEMM tiles (without them: a copy-only grid of one workgroup per CU).
// A tail launch (ag_gemm's tail split): the second launch of a call's tiles, with its own
// arguments, shape and grid; it carries no copies and marks no flags.
struct TailLaunch {
  const GemmArgs* g = nullptr;
  TileShape ts{0, 0};
  int grid = 0;
};

int launch_cu(agg_ctx* ctx, hipStream_t ls, const GemmArgs& g, TileShape ts, int dtype, int epi,
              int grid, const CopyPlan* sets, int nsets, bool delays, int world, uint32_t epoch,
              bool copies, bool tiles_on, bool timed, const Marks& marks, int pull_copiers = 0,
              const TailLaunch& tail = TailLaunch{}, int last_copiers = 0) {
  GemmArgs h = g;
  h.mark_count[0] = h.mark_count[1] = h.mark_count[2] = 0;
  if (copies) {
    for (int s = 0; s < 2; ++s)
      if (marks.copy_flags[s]) {
        h.mark_flags[s] = marks.copy_flags[s];
        h.mark_count[s] = marks.copy_count[s];
      }
  }
  if (tiles_on && marks.tile_flags) {
    h.mark_flags[2] = marks.tile_flags;
    h.mark_count[2] = marks.tile_count;
  }
  int gr = grid;
  // pull only where tiles and copies share the launch: the grid gains the copiers
  const bool pull = pull_copiers > 0 && copies && tiles_on;
  h.pull = pull ? 1 : 0;
  if (pull) gr = grid + pull_copiers;
  // small pushed gathers: the copiers after the tile workgroups
  const bool last = !pull && last_copiers > 0 && copies && tiles_on;
  h.copiers_last = last ? 1 : 0;
  if (last) gr = grid + last_copiers;
  if (!tiles_on) {
    h.n_row_tiles = 0;
    h.n_col_tiles = 0;
    h.n_row_tiles1 = 0;
    h.n_col_tiles1 = 0;
    h.trace = nullptr;
    h.trace_tiles = 0;
    h.n_lists = 1;
    h.list_cols = 1;
    h.ksplit = 1;
    h.epoch = epoch;
    gr = ctx->cus;
  }
  if (copies) {
    h.epoch = epoch;
    // (pulled: the copies gate no tile; 16 KiB pieces over more copiers end them sooner)
    fill_copies(ctx, h, sets, nsets, delays, world, gr, pull ? pull_copiers : last ? last_copiers : 0,
                pull ? 16384 : 65536);
  } else {
    h.copy_jobs = 0;
    std::memset(h.cs, 0, sizeof h.cs);
  }
  // with a tail launch (tiles only), the timing events span both: the start of the first and
  // the end of the second
  const bool two = tiles_on && tail.g;
  auto go = [&](hipEvent_t t0, hipEvent_t t1) -> hipError_t {
    if (!two) return launch_gemm(h, ts.bm, ts.bn, dtype, epi, gr, ls, t0, t1);
    const hipError_t e = launch_gemm(h, ts.bm, ts.bn, dtype, epi, gr, ls, t0, nullptr);
    if (e != hipSuccess) return e;
    return launch_gemm(*tail.g, tail.ts.bm, tail.ts.bn, dtype, epi, tail.grid, ls, nullptr, t1);
  };
  if (timed) return timed_launch(ctx, go);
  HIP_TRY(go(nullptr, nullptr));
  return AGG_OK;
}

// Whether the consumer kernel may run on the caller's stream beside the copy kernel: not on the
// legacy default stream (or the per-thread one), whose implicit synchronisation would hold the
// copy kernel's stream behind the consumer that waits for it.
bool own_queue_free(hipStream_t s) { return s != nullptr && s != hipStreamPerThread; }

// The producer a call runs: the ctx's choice, except that the copy kernel (AGG_PRODUCER_KERNEL)
// gives way to copy jobs inside the GEMM kernel where it cannot run beside it (the GEMM kernel
// leaves it too few registers on a SIMD) or where delays are asked for.
constexpr int kCopyGrid = 1024;           // copy-kernel workgroups (one wave each): one per SIMD
int effective_producer(agg_ctx* ctx, TileShape ts, int dtype, int epi, bool delays) {
  if (ctx->producer != AGG_PRODUCER_KERNEL) return ctx->producer;
  if (delays) return AGG_PRODUCER_CU;
  auto alloc = [](int r) { return (r + 7) / 8 * 8; };
  const int g = kernel_regs(ts.bm, ts.bn, dtype, epi), c = copy_kernel_regs();
  if (g < 0 || c < 0 || alloc(g) + alloc(c) > 512) return AGG_PRODUCER_CU;
  return AGG_PRODUCER_KERNEL;
}

// Enqueue the copy kernel for `plans` on `cs` (the producer as a kernel of its own).
int launch_copy_producer(agg_ctx* ctx, uint32_t* scratch, const CopyPlan* plans, int nsets, int world,
                         uint32_t epoch, const Marks& marks, hipStream_t cs) {
  GemmArgs gc;
  std::memset(&gc, 0, sizeof gc);
  gc.scratch = scratch;
  gc.epoch = epoch;
  // pieces sized for every copy-kernel workgroup (the CU producer's copy_wgs does not apply)
  fill_copies(ctx, gc, plans, nsets, false, world, kCopyGrid, kCopyGrid, 16384);
  for (int s = 0; s < 2; ++s) {
    gc.mark_flags[s] = marks.copy_flags[s];
    gc.mark_count[s] = marks.copy_flags[s] ? marks.copy_count[s] : 0;
  }
  HIP_TRY(launch_copy(gc, kCopyGrid, cs));
  return AGG_OK;
}

// Stream choreography under the CU producer. Nothing runs beside the kernel, so it goes on the
// caller's stream itself (no fork, no join, no second hardware queue):
//   OVERLAP:   one launch (copy jobs, then tiles)
//   SERIAL:    copy-only launch; GEMM launch
//   GEMM_ONLY: GEMM launch
//   COPY_ONLY: copy-only launch
// A non-NULL user copy stream is joined around the launches. `launch(copies, tiles, timed)`.
template <typename Launch>
int schedule_cu(agg_ctx* ctx, int mode, hipStream_t s, hipStream_t us, bool kernel, bool chunks,
                Launch launch) {
  if (chunks && us) {
    HIP_TRY(hipEventRecord(ctx->ev_user, us));
    HIP_TRY(hipStreamWaitEvent(s, ctx->ev_user, 0));
  }
  int rc = AGG_OK;
  if (mode == AGG_OVERLAP) {
    if (kernel || chunks) rc = launch(chunks, kernel, true);
  } else if (mode == AGG_SERIAL) {
    if (chunks) rc = launch(true, false, !kernel);
    if (rc == AGG_OK && kernel) rc = launch(false, true, true);
  } else if (mode == AGG_GEMM_ONLY) {
    if (kernel) rc = launch(false, true, true);
  } else if (chunks) {
    rc = launch(true, false, true);
  }
  if (rc != AGG_OK) return rc;
  if (chunks && us) {
    HIP_TRY(hipEventRecord(ctx->ev_kernel, s));
    HIP_TRY(hipStreamWaitEvent(us, ctx->ev_kernel, 0));
  }
  return AGG_OK;
}

}  // namespace

namespace {

// Find the device address of `scratch` on `device` (current) once, and clear its counters; the
// failed-flag word starts at "none". The partials need no initial value.
int static_scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(AGG_E_UNSUPPORTED, "device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static[device].words) return AGG_OK;
  void* p = nullptr;
  HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
  uint32_t* w = static_cast<uint32_t*>(p);
  HIP_TRY(launch_fill_u32(w, kScrWords, 0u, nullptr));
  HIP_TRY(launch_fill_u32(w + kScrFailed, 1, 0xFFFFFFFFu, nullptr));
  HIP_TRY(hipStreamSynchronize(nullptr));
  g_static[device].words = w;
  return AGG_OK;
}

Scratch static_scratch(int device) { return Scratch{g_static[device].words, g_static[device].up, true}; }

}  // namespace

// ------------------------------------------------------------------------------------------
// ctx
// ------------------------------------------------------------------------------------------

extern "C" int agg_ctx_create(int device, agg_ctx** out) {
  clear_error();
  if (!out) return fail(AGG_E_ARG, "out is NULL");
  *out = nullptr;
  int count = 0;
  HIP_TRY(hipGetDeviceCount(&count));
  if (device < 0 || device >= count) return fail(AGG_E_ARG, "device %d not in [0, %d)", device, count);
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(AGG_E_UNSUPPORTED, "device %d is %s, libagg is built for gfx950 only", device, prop.gcnArchName);
  int prev = 0;
  HIP_TRY(hipGetDevice(&prev));
  HIP_TRY(hipSetDevice(device));
  agg_ctx* ctx = new agg_ctx;
  ctx->device = device;
  ctx->cus = prop.multiProcessorCount;
  int rate_khz = 0;
  if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && rate_khz > 0)
    ctx->ticks_per_us = rate_khz / 1000.0;
  int rc = AGG_OK;
  auto step = [&](hipError_t e, const char* what) {
    if (rc == AGG_OK && e != hipSuccess) rc = fail(AGG_E_HIP, "%s: %s", what, hipGetErrorString(e));
  };
  step(hipMalloc(&ctx->scratch, kScrWords * sizeof(uint32_t)), "hipMalloc(scratch)");
  if (rc == AGG_OK) {
    std::vector<uint32_t> host(kScrWords, 0u);
    host[kScrFailed] = 0xFFFFFFFFu;
    step(hipMemcpy(ctx->scratch, host.data(), kScrWords * sizeof(uint32_t), hipMemcpyHostToDevice),
         "hipMemcpy(scratch)");
  }
  step(hipEventCreateWithFlags(&ctx->ev_fork, hipEventDisableTiming), "hipEventCreate");
  step(hipEventCreateWithFlags(&ctx->ev_kernel, hipEventDisableTiming), "hipEventCreate");
  step(hipEventCreateWithFlags(&ctx->ev_user, hipEventDisableTiming), "hipEventCreate");
  step(hipEventCreateWithFlags(&ctx->ev_upload, hipEventDisableTiming), "hipEventCreate");
  for (int j = 0; j < kMaxCopyStreams; ++j)
    step(hipEventCreateWithFlags(&ctx->ev_copy[j], hipEventDisableTiming), "hipEventCreate");
  if (rc == AGG_OK) step(make_own_queue_stream(ctx, &ctx->ks), "hipExtStreamCreateWithCUMask");
  step(hipHostMalloc(reinterpret_cast<void**>(&ctx->up_host), kTabHostWords * sizeof(uint32_t)),
       "hipHostMalloc(tables)");
  if (rc == AGG_OK) rc = static_scratch_setup(device);
  step(hipSetDevice(prev), "hipSetDevice");
  if (rc != AGG_OK) {
    agg_ctx_destroy(ctx);
    return rc;
  }
  *out = ctx;
  return AGG_OK;
}

extern "C" int agg_ctx_destroy(agg_ctx* ctx) {
  clear_error();
  if (!ctx) return AGG_OK;
  // best effort: release everything even if one call fails, report the first failure
  int rc = AGG_OK;
  auto step = [&](hipError_t e, const char* what) {
    if (rc == AGG_OK && e != hipSuccess) rc = fail(AGG_E_HIP, "%s: %s", what, hipGetErrorString(e));
  };
  int prev = 0;
  step(hipGetDevice(&prev), "hipGetDevice");
  step(hipSetDevice(ctx->device), "hipSetDevice");
  step(hipDeviceSynchronize(), "hipDeviceSynchronize");
  if (ctx->scratch) step(hipFree(ctx->scratch), "hipFree(scratch)");
  for (hipEvent_t e : {ctx->ev_fork, ctx->ev_kernel, ctx->ev_user, ctx->ev_upload})
    if (e) step(hipEventDestroy(e), "hipEventDestroy");
  if (ctx->up_host) step(hipHostFree(ctx->up_host), "hipHostFree");
  if (ctx->ws) step(hipFree(ctx->ws), "hipFree(ws)");
  for (int j = 0; j < kTimingRing; ++j) {
    if (ctx->ev_t0[j]) step(hipEventDestroy(ctx->ev_t0[j]), "hipEventDestroy");
    if (ctx->ev_t1[j]) step(hipEventDestroy(ctx->ev_t1[j]), "hipEventDestroy");
  }
  for (int j = 0; j < kMaxCopyStreams; ++j) {
    if (ctx->ev_copy[j]) step(hipEventDestroy(ctx->ev_copy[j]), "hipEventDestroy");
    if (ctx->cstream[j]) step(hipStreamDestroy(ctx->cstream[j]), "hipStreamDestroy");
  }
  if (ctx->ks) step(hipStreamDestroy(ctx->ks), "hipStreamDestroy");
  step(hipSetDevice(prev), "hipSetDevice");
  delete ctx;
  return rc;
}

extern "C" int agg_ctx_reset(agg_ctx* ctx, agg_stream stream) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  HIP_TRY(hipSetDevice(ctx->device));
  HIP_TRY(hipDeviceSynchronize());
  for (int s = 0; s < kFlagSlots; ++s) {
    if (ctx->bound[s]) HIP_TRY(launch_fill_u32(ctx->bound[s], ctx->bound_words[s], 0u, S(stream)));
    ctx->bound[s] = nullptr;
    ctx->bound_words[s] = 0;
  }
  HIP_TRY(launch_fill_u32(ctx->scratch, kScrWords, 0u, S(stream)));
  HIP_TRY(launch_fill_u32(ctx->scratch + kScrFailed, 1, 0xFFFFFFFFu, S(stream)));
  if (ctx->used_static) {
    // the device's static scratch too (shared by every ctx on the device)
    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticScratch& st = g_static[ctx->device];
    HIP_TRY(launch_fill_u32(st.words, kScrWords, 0u, S(stream)));
    HIP_TRY(launch_fill_u32(st.words + kScrFailed, 1, 0xFFFFFFFFu, S(stream)));
    for (auto& t : st.up) t.clear();
    ctx->used_static = false;
  }
  HIP_TRY(hipStreamSynchronize(S(stream)));
  ctx->epoch = 0;
  for (auto& t : ctx->up) t.clear();   // the scratch copies of the tables are gone too
  return AGG_OK;
}

extern "C" int agg_ctx_status(agg_ctx* ctx, agg_stream stream, uint32_t* status, int32_t* failed_chunk) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  HIP_TRY(hipSetDevice(ctx->device));
  HIP_TRY(hipStreamSynchronize(S(stream)));
  uint32_t words[2] = {0, 0};
  HIP_TRY(hipMemcpy(words, ctx->scratch + kScrStatus, sizeof words, hipMemcpyDeviceToHost));
  if (ctx->used_static) {
    uint32_t st[2] = {0, 0};
    HIP_TRY(hipMemcpy(st, g_static[ctx->device].words + kScrStatus, sizeof st, hipMemcpyDeviceToHost));
    if (!words[0]) words[1] = st[1];
    words[0] |= st[0];
  }
  if (status) *status = words[0];
  if (failed_chunk) *failed_chunk = words[1] == 0xFFFFFFFFu ? -1 : int32_t(words[1]);
  if (words[0]) return fail(AGG_E_TIMEOUT, "a chunk wait gave up (flag %d)", words[1] == 0xFFFFFFFFu ? -1 : int(words[1]));
  return AGG_OK;
}

extern "C" int agg_ctx_epoch(agg_ctx* ctx, uint32_t* epoch) {
  clear_error();
  if (!ctx || !epoch) return fail(AGG_E_ARG, "NULL argument");
  *epoch = ctx->epoch;
  return AGG_OK;
}

extern "C" int agg_ctx_set_epoch(agg_ctx* ctx, uint32_t epoch) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (epoch > kEpochLast) return fail(AGG_E_ARG, "epoch %u beyond %u", epoch, kEpochLast);
  for (int s = 0; s < kFlagSlots; ++s)
    if (ctx->bound[s]) return fail(AGG_E_STATE, "flags are bound; call agg_ctx_reset first");
  ctx->epoch = epoch;
  return AGG_OK;
}

extern "C" int agg_ctx_set_timeout_us(agg_ctx* ctx, uint64_t timeout_us) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (timeout_us == 0 || timeout_us > 30000000ull) return fail(AGG_E_ARG, "timeout must be in (0, 30 s]");
  ctx->timeout_us = timeout_us;
  return AGG_OK;
}

extern "C" int agg_ctx_set_tile(agg_ctx* ctx, int bm, int bn) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (bm == 0 && bn == 0) {
    ctx->force_bm = ctx->force_bn = 0;
    return AGG_OK;
  }
  for (const TileShape& t : tile_shapes())
    if (t.bm == bm && t.bn == bn) {
      ctx->force_bm = bm;
      ctx->force_bn = bn;
      return AGG_OK;
    }
  return fail(AGG_E_ARG, "no kernel for a %dx%d tile", bm, bn);
}

extern "C" int agg_ctx_set_producer(agg_ctx* ctx, int kind, int copy_wgs, int piece_kib) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (kind != AGG_PRODUCER_CU && kind != AGG_PRODUCER_SDMA && kind != AGG_PRODUCER_KERNEL)
    return fail(AGG_E_ARG, "unknown producer kind %d", kind);
  if (copy_wgs < 0 || piece_kib < 0) return fail(AGG_E_ARG, "negative copy_wgs or piece_kib");
  ctx->producer = kind;
  ctx->copy_wgs = copy_wgs;
  ctx->piece_bytes = piece_kib > 0 ? int64_t(piece_kib) << 10 : 0;
  return AGG_OK;
}

extern "C" int agg_ctx_last_producer(const agg_ctx* ctx, int* kind) {
  clear_error();
  if (!ctx || !kind) return fail(AGG_E_ARG, "ctx or kind is NULL");
  *kind = ctx->last_producer;
  return AGG_OK;
}

extern "C" int agg_ctx_set_pull(agg_ctx* ctx, int pull) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (pull < AGG_PULL_AUTO || pull > AGG_PULL_ON) return fail(AGG_E_ARG, "unknown pull mode %d", pull);
  ctx->pull = pull;
  return AGG_OK;
}

extern "C" int agg_ctx_set_split(agg_ctx* ctx, int ksplit) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (ksplit < 0 || ksplit > kMaxKSplit) return fail(AGG_E_ARG, "ksplit must be in [0, %d]", kMaxKSplit);
  ctx->force_split = ksplit;
  return AGG_OK;
}

extern "C" int agg_ctx_set_tail(agg_ctx* ctx, int mode) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (mode != AGG_TAIL_AUTO && mode != AGG_TAIL_OFF && mode != AGG_TAIL_ON)
    return fail(AGG_E_ARG, "unknown tail mode %d", mode);
  ctx->tail = mode;
  return AGG_OK;
}

extern "C" int agg_ctx_set_lists(agg_ctx* ctx, int lists, int list_cols) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (lists < 1 || lists > kMaxLists) return fail(AGG_E_ARG, "lists must be in [1, %d]", kMaxLists);
  if (list_cols < 0 || (list_cols > 0 && lists % list_cols != 0))
    return fail(AGG_E_ARG, "list_cols (%d) must be 0 or divide lists (%d)", list_cols, lists);
  ctx->lists = lists;
  ctx->list_cols = list_cols;
  return AGG_OK;
}

extern "C" int agg_ctx_set_reserved_cus(agg_ctx* ctx, int n) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (n < 0 || n >= ctx->cus) return fail(AGG_E_ARG, "reserved CUs must be in [0, %d)", ctx->cus);
  ctx->reserved_cus = n;
  return AGG_OK;
}

extern "C" int agg_ctx_set_copy_streams(agg_ctx* ctx, int n) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (n < 1 || n > kMaxCopyStreams) return fail(AGG_E_ARG, "copy streams must be in [1, %d]", kMaxCopyStreams);
  ctx->n_copy = n;
  return AGG_OK;
}

extern "C" int agg_ctx_set_timing(agg_ctx* ctx, int every) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (every < 0) return fail(AGG_E_ARG, "timing interval %d is negative", every);
  if (every && !ctx->ev_t0[0]) {
    HIP_TRY(hipSetDevice(ctx->device));
    for (int j = 0; j < kTimingRing; ++j) {
      HIP_TRY(hipEventCreate(&ctx->ev_t0[j]));
      HIP_TRY(hipEventCreate(&ctx->ev_t1[j]));
    }
  }
  ctx->timing_every = every;
  ctx->calls = 0;
  ctx->launches = 0;
  return AGG_OK;
}

extern "C" int agg_ctx_kernel_times(agg_ctx* ctx, float* ms, int max, int* n) {
  clear_error();
  if (!ctx || !n || (max > 0 && !ms)) return fail(AGG_E_ARG, "NULL argument");
  if (!ctx->timing_every) return fail(AGG_E_STATE, "timing is off (agg_ctx_set_timing)");
  HIP_TRY(hipSetDevice(ctx->device));
  const uint64_t have = std::min<uint64_t>(ctx->launches, kTimingRing);
  const int count = int(std::min<uint64_t>(have, uint64_t(std::max(max, 0))));
  for (int i = 0; i < count; ++i) {
    const int slot = int((ctx->launches - uint64_t(count) + uint64_t(i)) % kTimingRing);
    HIP_TRY(hipEventSynchronize(ctx->ev_t1[slot]));
    HIP_TRY(hipEventElapsedTime(&ms[i], ctx->ev_t0[slot], ctx->ev_t1[slot]));
  }
  *n = count;
  return AGG_OK;
}

extern "C" int agg_set_trace(agg_ctx* ctx, void* dev_buf, size_t bytes) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (dev_buf && (reinterpret_cast<uintptr_t>(dev_buf) & 3u)) return fail(AGG_E_ARG, "trace buffer not 4-byte aligned");
  ctx->trace = bytes >= 32 ? static_cast<uint32_t*>(dev_buf) : nullptr;
  ctx->trace_bytes = ctx->trace ? bytes : 0;
  return AGG_OK;
}

extern "C" int agg_put_signal(void* dst, const void* src, size_t bytes, uint32_t* flag, uint32_t value,
                              agg_stream copy_stream) {
  clear_error();
  if (!flag || (bytes && (!dst || !src))) return fail(AGG_E_ARG, "NULL argument");
  if (reinterpret_cast<uintptr_t>(flag) & 3u) return fail(AGG_E_ARG, "flag not 4-byte aligned");
  return put_signal(dst, src, bytes, flag, value, S(copy_stream));
}

// ------------------------------------------------------------------------------------------
// AllGather + GEMM
// ------------------------------------------------------------------------------------------

namespace {

// ag_gemm and ag_gemm_noalloc: the same call on the ctx's own scratch (noalloc false) or on the
// device's static array, without any allocation (noalloc true).
// AllGather+GEMM, and (with `counts`) AllToAll+GEMM: the same path over slots that hold only
// their first counts[p] rows.
int ag_gemm_impl(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t n, int64_t k,
                 int chunk_rows, int dtype, float scale_a, float scale_b,
                 const void* const* peer_src, void* gather, uint32_t* flags, const void* b, void* c,
                 const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                 agg_stream stream, agg_stream copy_stream, bool noalloc, const int32_t* counts = nullptr) {
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (counts) {
    if (int rc = agg_check_a2a_args(world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, counts,
                                    peer_src, gather, flags, b, c, order, n_order, mode, stream, copy_stream))
      return rc;
  } else if (int rc = agg_check_ag_args(world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b,
                                        peer_src, gather, flags, b, c, order, n_order, mode, stream,
                                        copy_stream)) {
    return rc;
  }
  if (noalloc && ctx->producer != AGG_PRODUCER_CU)
    return fail(AGG_E_STATE, "ag_gemm_noalloc runs the in-kernel producer only (agg_ctx_set_producer)");
  const Scratch sp = noalloc ? static_scratch(ctx->device) : own_scratch(ctx);
  if (!sp.words) return fail(AGG_E_STATE, "no static scratch on device %d", ctx->device);
  const int64_t m = int64_t(world) * m_shard;
  if (m == 0) return AGG_OK;
  const TileShape ts = tile_for(ctx, 0, dtype, m, n, k);
  if ((m + ts.bm - 1) / ts.bm > AGG_MAX_ROW_TILES)
    return fail(AGG_E_UNSUPPORTED, "%lld row tiles exceed %d", (long long)((m + ts.bm - 1) / ts.bm), AGG_MAX_ROW_TILES);
  HIP_TRY(hipSetDevice(ctx->device));
  const int cps = int(m_shard / chunk_rows);
  if (world > 1)
    if (int rc = bind_flags(ctx, kFlagsAg, flags, size_t(world) * cps)) return rc;
  std::vector<int32_t> ord = order ? std::vector<int32_t>(order, order + n_order) : ring_order(world, rank, cps);
  std::vector<uint32_t> delays_held;
  if (counts) {
    // chunks that hold no row go first (their copies are empty: only the flag is raised), the
    // others keep their order; delays stay with their chunks
    std::vector<int32_t> first, rest;
    std::vector<uint32_t> dfirst, drest;
    for (size_t i = 0; i < ord.size(); ++i) {
      const int32_t ch = ord[i];
      const bool holds = int64_t(ch % cps) * chunk_rows < counts[ch / cps];
      (holds ? rest : first).push_back(ch);
      if (delay_us) (holds ? drest : dfirst).push_back(delay_us[i]);
    }
    first.insert(first.end(), rest.begin(), rest.end());
    ord.swap(first);
    if (delay_us) {
      dfirst.insert(dfirst.end(), drest.begin(), drest.end());
      delays_held.swap(dfirst);
      delay_us = delays_held.data();
    }
  }
  hipStream_t s = S(stream);
  const std::vector<int32_t> rows =
      (mode != AGG_COPY_ONLY && n > 0) ? ag_row_tile_order(world, rank, m_shard, chunk_rows, ord, ts.bm, counts)
                                       : std::vector<int32_t>();
  const bool kernel = !rows.empty();
  const bool chunks = (mode != AGG_GEMM_ONLY) && world > 1;
  const int prod = effective_producer(ctx, ts, dtype, kEpiAllGather, delay_us != nullptr);
  ctx->last_producer = prod;
  const bool cu = prod == AGG_PRODUCER_CU;
  std::vector<hipStream_t> cstreams;
  if (chunks && !cu)
    if (int rc = copy_streams(ctx, prod == AGG_PRODUCER_SDMA ? ord.size() : 1, cstreams)) return rc;
  uint32_t epoch = ctx->epoch;
  if (chunks)
    if (int rc = next_epoch(ctx, s, &epoch)) return rc;

  ChunkCopy cc;
  cc.src = reinterpret_cast<const uint8_t* const*>(peer_src);
  cc.dst = static_cast<uint8_t*>(gather);
  cc.slot_rows = m_shard;
  cc.cr = chunk_rows;
  cc.row_bytes = k * elem_bytes(dtype);
  cc.cps = cps;
  cc.valid_rows = counts;

  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.scratch = sp.words;
  int64_t tiles = 0;
  int grid = 1;
  if (kernel) {
    g.a = static_cast<const uint8_t*>(gather);
    g.b = static_cast<const uint8_t*>(b);
    g.c = static_cast<uint16_t*>(c);
    g.flags = flags;
    g.M = m;
    g.N = n;
    g.K = k;
    g.world = world;
    g.rank = rank;
    g.chunk_rows = chunk_rows;
    g.cps = cps;
    g.n_row_tiles = int(rows.size());
    g.n_col_tiles = int((n + ts.bn - 1) / ts.bn);
    const KSplit ks = ksplit_for(ctx, ts, dtype, int64_t(g.n_row_tiles) * g.n_col_tiles, k);
    if (ks.ksplit > 1) {
      // the kernel's slice-pair pipeline starts every part on a whole pair
      if (ks.kps & 1) return fail(AGG_E_STATE, "split-K part of %d slices (must be even)", ks.kps);
      if (int64_t(g.n_row_tiles) * g.n_col_tiles > kMaxSplitTiles)
        return fail(AGG_E_UNSUPPORTED, "split-K over more than %d tiles", kMaxSplitTiles);
      const size_t ws_bytes = size_t(ks.ksplit) * size_t(m) * size_t(n) * sizeof(float);
      if (ws_bytes >= (size_t(1) << 31)) return fail(AGG_E_UNSUPPORTED, "split-K partials exceed 2 GiB");
      if (sp.fixed) {
        if (ws_bytes > kStaticWsBytes)
          return fail(AGG_E_UNSUPPORTED, "ag_gemm_noalloc: split-K partials of %zu bytes exceed its %zu-byte scratch",
                      ws_bytes, kStaticWsBytes);
        g.ws = reinterpret_cast<float*>(sp.words + kStaticWords);
      } else {
        if (int rc = ensure_ws(ctx, ws_bytes)) return rc;
        g.ws = ctx->ws;
      }
    }
    g.ksplit = ks.ksplit;
    g.kps = ks.kps;
    g.n_col_tiles *= ks.ksplit;
    g.epoch = world > 1 ? epoch : 0;
    g.concurrent_producer = (mode == AGG_OVERLAP && chunks) ? 1 : 0;
    g.scale = dtype == AGG_FP8_E4M3 ? scale_a * scale_b : 1.0f;
    tiles = int64_t(g.n_row_tiles) * g.n_col_tiles;
    grid = grid_for(ctx, tiles, mode == AGG_OVERLAP && chunks && prod == AGG_PRODUCER_SDMA);
    // every split part claims its workgroup at launch (no more parts than workgroups): the parts
    // of a tile can wait for each other and sum the tile together
    // (and only when the whole grid fits on the GPU at once, so that no part waits for a sibling
    // that has no CU)
    g.split_together = (g.ksplit > 1 && tiles <= grid &&
                        int64_t(max_blocks_per_cu(ts.bm, ts.bn, dtype, kEpiAllGather)) * ctx->cus >= grid)
                           ? 1 : 0;
    fill_common(ctx, g, ts, grid);
    attach_trace(ctx, g, tiles);
  }
  if (noalloc) ctx->used_static = true;
  if (!cu && kernel)
    if (int rc = upload_rows(ctx, sp, s, rows)) return rc;
  if (cu) {
    if (chunks)
      if (int rc = upload_schedule(ctx, sp, s, ord, delay_us)) return rc;
    // pull: an overlapped call whose row tiles each lie inside one shard, with compute units to
    // spare for the copiers, reads the remote rows straight from the peers' blocks (automatic
    // for small gathers, where the chunk copy's latency would otherwise be exposed)
    int pull_copiers = 0;
    if (kernel && chunks && mode == AGG_OVERLAP && ctx->pull != AGG_PULL_OFF && delay_us == nullptr && !counts &&
        (m_shard % ts.bm == 0 || (ts.bm <= 128 && m_shard % 16 == 0))) {
      const int64_t remote = int64_t(world - 1) * m_shard * cc.row_bytes;
      const int64_t spare = int64_t(ctx->cus) - grid;
      if (spare >= 1 && (ctx->pull == AGG_PULL_ON || remote <= kPullMaxBytes))
        pull_copiers = int(std::min<int64_t>(spare, std::max<int64_t>(1, (remote + 16383) / 16384)));
    }
    // tail split: the row tiles of the whole waves in this launch, the rest cut into the next
    // smaller shape in a second launch right after it (after the copy jobs, which the first
    // launch carries, have all completed). Both launches' row tiles share one order table.
    std::vector<int32_t> table = rows;
    GemmArgs g2;
    TailLaunch tl;
    if (kernel && pull_copiers == 0 && g.ksplit == 1 && !ctx->trace && ctx->tail != AGG_TAIL_OFF) {
      const TailSplit plan2 = tail_split(ts, m, n, int(rows.size()), ctx->cus, ctx->tail);
      if (plan2.head_rows > 0) {
        const TileShape ts2 = plan2.tail;
        const int sub = ts.bm / ts2.bm;
        const int64_t row_tiles2 = (m + ts2.bm - 1) / ts2.bm;
        std::vector<int32_t> rows2;
        for (size_t i = size_t(plan2.head_rows); i < rows.size(); ++i)
          for (int j = 0; j < sub; ++j) {
            const int64_t r2 = int64_t(rows[i]) * sub + j;
            if (r2 < row_tiles2) rows2.push_back(int32_t(r2));
          }
        if (!rows2.empty() && size_t(plan2.head_rows) + rows2.size() <= size_t(AGG_MAX_ROW_TILES)) {
          g2 = g;
          g2.n_row_tiles = int(rows2.size());
          g2.row_base = plan2.head_rows;
          g2.n_col_tiles = int((n + ts2.bn - 1) / ts2.bn);
          g2.concurrent_producer = 0;
          g2.trace = nullptr;
          g2.trace_tiles = 0;
          const int grid2 = grid_for(ctx, int64_t(g2.n_row_tiles) * g2.n_col_tiles, false);
          fill_common(ctx, g2, ts2, grid2);
          g.n_row_tiles = plan2.head_rows;
          grid = grid_for(ctx, int64_t(g.n_row_tiles) * g.n_col_tiles, false);
          fill_common(ctx, g, ts, grid);
          table.resize(size_t(plan2.head_rows));
          table.insert(table.end(), rows2.begin(), rows2.end());
          tl.g = &g2;
          tl.ts = ts2;
          tl.grid = grid2;
        }
      }
    }
    // small pushed gathers with compute units to spare: the copies on workgroups of their own
    // after the tile workgroups (which then start their tiles, local chunks first, at once)
    int last_copiers = 0;
    if (kernel && chunks && mode == AGG_OVERLAP && pull_copiers == 0 && !tl.g && delay_us == nullptr) {
      const int64_t remote = int64_t(world - 1) * m_shard * cc.row_bytes;
      const int64_t spare = int64_t(ctx->cus) - grid;
      if (spare >= 1 && remote <= kPullMaxBytes && ctx->copy_wgs == 0)
        last_copiers = int(std::min<int64_t>(spare, std::max<int64_t>(1, (remote + 65535) / 65536)));
    }
    if (kernel)
      if (int rc = upload_rows(ctx, sp, s, table)) return rc;
    Marks marks;
    if (world > 1) {
      marks.copy_flags[0] = flags + size_t(rank) * cps;
      marks.copy_count[0] = cps;
    }
    const CopyPlan plan{cc, flags, ord.size()};
    return schedule_cu(ctx, mode, s, S(copy_stream), kernel, chunks,
                       [&](bool copies, bool tiles_on, bool timed) {
                         return launch_cu(ctx, s, g, ts, dtype, kEpiAllGather, grid, &plan, 1,
                                          delay_us != nullptr, world, epoch, copies, tiles_on,
                                          timed, marks, pull_copiers, tl, last_copiers);
                       });
  }
  // the copy engines' producer keeps the kernel on a queue of its own (see the top of this
  // file); beside the copy kernel it runs on the caller's stream where that stream allows it
  // (no fork and join of the kernel's queue)
  hipStream_t ls = prod == AGG_PRODUCER_KERNEL && own_queue_free(s) ? s : ctx->ks;
  auto launch = [&]() -> int {
    return timed_launch(ctx, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm(g, ts.bm, ts.bn, dtype, kEpiAllGather, grid, ls, t0, t1);
    });
  };
  const CopyPlan kplan{cc, flags, ord.size()};
  Marks kmarks;
  if (world > 1) {
    kmarks.copy_flags[0] = flags + size_t(rank) * cps;
    kmarks.copy_count[0] = cps;
  }
  if (prod == AGG_PRODUCER_KERNEL && chunks)
    if (int rc = upload_schedule(ctx, sp, s, ord, nullptr)) return rc;
  return schedule(ctx, mode, s, S(copy_stream), cstreams, kernel, launch, chunks, [&]() -> int {
    if (prod == AGG_PRODUCER_KERNEL)
      return launch_copy_producer(ctx, sp.words, &kplan, 1, world, epoch, kmarks, cstreams[0]);
    return produce(cc, flags, ord, delay_us, epoch, cstreams, rank);
  }, ls);
}

}  // namespace

extern "C" int ag_gemm(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t n, int64_t k,
                       int chunk_rows, int dtype, float scale_a, float scale_b,
                       const void* const* peer_src, void* gather, uint32_t* flags, const void* b, void* c,
                       const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                       agg_stream stream, agg_stream copy_stream) {
  return ag_gemm_impl(ctx, world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
                      gather, flags, b, c, order, n_order, delay_us, mode, stream, copy_stream, false);
}

extern "C" int ag_gemm_noalloc(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t n, int64_t k,
                               int chunk_rows, int dtype, float scale_a, float scale_b,
                               const void* const* peer_src, void* gather, uint32_t* flags, const void* b,
                               void* c, const int32_t* order, int n_order, const uint32_t* delay_us,
                               int mode, agg_stream stream, agg_stream copy_stream) {
  return ag_gemm_impl(ctx, world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
                      gather, flags, b, c, order, n_order, delay_us, mode, stream, copy_stream, true);
}

extern "C" int a2a_gemm(agg_ctx* ctx, int world, int rank, int64_t cap, int64_t n, int64_t k, int chunk_rows,
                        int dtype, float scale_a, float scale_b, const int32_t* counts,
                        const void* const* peer_src, void* recv, uint32_t* flags, const void* b, void* c,
                        const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                        agg_stream stream, agg_stream copy_stream) {
  if (!counts) return fail(AGG_E_ARG, "counts is NULL");
  return ag_gemm_impl(ctx, world, rank, cap, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src, recv,
                      flags, b, c, order, n_order, delay_us, mode, stream, copy_stream, false, counts);
}

// ------------------------------------------------------------------------------------------
// GEMM + ReduceScatter
// ------------------------------------------------------------------------------------------

extern "C" int gemm_rs(agg_ctx* ctx, int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                       const void* a, const void* b, float* send, uint32_t* send_flags,
                       const float* const* peer_src, float* recv, uint32_t* flags, float* out,
                       const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                       agg_stream stream, agg_stream copy_stream) {
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (int rc = agg_check_rs_args(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src,
                                 recv, flags, out, order, n_order, mode, stream, copy_stream))
    return rc;
  const int64_t mb = m / world;
  if (mb == 0 || n == 0) return AGG_OK;
  const TileShape ts = tile_for(ctx, 1, AGG_BF16, m, n, k);
  if (world * ((mb + ts.bm - 1) / ts.bm) > AGG_MAX_ROW_TILES)
    return fail(AGG_E_UNSUPPORTED, "row tiles exceed %d", AGG_MAX_ROW_TILES);
  HIP_TRY(hipSetDevice(ctx->device));
  const int cpb = int(mb / chunk_rows);
  if (world > 1) {
    if (int rc = bind_flags(ctx, kFlagsRsRecv, flags, size_t(world) * cpb)) return rc;
    if (int rc = bind_flags(ctx, kFlagsRsSend, send_flags, size_t(world) * cpb)) return rc;
  }
  const std::vector<int32_t> ord = order ? std::vector<int32_t>(order, order + n_order) : ring_order(world, rank, cpb);
  hipStream_t s = S(stream);
  const bool kernel = mode != AGG_COPY_ONLY;
  const bool chunks = (mode != AGG_GEMM_ONLY) && world > 1;
  const int prod = effective_producer(ctx, ts, AGG_BF16, kEpiReduceScatter, delay_us != nullptr);
  ctx->last_producer = prod;
  const bool cu = prod == AGG_PRODUCER_CU;
  std::vector<hipStream_t> cstreams;
  if (chunks && !cu)
    if (int rc = copy_streams(ctx, prod == AGG_PRODUCER_SDMA ? ord.size() : 1, cstreams)) return rc;
  uint32_t epoch = ctx->epoch;
  if (chunks)
    if (int rc = next_epoch(ctx, s, &epoch)) return rc;

  ChunkCopy cc;
  cc.src = reinterpret_cast<const uint8_t* const*>(peer_src);
  cc.dst = reinterpret_cast<uint8_t*>(recv);
  cc.slot_rows = mb;
  cc.cr = chunk_rows;
  cc.row_bytes = n * 4;
  cc.cps = cpb;

  const Scratch sp = own_scratch(ctx);
  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.scratch = sp.words;
  int64_t tiles = 0;
  int grid = 1;
  if (kernel) {
    const std::vector<int32_t> rows = rs_row_tile_order(world, rank, m, chunk_rows, ord, ts.bm);
    if (int rc = upload_rows(ctx, sp, s, rows)) return rc;
    g.a = static_cast<const uint8_t*>(a);
    g.b = static_cast<const uint8_t*>(b);
    g.send = send;
    g.out = out;
    g.recv = recv;
    g.flags = flags;
    g.send_flags = send_flags;
    g.M = m;
    g.N = n;
    g.K = k;
    g.m_block = mb;
    g.world = world;
    g.rank = rank;
    g.chunk_rows = chunk_rows;
    g.cps = cpb;
    g.tpb = int((mb + ts.bm - 1) / ts.bm);
    g.n_row_tiles = int(rows.size());
    g.n_col_tiles = int((n + ts.bn - 1) / ts.bn);
    g.ksplit = 1;
    g.kps = int(std::max<int64_t>(1, (k * 2 + slice_bytes(AGG_BF16) - 1) / slice_bytes(AGG_BF16)));
    g.epoch = world > 1 ? epoch : 0;
    g.scale = 1.0f;
    tiles = int64_t(g.n_row_tiles) * g.n_col_tiles;
    grid = grid_for(ctx, tiles, mode == AGG_OVERLAP && chunks && prod == AGG_PRODUCER_SDMA);
    // the local block's tiles reduce it themselves (no round trip of its partial through `out`)
    // when they are at least half the grid: fewer of them would leave the HBM-bound reduction to
    // a few compute units, where the grid-wide reduction after the tiles spreads it over all
    g.fuse_local = (world > 1 && int64_t(g.tpb) * g.n_col_tiles * 2 >= grid) ? 1 : 0;
    fill_common(ctx, g, ts, grid);
    attach_trace(ctx, g, tiles);
    if (world > 1) {
      // nothing is sent for the local block: its send flags are raised with the others' epoch
      g.mark_flags[2] = send_flags + size_t(rank) * cpb;
      g.mark_count[2] = cpb;
    }
  }
  if (cu) {
    if (chunks)
      if (int rc = upload_schedule(ctx, sp, s, ord, delay_us)) return rc;
    Marks marks;
    if (world > 1) {
      marks.copy_flags[0] = flags + size_t(rank) * cpb;
      marks.copy_count[0] = cpb;
      marks.tile_flags = send_flags + size_t(rank) * cpb;
      marks.tile_count = cpb;
    }
    const CopyPlan plan{cc, flags, ord.size()};
    return schedule_cu(ctx, mode, s, S(copy_stream), kernel, chunks,
                       [&](bool copies, bool tiles_on, bool timed) {
                         return launch_cu(ctx, s, g, ts, AGG_BF16, kEpiReduceScatter, grid, &plan, 1,
                                          delay_us != nullptr, world, epoch, copies, tiles_on, timed,
                                          marks);
                       });
  }
  hipStream_t ls = prod == AGG_PRODUCER_KERNEL && own_queue_free(s) ? s : ctx->ks;
  auto launch = [&]() -> int {
    return timed_launch(ctx, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm(g, ts.bm, ts.bn, AGG_BF16, kEpiReduceScatter, grid, ls, t0, t1);
    });
  };
  const CopyPlan kplan{cc, flags, ord.size()};
  Marks kmarks;
  if (world > 1) {
    kmarks.copy_flags[0] = flags + size_t(rank) * cpb;
    kmarks.copy_count[0] = cpb;
  }
  if (prod == AGG_PRODUCER_KERNEL && chunks)
    if (int rc = upload_schedule(ctx, sp, s, ord, nullptr)) return rc;
  return schedule(ctx, mode, s, S(copy_stream), cstreams, kernel, launch, chunks, [&]() -> int {
    if (prod == AGG_PRODUCER_KERNEL)
      return launch_copy_producer(ctx, sp.words, &kplan, 1, world, epoch, kmarks, cstreams[0]);
    return produce(cc, flags, ord, delay_us, epoch, cstreams, rank);
  }, ls);
}

// ------------------------------------------------------------------------------------------
// GEMM + AllReduce
// ------------------------------------------------------------------------------------------

extern "C" int gemm_ar(agg_ctx* ctx, int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                       const void* a, const void* b, float* send, uint32_t* send_flags,
                       const float* const* peer_src, float* recv, uint32_t* flags, float* out,
                       const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                       agg_stream stream, agg_stream copy_stream) {
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  if (int rc = agg_check_ar_args(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src,
                                 recv, flags, out, order, n_order, mode, stream, copy_stream))
    return rc;
  if (m == 0 || n == 0) return AGG_OK;
  const TileShape ts = tile_for(ctx, 2, AGG_BF16, m, n, k);
  if ((m + ts.bm - 1) / ts.bm > AGG_MAX_ROW_TILES) return fail(AGG_E_UNSUPPORTED, "row tiles exceed %d", AGG_MAX_ROW_TILES);
  HIP_TRY(hipSetDevice(ctx->device));
  const int cpb = int(m / chunk_rows);
  if (world > 1) {
    if (int rc = bind_flags(ctx, kFlagsArRecv, flags, size_t(world) * cpb)) return rc;
    if (int rc = bind_flags(ctx, kFlagsArSend, send_flags, size_t(cpb))) return rc;
  }
  const std::vector<int32_t> ord = order ? std::vector<int32_t>(order, order + n_order) : ring_order(world, rank, cpb);
  hipStream_t s = S(stream);
  const bool kernel = mode != AGG_COPY_ONLY;
  const bool chunks = (mode != AGG_GEMM_ONLY) && world > 1;
  const int prod = effective_producer(ctx, ts, AGG_BF16, kEpiAllReduce, delay_us != nullptr);
  ctx->last_producer = prod;
  const bool cu = prod == AGG_PRODUCER_CU;
  std::vector<hipStream_t> cstreams;
  if (chunks && !cu)
    if (int rc = copy_streams(ctx, prod == AGG_PRODUCER_SDMA ? ord.size() : 1, cstreams)) return rc;
  uint32_t epoch = ctx->epoch;
  if (chunks)
    if (int rc = next_epoch(ctx, s, &epoch)) return rc;

  // chunk q of peer p: rows [q*cr, (q+1)*cr) of its M x N partial, into receive slot p
  ChunkCopy cc;
  cc.src = reinterpret_cast<const uint8_t* const*>(peer_src);
  cc.dst = reinterpret_cast<uint8_t*>(recv);
  cc.slot_rows = m;
  cc.cr = chunk_rows;
  cc.row_bytes = n * 4;
  cc.cps = cpb;

  const Scratch sp = own_scratch(ctx);
  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.scratch = sp.words;
  int grid = 1;
  if (kernel) {
    // every tile reduces every peer's rows: plain ascending row tiles
    std::vector<int32_t> rows(size_t((m + ts.bm - 1) / ts.bm));
    for (size_t i = 0; i < rows.size(); ++i) rows[i] = int32_t(i);
    if (int rc = upload_rows(ctx, sp, s, rows)) return rc;
    g.a = static_cast<const uint8_t*>(a);
    g.b = static_cast<const uint8_t*>(b);
    g.send = send;
    g.out = out;
    g.recv = recv;
    g.flags = flags;
    g.send_flags = send_flags;
    g.M = m;
    g.N = n;
    g.K = k;
    g.m_block = m;
    g.world = world;
    g.rank = rank;
    g.chunk_rows = chunk_rows;
    g.cps = cpb;
    g.n_row_tiles = int(rows.size());
    g.n_col_tiles = int((n + ts.bn - 1) / ts.bn);
    g.ksplit = 1;
    g.kps = int(std::max<int64_t>(1, (k * 2 + slice_bytes(AGG_BF16) - 1) / slice_bytes(AGG_BF16)));
    g.epoch = world > 1 ? epoch : 0;
    g.scale = 1.0f;
    const int64_t tiles = int64_t(g.n_row_tiles) * g.n_col_tiles;
    grid = grid_for(ctx, tiles, mode == AGG_OVERLAP && chunks && prod == AGG_PRODUCER_SDMA);
    fill_common(ctx, g, ts, grid);
    attach_trace(ctx, g, tiles);
  }
  if (cu) {
    if (chunks)
      if (int rc = upload_schedule(ctx, sp, s, ord, delay_us)) return rc;
    Marks marks;
    if (world > 1) {
      marks.copy_flags[0] = flags + size_t(rank) * cpb;   // nothing arrives for this rank's own slot
      marks.copy_count[0] = cpb;
    }
    const CopyPlan plan{cc, flags, ord.size()};
    return schedule_cu(ctx, mode, s, S(copy_stream), kernel, chunks,
                       [&](bool copies, bool tiles_on, bool timed) {
                         return launch_cu(ctx, s, g, ts, AGG_BF16, kEpiAllReduce, grid, &plan, 1,
                                          delay_us != nullptr, world, epoch, copies, tiles_on, timed,
                                          marks);
                       });
  }
  hipStream_t ls = prod == AGG_PRODUCER_KERNEL && own_queue_free(s) ? s : ctx->ks;
  auto launch = [&]() -> int {
    return timed_launch(ctx, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm(g, ts.bm, ts.bn, AGG_BF16, kEpiAllReduce, grid, ls, t0, t1);
    });
  };
  const CopyPlan kplan{cc, flags, ord.size()};
  Marks kmarks;
  if (world > 1) {
    kmarks.copy_flags[0] = flags + size_t(rank) * cpb;
    kmarks.copy_count[0] = cpb;
  }
  if (prod == AGG_PRODUCER_KERNEL && chunks)
    if (int rc = upload_schedule(ctx, sp, s, ord, nullptr)) return rc;
  return schedule(ctx, mode, s, S(copy_stream), cstreams, kernel, launch, chunks, [&]() -> int {
    if (prod == AGG_PRODUCER_KERNEL)
      return launch_copy_producer(ctx, sp.words, &kplan, 1, world, epoch, kmarks, cstreams[0]);
    return produce(cc, flags, ord, delay_us, epoch, cstreams, rank);
  }, ls);
}

// ------------------------------------------------------------------------------------------
// The FFN chain: AllGather+GEMM -> SiLU -> GEMM+ReduceScatter
// ------------------------------------------------------------------------------------------

extern "C" int agg_ctx_set_chain_fused(agg_ctx* ctx, int on) {
  clear_error();
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  ctx->chain_fused = on != 0;
  return AGG_OK;
}

extern "C" int ffn_chain(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t k1, int64_t n1,
                         int64_t n2, int chunk_rows, int rs_chunk_rows, const void* const* peer_src,
                         void* gather, uint32_t* flags, const void* w1, void* h, const void* w2,
                         float* send, uint32_t* send_flags, const float* const* rs_peer_src, float* recv,
                         uint32_t* rs_flags, float* out, const int32_t* order, int n_order,
                         const int32_t* rs_order, int n_rs_order, int mode, agg_stream stream,
                         agg_stream copy_stream) {
  if (!ctx) return fail(AGG_E_ARG, "ctx is NULL");
  const int64_t m = int64_t(world) * m_shard;
  // the two layers' arguments, each checked as the operation it is
  if (int rc = agg_check_ag_args(world, rank, m_shard, n1, k1, chunk_rows, AGG_BF16, 1.0f, 1.0f, peer_src,
                                 gather, flags, w1, h, order, n_order, mode, stream, copy_stream))
    return rc;
  if (int rc = agg_check_rs_args(world, rank, m, n2, n1, rs_chunk_rows, h, w2, send, send_flags,
                                 rs_peer_src, recv, rs_flags, out, rs_order, n_rs_order, mode, stream,
                                 copy_stream))
    return rc;
  const int cps = int(m_shard / chunk_rows), cpb = int(m_shard / rs_chunk_rows);
  if (world * cps > AGG_MAX_CHUNKS / 2 || world * cpb > AGG_MAX_CHUNKS / 2)
    return fail(AGG_E_UNSUPPORTED, "each layer's chunks must stay within %d", AGG_MAX_CHUNKS / 2);
  if (m == 0 || n1 == 0 || n2 == 0) return AGG_OK;
  const TileShape ts{256, 256};
  if ((m + ts.bm - 1) / ts.bm * 2 + world > AGG_MAX_ROW_TILES)
    return fail(AGG_E_UNSUPPORTED, "row tiles exceed %d", AGG_MAX_ROW_TILES);
  HIP_TRY(hipSetDevice(ctx->device));
  if (world > 1) {
    if (int rc = bind_flags(ctx, kFlagsAg, flags, size_t(world) * cps)) return rc;
    if (int rc = bind_flags(ctx, kFlagsRsRecv, rs_flags, size_t(world) * cpb)) return rc;
    if (int rc = bind_flags(ctx, kFlagsRsSend, send_flags, size_t(world) * cpb)) return rc;
  }
  const std::vector<int32_t> ord = order ? std::vector<int32_t>(order, order + n_order) : ring_order(world, rank, cps);
  const std::vector<int32_t> ord2 =
      rs_order ? std::vector<int32_t>(rs_order, rs_order + n_rs_order) : ring_order(world, rank, cpb);
  hipStream_t s = S(stream);
  const bool kernel = mode != AGG_COPY_ONLY;
  const bool chunks = (mode != AGG_GEMM_ONLY) && world > 1;
  const int prod = effective_producer(ctx, ts, AGG_BF16, kEpiFfn, false);
  ctx->last_producer = prod;
  const bool cu = prod == AGG_PRODUCER_CU;
  std::vector<hipStream_t> cstreams;
  if (chunks && !cu)
    if (int rc = copy_streams(ctx, prod == AGG_PRODUCER_SDMA ? ord.size() + ord2.size() : 1, cstreams)) return rc;
  uint32_t epoch = ctx->epoch;
  if (chunks)
    if (int rc = next_epoch(ctx, s, &epoch)) return rc;

  CopyPlan plans[2];
  plans[0].cc = ChunkCopy{reinterpret_cast<const uint8_t* const*>(peer_src), static_cast<uint8_t*>(gather),
                          m_shard, chunk_rows, k1 * 2, cps};
  plans[0].flags = flags;
  plans[0].n_order = ord.size();
  plans[1].cc = ChunkCopy{reinterpret_cast<const uint8_t* const*>(rs_peer_src), reinterpret_cast<uint8_t*>(recv),
                          m_shard, rs_chunk_rows, n2 * 4, cpb};
  plans[1].flags = rs_flags;
  plans[1].n_order = ord2.size();

  const Scratch sp = own_scratch(ctx);
  GemmArgs g;
  std::memset(&g, 0, sizeof g);
  g.scratch = sp.words;
  int grid = 1;
  if (kernel) {
    // phase 1's row tiles in arrival order, then phase 2's in ReduceScatter order
    const std::vector<int32_t> rows1 = ag_row_tile_order(world, rank, m_shard, chunk_rows, ord, ts.bm);
    const std::vector<int32_t> rows2 = rs_row_tile_order(world, rank, m, rs_chunk_rows, ord2, ts.bm);
    std::vector<int32_t> rows(rows1);
    rows.insert(rows.end(), rows2.begin(), rows2.end());
    if (int rc = upload_rows(ctx, sp, s, rows)) return rc;
    // phase 2: GEMM+ReduceScatter of h
    g.a = static_cast<const uint8_t*>(h);
    g.b = static_cast<const uint8_t*>(w2);
    g.send = send;
    g.out = out;
    g.recv = recv;
    g.flags = rs_flags;
    g.send_flags = send_flags;
    g.M = m;
    g.N = n2;
    g.K = n1;
    g.m_block = m_shard;
    g.world = world;
    g.rank = rank;
    g.chunk_rows = rs_chunk_rows;
    g.cps = cpb;
    g.tpb = int((m_shard + ts.bm - 1) / ts.bm);
    g.n_row_tiles = int(rows2.size());
    g.n_col_tiles = int((n2 + ts.bn - 1) / ts.bn);
    // phase 1: AllGather+GEMM into h
    g.a1 = static_cast<const uint8_t*>(gather);
    g.b1 = static_cast<const uint8_t*>(w1);
    g.h = static_cast<uint16_t*>(h);
    g.flags1 = flags;
    g.K1 = k1;
    g.N1 = n1;
    g.chunk_rows1 = chunk_rows;
    g.cps1 = cps;
    g.n_row_tiles1 = int(rows1.size());
    g.n_col_tiles1 = int((n1 + ts.bn - 1) / ts.bn);
    g.ksplit = 1;
    g.kps = 1 << 28;                       // no split: every tile covers its whole K
    g.epoch = world > 1 ? epoch : 0;
    g.concurrent_producer = (mode == AGG_OVERLAP && chunks) ? 1 : 0;
    g.scale = 1.0f;
    g.n_lists = 1;
    g.list_cols = 1;
    g.timeout_ticks = uint64_t(double(ctx->timeout_us) * ctx->ticks_per_us);
    const int64_t tasks = int64_t(g.n_row_tiles1) * g.n_col_tiles1 + int64_t(g.n_row_tiles) * g.n_col_tiles;
    grid = grid_for(ctx, tasks, mode == AGG_OVERLAP && chunks && prod == AGG_PRODUCER_SDMA);
    if (world > 1) {
      g.mark_flags[2] = send_flags + size_t(rank) * cpb;   // nothing is sent for the local block
      g.mark_count[2] = cpb;
    }
  }
  // The tiles as one launch (fused) or as two: phase 1 alone, then phase 2 alone.
  auto tile_launches = [&](auto&& launch_one) -> int {
    if (ctx->chain_fused) return launch_one(g, true);
    GemmArgs g1 = g, g2 = g;
    g1.n_row_tiles = 0;                    // phase 1 only
    g2.n_row_tiles1 = 0;                   // phase 2 only: no phase-1 tile to wait for
    g2.n_col_tiles1 = 0;
    if (int rc = launch_one(g1, true)) return rc;
    return launch_one(g2, false);
  };
  if (cu) {
    if (chunks) {
      std::vector<int32_t> both(ord);
      both.insert(both.end(), ord2.begin(), ord2.end());
      if (int rc = upload_schedule(ctx, sp, s, both, nullptr)) return rc;
    }
    Marks marks;
    if (world > 1) {
      marks.copy_flags[0] = flags + size_t(rank) * cps;
      marks.copy_count[0] = cps;
      marks.copy_flags[1] = rs_flags + size_t(rank) * cpb;
      marks.copy_count[1] = cpb;
      marks.tile_flags = send_flags + size_t(rank) * cpb;
      marks.tile_count = cpb;
    }
    return schedule_cu(ctx, mode, s, S(copy_stream), kernel, chunks,
                       [&](bool copies, bool tiles_on, bool timed) {
                         if (!tiles_on)
                           return launch_cu(ctx, s, g, ts, AGG_BF16, kEpiFfn, grid, plans, 2, false, world,
                                            epoch, copies, false, timed, marks);
                         return tile_launches([&](const GemmArgs& gg, bool first) {
                           // the copies go with the first (or only) tile launch
                           return launch_cu(ctx, s, gg, ts, AGG_BF16, kEpiFfn, grid, plans, 2, false, world,
                                            epoch, copies && first, true, timed, marks);
                         });
                       });
  }
  hipStream_t ls = prod == AGG_PRODUCER_KERNEL && own_queue_free(s) ? s : ctx->ks;
  auto launch = [&]() -> int {
    return tile_launches([&](const GemmArgs& gg, bool) {
      return timed_launch(ctx, [&](hipEvent_t t0, hipEvent_t t1) {
        return launch_gemm(gg, ts.bm, ts.bn, AGG_BF16, kEpiFfn, grid, ls, t0, t1);
      });
    });
  };
  Marks kmarks;
  if (world > 1) {
    kmarks.copy_flags[0] = flags + size_t(rank) * cps;
    kmarks.copy_count[0] = cps;
    kmarks.copy_flags[1] = rs_flags + size_t(rank) * cpb;
    kmarks.copy_count[1] = cpb;
  }
  if (prod == AGG_PRODUCER_KERNEL && chunks) {
    std::vector<int32_t> both(ord);
    both.insert(both.end(), ord2.begin(), ord2.end());
    if (int rc = upload_schedule(ctx, sp, s, both, nullptr)) return rc;
  }
  return schedule(ctx, mode, s, S(copy_stream), cstreams, kernel, launch, chunks, [&]() -> int {
    if (prod == AGG_PRODUCER_KERNEL)
      return launch_copy_producer(ctx, sp.words, plans, 2, world, epoch, kmarks, cstreams[0]);
    if (int rc = produce(plans[0].cc, flags, ord, nullptr, epoch, cstreams, rank)) return rc;
    return produce(plans[1].cc, rs_flags, ord2, nullptr, epoch, cstreams, rank);
  }, ls);
}

// ------------------------------------------------------------------------------------------
// diagnostics
// ------------------------------------------------------------------------------------------

extern "C" int agg_kernel_regs(int op, int dtype, int bm, int bn, int* gemm_regs, int* copy_regs) {
  clear_error();
  if (!gemm_regs || !copy_regs) return fail(AGG_E_ARG, "NULL output");
  static const int epi[4] = {kEpiAllGather, kEpiReduceScatter, kEpiAllReduce, kEpiFfn};
  if (op < 0 || op > 3) return fail(AGG_E_ARG, "unknown op %d", op);
  *gemm_regs = kernel_regs(bm, bn, dtype, epi[op]);
  *copy_regs = copy_kernel_regs();
  if (*gemm_regs < 0) return fail(AGG_E_ARG, "no kernel for op %d dtype %d tile %dx%d", op, dtype, bm, bn);
  return AGG_OK;
}
