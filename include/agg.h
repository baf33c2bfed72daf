/*
 * agg.h — C ABI of libagg: one rank's share of an overlapped AllGather+GEMM and of a
 * GEMM+ReduceScatter on one AMD Instinct MI355X (gfx950), peers emulated on the same GPU.
 *
 * Source of the method: the page "Triton-distributed is turning communication into compiler
 * territory" (cronfeed.work), section "The first move was to expose the overlap": an AllGather
 * moves shards into place and a GEMM consumes them; serialized, the transfer stays visible; cut
 * into chunks, computation on arrived chunks proceeds while others still move; the building
 * blocks are symmetric memory, remote data access, signaling and asynchronous tasks. Section
 * "DITRON adds three levels of tiling": collectives are broken into chunks paired with
 * computation tiles, with synchronization inserted; device-level tiles are data movements on
 * DMA engines, core-level tiles live in registers, shared memory and matrix units.
 *
 * On one GPU the W-1 peers are "staging" regions in HBM. A producer moves them chunk by chunk,
 * in arrival order, into a symmetric gather buffer and after each chunk releases the call's
 * epoch into that chunk's flag word. A persistent MFMA GEMM kernel (on a ctx-owned stream with a
 * hardware queue of its own) claims output tiles in the order their chunks arrive, waits on the
 * flags each tile needs, and computes. Two producers are built (agg_ctx_set_producer):
 *  - AGG_PRODUCER_CU (default): copy workgroups inside the persistent kernel itself take the
 *    chunk copies as jobs before they turn to tiles, the communication-by-compute-units form
 *    (thread blocks dedicated to data movement) of the same overlap;
 *  - AGG_PRODUCER_SDMA: the copy engines, one hipMemcpyAsync (no CU) plus one stream write per
 *    chunk on side streams; while chunks are in flight the kernel leaves a few CUs free for the
 *    runtime's own helper kernels (agg_ctx_set_reserved_cus);
 *  - AGG_PRODUCER_KERNEL: a kernel of its own on one ctx stream, beside the persistent kernel:
 *    one-wave workgroups, each taking chunk pieces in arrival order, that fit in the registers
 *    the persistent kernel leaves free on every SIMD, so both run at once on every CU.
 *
 * Each declaration below names the passage it implements: "section ..." refers to a section of the
 * page "Triton-distributed is turning communication into compiler territory" (cronfeed.work).
 *
 * Conventions (every entry point):
 *  - Returns AGG_OK (0) or an AGG_E_* code; agg_last_error() then holds a text for the
 *    calling thread. No C++ exception crosses this boundary.
 *  - Argument checks run before anything is enqueued: a call that returns AGG_E_ARG has
 *    enqueued nothing.
 *  - All device pointers are HIP device allocations of the ctx's device; they and the streams
 *    stay owned by the caller and must outlive the enqueued work. Host arrays are read during
 *    the call only.
 *  - Streams are hipStream_t values passed as agg_stream (void*). Calls are asynchronous with
 *    respect to the host, except that a non-NULL delay_us makes the calling thread wait between
 *    chunk enqueues (a test device: it emulates late peers).
 *  - A ctx serialises its calls: use one ctx from one host thread with one main stream.
 *  - Matrix layouts are row-major: A and the gather buffer M x K (K contiguous), the weight B
 *    K x N (N contiguous), C M x N. The kernel turns B's rows into K-packed MFMA fragments with
 *    gfx950's transposing LDS reads, so no layout change is needed on either side.
 */
#ifndef AGG_H
#define AGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* agg_stream;            /* a hipStream_t */
typedef struct agg_ctx agg_ctx;

enum agg_status {
  AGG_OK = 0,
  AGG_E_ARG = 1,          /* invalid argument; nothing was enqueued */
  AGG_E_UNSUPPORTED = 2,  /* not a gfx950 device, or a size beyond a documented limit */
  AGG_E_HIP = 3,          /* a HIP runtime call failed (its text is in agg_last_error) */
  AGG_E_TIMEOUT = 4,      /* a device-side wait on a chunk flag gave up (agg_ctx_status) */
  AGG_E_STATE = 5         /* the ctx is in the wrong state for the call (see each call) */
};

enum agg_dtype {
  AGG_BF16 = 0,           /* bfloat16 operands */
  AGG_FP8_E4M3 = 1        /* OCP float8 E4M3 ("fn": max 448, no inf) operands, per-tensor scales */
};

enum agg_mode {
  AGG_OVERLAP = 0,        /* producer on copy_stream concurrent with the consumer kernel */
  AGG_SERIAL = 1,         /* all chunks copied and flagged first, then the same kernel */
  AGG_GEMM_ONLY = 2,      /* the kernel alone on already gathered data: no copy; tiles check
                             their flags against the ctx's current epoch, which the last
                             producing call left in them, so no wait lasts */
  AGG_COPY_ONLY = 3       /* the producer alone (new epoch), no kernel */
};

/* Limits. */
#define AGG_MAX_WORLD 8           /* emulated ranks */
#define AGG_MAX_ROW_TILES 1024    /* row tiles of the output per call */
#define AGG_MAX_CHUNKS 4096       /* world * chunks per shard (or per block) */

/* ---- context -------------------------------------------------------------------------- */

/* Create a ctx on HIP device `device`. Allocates the ctx's device scratch (claim counters, status
 * word, completion counters and the tables the kernel reads, 78 KiB) and pinned host staging for
 * those tables, creates its kernel stream, and, for the first ctx on a device, finds and clears
 * that device's static scratch (ag_gemm_noalloc). AGG_E_UNSUPPORTED unless the device's
 * architecture is gfx950.
 * Passage: section "The first move was to expose the overlap": symmetric memory and signaling as
 *  the building blocks; the ctx holds the signaling state (epoch, counters) of the calls.
 */
int agg_ctx_create(int device, agg_ctx** out);

/* Free the ctx (synchronises the device first). NULL is accepted.
 * Passage: section "The first move was to expose the overlap" (the ctx's signaling state).
 */
int agg_ctx_destroy(agg_ctx* ctx);

/* After AGG_E_TIMEOUT, or before passing different flags buffers: synchronises the device,
 * zero-fills the flags buffers bound to the ctx (they must still be allocated), unbinds them,
 * clears counters and status, and restarts the epoch at 0.
 * Passage: section "The first move was to expose the overlap" (signaling); recovery after an
 *  abandoned wait is this library's own, the pages describe none.
 */
int agg_ctx_reset(agg_ctx* ctx, agg_stream stream);

/* Synchronise `stream` and read the ctx's device status: *status = 0 when no wait gave up,
 * else bit 0 set; *failed_chunk = the first flag index whose wait gave up, or -1.
 * Returns AGG_E_TIMEOUT when status != 0. Either output pointer may be NULL.
 * Passage: section "DITRON adds three levels of tiling" (synchronization inserted between chunks
 *  and tiles: the status of those waits).
 */
int agg_ctx_status(agg_ctx* ctx, agg_stream stream, uint32_t* status, int32_t* failed_chunk);

/* Current epoch: the value the last producing call wrote into its flags (0 before any).
 * Passage: section "The first move was to expose the overlap" (signaling: a flag carries the epoch
 *  of the call that delivered its chunk).
 */
int agg_ctx_epoch(agg_ctx* ctx, uint32_t* epoch);

/* Move the epoch (tests of the wrap-around): the next producing call uses epoch+1. Epochs run
 * 1 .. 0xFFFFFFFE; past the end the ctx zero-fills its bound flags and restarts at 1.
 * Requires no bound flags buffer (fresh ctx or after agg_ctx_reset); AGG_E_STATE otherwise.
 * Passage: section "The first move was to expose the overlap" (signaling: epoch-tagged flags).
 */
int agg_ctx_set_epoch(agg_ctx* ctx, uint32_t epoch);

/* Device-side wait limit in microseconds (default 2,000,000). A wait that runs past it sets
 * the status word and abandons its tile; later waits of the same call give up at once.
 * Passage: section "DITRON adds three levels of tiling" (synchronization inserted); the bound on a
 *  wait is this library's own.
 */
int agg_ctx_set_timeout_us(agg_ctx* ctx, uint64_t timeout_us);

/* Number of copy streams the producer spreads chunks over (1..8, default 4), all created by
 * the ctx with hardware queues of their own. Chunk i of the arrival order goes to stream i mod n,
 * so every stream keeps the arrival order and the SDMA engines work in parallel.
 * Passage: section "DITRON adds three levels of tiling" (device-level tiles are data movements on
 *  DMA engines).
 */
int agg_ctx_set_copy_streams(agg_ctx* ctx, int n);

/* Producer kinds. */
enum {
  AGG_PRODUCER_CU = 0,    /* copy jobs inside the persistent kernel (default) */
  AGG_PRODUCER_SDMA = 1,  /* hipMemcpyAsync (copy engines) + stream write per chunk */
  AGG_PRODUCER_KERNEL = 2 /* a copy kernel of one-wave workgroups on a ctx stream, beside the GEMM
                             kernel in the registers it leaves free on each SIMD; where the GEMM
                             kernel leaves too few (agg_kernel_regs), or with delays, the call
                             uses AGG_PRODUCER_CU instead */
};

/* Select the producer of later calls. For AGG_PRODUCER_CU, `copy_wgs` workgroups of the
 * persistent grid (0: all of them) first take copy jobs, each moving `piece_kib` KiB of one chunk
 * (0: a chunk is cut into floor(copying workgroups / remote chunks) pieces, at least one, each
 * rounded up to whole 4 KiB and at least 64 KiB (16 KiB when pulled and for AGG_PRODUCER_KERNEL), so that every job fits in one round of the
 * copying workgroups; a chunk is cut into ceil(chunk bytes / piece) pieces), in arrival order, and only then
 * claim tiles; the workgroup that completes a chunk's last piece releases its flag. The other
 * arguments are ignored for AGG_PRODUCER_SDMA. AGG_PRODUCER_KERNEL cuts chunks into `piece_kib`
 * KiB pieces the same way (its grid is 1024 one-wave workgroups; `copy_wgs` is ignored); a call
 * whose persistent kernel leaves the copy kernel too few registers (agg_kernel_regs), or that is
 * given delays, runs AGG_PRODUCER_CU instead (agg_ctx_last_producer says which ran). AGG_E_ARG
 * for an unknown kind or a negative count.
 * Passage: section "The first move was to expose the overlap" (remote data access and signaling)
 *  and section "DITRON adds three levels of tiling" (device-level tiles on DMA engines).
 */
int agg_ctx_set_producer(agg_ctx* ctx, int kind, int copy_wgs, int piece_kib);

/* Store in *kind the producer (AGG_PRODUCER_*) the last ag_gemm, gemm_rs, gemm_ar or ffn_chain
 * call on `ctx` ran, -1 before the first. AGG_E_ARG for a NULL ctx or kind.
 * Passage: section "The first move was to expose the overlap" (the producer side of a call).
 */
int agg_ctx_last_producer(const agg_ctx* ctx, int* kind);

/* Pull modes of ag_gemm (AGG_OVERLAP calls under AGG_PRODUCER_CU without delays). */
enum {
  AGG_PULL_AUTO = 0,   /* pull when the remote rows total at most 4 MiB (default) */
  AGG_PULL_OFF = 1,    /* always push: tiles wait for their chunks' flags */
  AGG_PULL_ON = 2      /* pull whenever it applies */
};

/* Select the pull mode of later ag_gemm calls. In a pulled call the tiles read remote rows
 * straight from the peers' blocks (peer_src; in a multi-GPU setting, loads over the GPU links)
 * instead of waiting for their chunks to reach the gather buffer; the same launch still copies
 * every remote chunk into `gather` and releases its flag, on extra workgroups that take no tile
 * before they finish copying. It applies when the tile's rows can be read shard by shard (m_shard
 * a multiple of the tile height, or, for tiles of up to 128 rows, of 16 rows) and fewer tiles
 * than compute units leave room for the copiers;
 * otherwise the call pushes. Results are identical either way. The pages' overlap puts a
 * chunk's transfer before its tiles; pulling takes that transfer off the tiles' path for small
 * gathers, whose cost is latency rather than bandwidth. AGG_E_ARG for an unknown mode.
 * Passage: section "The first move was to expose the overlap" (remote data access; compute on
 *  arrived data while the rest moves).
 */
int agg_ctx_set_pull(agg_ctx* ctx, int pull);

/* CUs the persistent grid leaves free in AGG_OVERLAP mode (default 32, four per XCD), where
 * the producer's copies and flag writes must run beside it: in the HIP runtime shipped with
 * torch several of them execute as runtime kernels and need a CU. 0..CUs-1.
 * Passage: section "DITRON adds three levels of tiling" (data movements on DMA engines beside the
 *  compute tiles).
 */
int agg_ctx_set_reserved_cus(agg_ctx* ctx, int n);

/* Force the output tile shape (bm x bn) of later calls; 0, 0 restores the automatic choice.
 * Shapes: 256x256, 256x224, 128x128, 128x64, 64x64; anything else is AGG_E_ARG.
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles in registers, shared
 *  memory and matrix units).
 */
int agg_ctx_set_tile(agg_ctx* ctx, int bm, int bn);

/* Split-K of later AllGather+GEMM calls. With few output tiles (fewer than half the CUs) and a
 * long K, the library cuts each tile's K range into parts computed by different workgroups;
 * every part writes an fp32 partial into a ctx-owned buffer (ksplit x M x N floats, allocated
 * and grown by the ctx) and the parts are summed in part order (by the last part to finish, or,
 * when every part has a workgroup of its own, by all parts together, a row range each), so C
 * does not depend on which part finishes last. `ksplit` 1..16 asks for that many parts for
 * tiles of up to 128 x 128 (larger tiles are never split); parts span a whole number of 64-byte
 * K slice pairs, so fewer parts may result (at most one per pair). 0 restores the automatic
 * choice. A chunk wait that times out leaves split-K tile counters behind: call agg_ctx_reset
 * before the next call.
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles).
 */
int agg_ctx_set_split(agg_ctx* ctx, int ksplit);

/* Tile-claim lists of later calls. The persistent workgroups claim tiles from `lists` lists
 * (1..16, default 8: one per XCD, a workgroup starting on the list of the XCD it runs on and
 * stealing from the others when that is empty). The lists form a (lists / list_cols) x list_cols
 * grid over the output: row tiles dealt round-robin in compute order to the grid rows, column
 * tiles in list_cols contiguous blocks, so the tiles in flight on one XCD share A rows and B
 * columns in its L2. list_cols must divide lists; 0 picks it per call from the tile counts.
 * Passage: section "DITRON adds three levels of tiling" (collectives cut into chunks paired with
 *  computation tiles: the order tiles are taken in).
 */
int agg_ctx_set_lists(agg_ctx* ctx, int lists, int list_cols);

/* Tail split of ag_gemm / a2a_gemm calls under the in-kernel producer (AGG_PRODUCER_CU, no
 * pull, no split-K, no per-tile trace attached). A call whose output tiles fill some waves of
 * the grid and spill a partly filled last wave runs its compute in two launches on the same
 * stream: the first (with the copy jobs) takes the row tiles of the whole waves, in compute
 * order; the second, right after it, takes the remaining row tiles, each cut into tiles of the
 * next smaller shape (256-row tiles into 128 x 128, 128 x 128 into 128 x 64, 128 x 64 into
 * 64 x 64), so the last wave's work is spread over more compute units. The same rows are
 * computed with the same per-element K order, so C is bit-identical either way. With kernel
 * timing on, one duration spans both launches.
 *   AGG_TAIL_AUTO (default): split when a tile-time model says the second launch takes less
 *                 than the last wave of big tiles; AGG_TAIL_OFF: never; AGG_TAIL_ON: whenever a
 *                 smaller shape exists and the call has two row tiles or more (at least one
 *                 row tile in each launch).
 * AGG_E_ARG for an unknown mode.
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles; tiles paired with
 *  the chunks) and section "The performance case has a narrow, useful boundary" (wave
 *  quantisation of small and ragged shapes).
 */
enum { AGG_TAIL_AUTO = 0, AGG_TAIL_OFF = 1, AGG_TAIL_ON = 2 };
int agg_ctx_set_tail(agg_ctx* ctx, int mode);

/* Kernel timing: with every = n >= 1, the 1st, (n+1)-th, (2n+1)-th, ... consumer-kernel launch
 * after this call carries a start and an end timing event on the kernel's own stream (n = 1:
 * every launch); the recorded durations go to a ring of the last 256 (switching timing on, or
 * changing n, clears it); every = 0 switches timing off. The events cost a launch some
 * microseconds of its own and of the gap to the next one, so a long run samples. A negative n
 * is AGG_E_ARG. agg_ctx_kernel_times waits for and returns the durations in milliseconds of
 * the last min(max, recorded) timed launches, oldest first, in ms[0..*n); with timing off it
 * is AGG_E_STATE.
 * Passage: section "What would prove the compiler layer is portable" (measurements disclosed with
 *  the numerical checks).
 */
int agg_ctx_set_timing(agg_ctx* ctx, int every);
int agg_ctx_kernel_times(agg_ctx* ctx, float* ms, int max, int* n);

/* Optional per-tile trace (NULL or 0 bytes disables). The buffer is device memory of
 * `bytes` >= 32 * tiles bytes; each computed tile (m-tile i, n-tile j) writes the 8 words
 * agg_trace_rec at index i * n_tiles + j: claim list, position in that list, XCD id of the
 * claiming workgroup, minimum flag value it observed (0xFFFFFFFF if it needed none), visit
 * count (atomic increment), and the three 100 MHz timestamps: claimed, flags seen, done.
 * Passage: section "DITRON adds three levels of tiling" (synchronization inserted: each tile's
 *  claim and flag observation).
 */
int agg_set_trace(agg_ctx* ctx, void* dev_buf, size_t bytes);

typedef struct agg_trace_rec {
  uint32_t list, pos, xcd, min_flag, visits, t_claim, t_ready, t_done;
} agg_trace_rec;

/* Thread-local text describing the last non-OK return of this thread.
 * Passage: none (the library's error convention).
 */
const char* agg_last_error(void);

/* ---- primitive: put with signal -------------------------------------------------------- */

/* Enqueue on copy_stream: copy `bytes` from src to dst (hipMemcpyDeviceToDeviceNoCU), then
 * write `value` into *flag (4-byte aligned) with a stream write, so that stream order places the
 * flag after the data. This is the one-GPU form of the remote data access + signaling pair.
 * Passage: section "The first move was to expose the overlap" (remote data access followed by a
 *  signal); the project page "Triton-distributed" (sourcepulse.org), "How It Works" (low-level
 *  communication primitives).
 */
int agg_put_signal(void* dst, const void* src, size_t bytes, uint32_t* flag, uint32_t value,
                   agg_stream copy_stream);

/* ---- AllGather + GEMM ------------------------------------------------------------------ */

/* C = concat(shard_0, ..., shard_{W-1}) @ B, one rank's share.
 *   world, rank      1 <= world <= 8, 0 <= rank < world
 *   m_shard          rows per shard (Ms >= 0); M = world * m_shard
 *   n, k             output columns and contraction length (n, k >= 0)
 *   chunk_rows       rows per chunk (>= 1, divides m_shard); chunk c (global id) covers gathered
 *                    rows [c*cr, (c+1)*cr) and belongs to shard c / (m_shard/cr)
 *   dtype            AGG_BF16 or AGG_FP8_E4M3; A and B share it
 *   scale_a/scale_b  fp8 per-tensor dequantisation scales (finite, > 0); ignored for bf16
 *   peer_src         HOST array of `world` device pointers: peer p's shard (m_shard x k), the
 *                    emulated remote memory; entry `rank` is ignored
 *   gather           device (M x k): the symmetric gather buffer; rows of shard `rank` must
 *                    already hold the local shard; the producer fills the others
 *   flags            device uint32[world * m_shard/cr], zero-filled once at allocation and then
 *                    bound to this ctx (the first call binds it; another pointer gives
 *                    AGG_E_STATE until agg_ctx_reset). Every flag ends at the call's epoch: the
 *                    local shard's chunks are raised first (their rows are in place at the call),
 *                    each remote chunk's once its rows have landed
 *   b                device (k x n), N contiguous, same dtype
 *   c                device (M x n) bfloat16, row-major, rows in gathered (rank) order
 *   order, n_order   HOST: the remote chunk ids in arrival order, a permutation of all
 *                    (world-1)*m_shard/cr of them; NULL with n_order 0 = ring order (peers
 *                    rank+1, rank+2, ... mod world; chunks ascending within a peer)
 *   delay_us         HOST, NULL or n_order entries: emulated late peers. Chunk i of the arrival
 *                    order starts no earlier than delay_us[0] + ... + delay_us[i] after the
 *                    first chunk could (SDMA producer: the calling thread waits delay_us[i]
 *                    before enqueueing chunk i; CU producer: the copy job waits on the GPU)
 *   mode             AGG_OVERLAP / AGG_SERIAL / AGG_GEMM_ONLY / AGG_COPY_ONLY
 *   stream           the caller's stream: the call is ordered after earlier work on it, and
 *                    later work on it is ordered after the call (kernel and copies)
 *   copy_stream      optional (NULL allowed, else != stream): the copies also start after
 *                    earlier work on it, and later work on it starts after the copies. The
 *                    copies themselves run on the ctx's own streams (agg_ctx_set_copy_streams)
 *                    or inside the kernel (AGG_PRODUCER_CU)
 * Alignment: k * elem, n * elem and n * 2 bytes multiples of 16 (rows of A, B and C), device
 * pointers 16-byte aligned.
 * Passage: section "The first move was to expose the overlap" (an AllGather moves shards into
 *  place, a GEMM consumes them; cut into chunks, computation proceeds on arrived chunks) and
 *  section "DITRON adds three levels of tiling" (chunks paired with computation tiles,
 *  synchronization inserted).
 */
int ag_gemm(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t n, int64_t k,
            int chunk_rows, int dtype, float scale_a, float scale_b,
            const void* const* peer_src, void* gather, uint32_t* flags, const void* b, void* c,
            const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
            agg_stream stream, agg_stream copy_stream);

/* ---- AllGather + GEMM without allocation ------------------------------------------------ */

/* For callers that cannot allocate device memory while they run (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ag_gemm, with the same arguments,
 * results and errors, except that it allocates nothing. Its kernels keep their counters, status,
 * tables and split-K partials in a static device array of 8 MiB + 78 KiB that the library holds
 * on each GPU until the process ends (its address is looked up, and its counters cleared, once
 * per device when the first ctx on that device is created), instead of in the ctx's scratch and
 * the partial buffer ag_gemm grows on demand.
 *  - AGG_E_UNSUPPORTED when the call's split-K partials (parts x M x N x 4 bytes) exceed 8 MiB.
 *  - AGG_E_STATE unless the ctx's producer is AGG_PRODUCER_CU (the copy engines' streams are
 *    created on demand).
 *  - Every ctx on a GPU shares that GPU's array and the array keeps the last call's contents:
 *    calls that overlap in time on one GPU (two streams, two threads, two ctxs) race. After
 *    AGG_E_TIMEOUT, agg_ctx_reset clears the array's counters too; agg_ctx_status reports its
 *    status together with the ctx's own. */
int ag_gemm_noalloc(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t n, int64_t k,
                    int chunk_rows, int dtype, float scale_a, float scale_b,
                    const void* const* peer_src, void* gather, uint32_t* flags, const void* b, void* c,
                    const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
                    agg_stream stream, agg_stream copy_stream);

/* ---- AllToAll + GEMM -------------------------------------------------------------------- */

/* One rank's share of an AllToAll (dispatch) and the GEMM on what it delivers: every source
 * rank p sends this rank the tokens it routed here, counts[p] rows of k (at most `cap`), which
 * land in slot p of the receive buffer; then C = recv @ B over the rows that hold tokens. The
 * path is ag_gemm's over slots of `cap` rows that hold only their first counts[p] rows:
 *   cap              rows per slot (>= 0, a multiple of chunk_rows); M = world * cap
 *   counts           HOST int32[world], 0 <= counts[p] <= cap: rows source p sends this rank
 *                    (counts[rank]: the rank's own tokens routed to itself, already in place)
 *   peer_src         HOST array of `world` device pointers: source p's block for this rank
 *                    (cap x k, its first counts[p] rows are the tokens); entry `rank` ignored
 *   recv             device (M x k): the symmetric receive buffer; slot `rank` must already
 *                    hold the local rows; the producer copies rows [0, counts[p]) of each
 *                    other slot and leaves the rest of the slot alone
 *   flags            as ag_gemm's (one per chunk of cr rows of a slot); every flag ends at the
 *                    call's epoch. A chunk that holds no row (its first row at or past
 *                    counts[p]) is raised at the start without a copy; a partly filled chunk
 *                    copies its rows below the count
 *   b, c             device (k x n) weight, N contiguous; device (M x n) bf16 output. Rows of
 *                    slot p below counts[p] hold the product; a row tile that holds no token
 *                    is not computed (its rows of c are left alone); the other rows at or past
 *                    a count are computed from whatever the receive buffer holds there
 *   order, n_order   HOST: every remote chunk id in arrival order (as ag_gemm's, empty chunks
 *                    included; they are raised first whatever their position), NULL = ring
 *   other arguments  as ag_gemm's (dtype, scales, delay_us, mode, streams); tiles never read
 *                    the sources' blocks directly (no pull)
 * Errors: those of ag_gemm with m_shard = cap, AGG_E_ARG for NULL counts or a count outside
 * [0, cap].
 * Passage: section "DITRON adds three levels of tiling" (AllToAll among the collectives cut
 *  into chunks and paired with computation tiles) and section "The first move was to expose
 *  the overlap" (computation proceeds on the chunks that have arrived).
 */
int a2a_gemm(agg_ctx* ctx, int world, int rank, int64_t cap, int64_t n, int64_t k, int chunk_rows,
             int dtype, float scale_a, float scale_b, const int32_t* counts,
             const void* const* peer_src, void* recv, uint32_t* flags, const void* b, void* c,
             const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
             agg_stream stream, agg_stream copy_stream);

/* ---- GEMM + ReduceScatter -------------------------------------------------------------- */

/* P = A @ B in fp32 (bf16 operands); rows split into `world` blocks of Mb = m/world rows.
 *   a                device (m x k) bf16; b: device (k x n) bf16, N contiguous
 *   send             device fp32 (world-1) x Mb x n: the non-local blocks j != rank of P,
 *                    ascending j (what this rank would push to rank j)
 *   send_flags       device uint32[world * Mb/cr]: entry j*Mb/cr + q is set to the epoch
 *                    when rows [q*cr, (q+1)*cr) of block j are complete in `send` (j != rank)
 *   peer_src         HOST array of `world` device pointers to fp32 Mb x n blocks: the partial
 *                    block each peer p contributes to this rank's block; entry `rank` ignored
 *   recv             device fp32 world x Mb x n: symmetric receive buffer; the producer copies
 *                    peer p's block into slot p chunk by chunk (slot `rank` unused)
 *   flags            device uint32[world * Mb/cr]: the receive flags (chunk p*Mb/cr + q)
 *   out              device fp32 Mb x n: P[block rank] + sum over p != rank, ascending p, of
 *                    recv[p]; a fixed summation order, so the result does not depend on arrival
 *   order/n_order, delay_us, mode, streams: as for ag_gemm, over the (world-1)*Mb/cr incoming
 *   chunks. flags and send_flags are bound to the ctx like ag_gemm's flags; both end at the
 *   epoch everywhere, the local block's entries included (nothing arrives or leaves for them).
 * Alignment: k*2 and n*2 bytes multiples of 16; m a multiple of world; cr divides Mb.
 * Passage: section "The first move was to expose the overlap" (GEMM+ReduceScatter, reducing partial
 *  results) and section "DITRON adds three levels of tiling" (ReduceScatter cut into chunks paired
 *  with tiles).
 */
int gemm_rs(agg_ctx* ctx, int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
            const void* a, const void* b, float* send, uint32_t* send_flags,
            const float* const* peer_src, float* recv, uint32_t* flags, float* out,
            const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
            agg_stream stream, agg_stream copy_stream);

/* ---- GEMM + AllReduce -------------------------------------------------------------------- */

/* One rank's share of GEMM+AllReduce (page "Triton-distributed is turning communication into
 * compiler territory", section "DITRON adds three levels of tiling": AllReduce is one of the
 * collectives cut into chunks paired with compute tiles). Every rank holds a partial P_q of the
 * same M x N output (its K shard of the activations times its rows of the weight); AllReduce
 * leaves their sum on every rank. One-shot form: each rank sends its whole partial to every
 * peer and adds the W-1 it receives. Each output tile computes its part of P = A @ B (fp32),
 * stores it to `send`, waits for every peer's chunks of its rows and writes
 * out = P + recv[p] for p != rank in ascending rank order, all in one kernel.
 *   a                device (m x k) bf16; b: device (k x n) bf16, N contiguous
 *   send             device fp32 m x n: this rank's partial P, what every peer receives
 *   send_flags       device uint32[m/cr]: entry q is set to the epoch once rows [q*cr, (q+1)*cr)
 *                    of `send` are complete
 *   peer_src         HOST array of `world` device pointers to fp32 m x n partials: what peer p
 *                    sends; entry `rank` ignored
 *   recv             device fp32 world x m x n: symmetric receive buffer; the producer copies
 *                    peer p's partial into slot p chunk by chunk (cr rows each; slot `rank` unused)
 *   flags            device uint32[world * m/cr]: receive flag of chunk q of peer p is
 *                    p*(m/cr) + q; every entry ends at the epoch (the rank's own slot included)
 *   out              device fp32 m x n: P + sum over p != rank, ascending p, of recv[p]; a fixed
 *                    summation order, so the result does not depend on arrival order
 *   order/n_order, delay_us, mode, streams: as for gemm_rs, over the (world-1)*m/cr incoming
 *   chunks (NULL order = ring order). flags and send_flags are bound to the ctx like ag_gemm's.
 * Alignment: k*2 and n*2 bytes multiples of 16; cr divides m. */
int gemm_ar(agg_ctx* ctx, int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
            const void* a, const void* b, float* send, uint32_t* send_flags,
            const float* const* peer_src, float* recv, uint32_t* flags, float* out,
            const int32_t* order, int n_order, const uint32_t* delay_us, int mode,
            agg_stream stream, agg_stream copy_stream);

/* ---- The FFN chain: AllGather+GEMM -> SiLU -> GEMM+ReduceScatter ------------------------- */

/* One rank's share of a tensor-parallel FFN built from the two overlapped operations, run as one
 * persistent kernel over a task graph (page "Triton-distributed is turning communication into
 * compiler territory", section "DITRON adds three levels of tiling": task-level tiles scheduled
 * in one persistent kernel; section "The performance case has a narrow, useful boundary": the
 * FFN module on AMD GPUs). M = world * m_shard.
 *   phase 1  h = silu(concat(shards) @ W1): AllGather+GEMM tiles (as ag_gemm: chunk flags, arrival
 *            order) whose epilogue applies x * sigmoid(x) in fp32 and stores bf16
 *   phase 2  y = h @ W2 in fp32, reduce-scattered over row blocks of m_shard rows (as gemm_rs)
 * A phase-2 tile starts once every phase-1 tile of its rows has stored its part of h; both phases'
 * tiles are claimed from one ordered list, so a tile only ever waits for tiles claimed before it.
 *   k1, n1, n2       W1 is k1 x n1, W2 is n1 x n2 (bf16, N contiguous)
 *   chunk_rows       rows per gather chunk (divides m_shard); order/n_order: gather arrival order
 *   rs_chunk_rows    rows per receive chunk (divides m_shard); rs_order/n_rs_order: their order
 *   peer_src, gather, flags       as ag_gemm's (the activations' shards)
 *   h                device (M x n1) bf16: phase 1's output, phase 2's input
 *   send, send_flags, rs_peer_src, recv, rs_flags, out   as gemm_rs's (m = M, n = n2, k = n1)
 *   mode, streams    as ag_gemm; the producer copies both layers' chunks (gather chunks first)
 * Errors: those of ag_gemm and gemm_rs on their halves; AGG_E_UNSUPPORTED beyond 2048 chunks per
 * layer. agg_ctx_set_chain_fused(ctx, 0) runs the same tiles as two launches, all of phase 1 then
 * all of phase 2 (the unfused baseline; results identical). */
int ffn_chain(agg_ctx* ctx, int world, int rank, int64_t m_shard, int64_t k1, int64_t n1, int64_t n2,
              int chunk_rows, int rs_chunk_rows, const void* const* peer_src, void* gather,
              uint32_t* flags, const void* w1, void* h, const void* w2, float* send,
              uint32_t* send_flags, const float* const* rs_peer_src, float* recv, uint32_t* rs_flags,
              float* out, const int32_t* order, int n_order, const int32_t* rs_order, int n_rs_order,
              int mode, agg_stream stream, agg_stream copy_stream);

/* Whether later ffn_chain calls run both phases in one launch (on, the default) or in two.
 * Passage: section "DITRON adds three levels of tiling" (task-level tiles in one persistent kernel)
 *  and section "The performance case has a narrow, useful boundary" (the FFN module).
 */
int agg_ctx_set_chain_fused(agg_ctx* ctx, int on);

/* ---- host-only planning (no device needed; used by the calls above) --------------------- */

/* The tile shape the library uses for a call: *bm x *bn output tiles.
 * op: 0 = ag_gemm (and a2a_gemm), 1 = gemm_rs, 2 = gemm_ar. m is M (ag: world*m_shard; a2a:
 * world*cap).
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles).
 */
int agg_tile_shape(int op, int dtype, int64_t m, int64_t n, int64_t k, int* bm, int* bn);

/* The tail split (agg_ctx_set_tail) of a call computing n_row_tiles row tiles of bm x bn over an
 * m x n output on `units` compute units: *head_rows row tiles in the first launch (0: no split)
 * and the second launch's tile shape *tail_bm x *tail_bn. AGG_E_ARG for an unknown mode or
 * NULL outputs.
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles).
 */
int agg_tail_split(int bm, int bn, int64_t m, int64_t n, int n_row_tiles, int units, int mode,
                   int* head_rows, int* tail_bm, int* tail_bn);

/* Row-tile order of ag_gemm: tiles of `bm` rows of C sorted by the arrival position of the
 * latest remote chunk they overlap (-1 when none), ties by tile index. Writes
 * ceil(world*m_shard/bm) entries to out_tiles (capacity max_tiles); *n_tiles = that count.
 * Passage: section "DITRON adds three levels of tiling" (chunks paired with computation tiles) and
 *  section "The first move was to expose the overlap" (computation on the chunks that have
 *  arrived).
 */
int agg_ag_row_tile_order(int world, int rank, int64_t m_shard, int chunk_rows,
                          const int32_t* order, int n_order, int bm, int32_t* out_tiles,
                          int max_tiles, int* n_tiles);

/* The row tiles (of bm rows over the world*cap receive rows) a2a_gemm computes, in the order it
 * takes them: tiles that hold no token are left out; the others by the arrival position of the
 * latest chunk they cover that holds rows (local chunks and empty ones count as present from
 * the start), ties by tile index. Writes *n_tiles entries to out_tiles (max_tiles room);
 * AGG_E_ARG for bad geometry, counts or order, or too little room.
 * Passage: section "DITRON adds three levels of tiling" (chunks paired with tiles).
 */
int agg_a2a_row_tile_order(int world, int rank, int64_t cap, int chunk_rows, const int32_t* counts,
                           const int32_t* order, int n_order, int bm, int32_t* out_tiles,
                           int max_tiles, int* n_tiles);

/* Row-tile order of gemm_rs as (block, tile-in-block) pairs flattened to block*tpb + tile,
 * tpb = ceil(Mb/bm): non-local blocks in send order rank+1, ..., rank+world-1 (mod world), each
 * ascending; then the local block's tiles by the arrival position of the latest incoming
 * chunk they need, ties by index.
 * Passage: section "DITRON adds three levels of tiling" (chunks paired with computation tiles).
 */
int agg_rs_row_tile_order(int world, int rank, int64_t m, int chunk_rows, const int32_t* order,
                          int n_order, int bm, int32_t* out_tiles, int max_tiles, int* n_tiles);

/* The argument checks ag_gemm / gemm_rs run first (pointers are checked for NULL and 16-byte
 * alignment only). AGG_OK or AGG_E_ARG / AGG_E_UNSUPPORTED with agg_last_error set.
 * Passage: the passages of ag_gemm, gemm_rs and gemm_ar, whose argument contracts these checks
 *  enforce.
 */
int agg_check_ag_args(int world, int rank, int64_t m_shard, int64_t n, int64_t k, int chunk_rows,
                      int dtype, float scale_a, float scale_b, const void* const* peer_src,
                      const void* gather, const void* flags, const void* b, const void* c,
                      const int32_t* order, int n_order, int mode, agg_stream stream,
                      agg_stream copy_stream);

/* a2a_gemm's argument checks alone (no ctx, no GPU work): agg_check_ag_args with m_shard = cap,
 * then counts. Returns AGG_OK or the code a2a_gemm would return.
 * Passage: section "DITRON adds three levels of tiling" (AllToAll chunks).
 */
int agg_check_a2a_args(int world, int rank, int64_t cap, int64_t n, int64_t k, int chunk_rows,
                       int dtype, float scale_a, float scale_b, const int32_t* counts,
                       const void* const* peer_src, const void* recv, const void* flags,
                       const void* b, const void* c, const int32_t* order, int n_order, int mode,
                       agg_stream stream, agg_stream copy_stream);
int agg_check_rs_args(int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                      const void* a, const void* b, const void* send, const void* send_flags,
                      const float* const* peer_src, const void* recv, const void* flags,
                      const void* out, const int32_t* order, int n_order, int mode,
                      agg_stream stream, agg_stream copy_stream);
int agg_check_ar_args(int world, int rank, int64_t m, int64_t n, int64_t k, int chunk_rows,
                      const void* a, const void* b, const void* send, const void* send_flags,
                      const float* const* peer_src, const void* recv, const void* flags,
                      const void* out, const int32_t* order, int n_order, int mode,
                      agg_stream stream, agg_stream copy_stream);

/* ---- diagnostics ---------------------------------------------------------------------- */

/* Registers per lane that the runtime reports for the GEMM kernel instance of (op, dtype, bm x bn)
 * (op: 0 = ag_gemm, 1 = gemm_rs, 2 = gemm_ar, 3 = ffn_chain) and for the copy kernel of
 * AGG_PRODUCER_KERNEL. AGG_E_ARG for a combination without a kernel.
 * Passage: section "DITRON adds three levels of tiling" (core-level tiles in registers). */
int agg_kernel_regs(int op, int dtype, int bm, int bn, int* gemm_regs, int* copy_regs);

#ifdef __cplusplus
}
#endif

#endif /* AGG_H */
