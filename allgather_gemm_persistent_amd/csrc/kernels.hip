// Persistent MFMA GEMM for gfx950 (CDNA4) that consumes rows as their chunks arrive.
//
// The method: page "Triton-distributed is turning communication into compiler territory",
// section "The first move was to expose the overlap" (compute on chunks that arrived while
// others still move) and section "DITRON adds three levels of tiling" (core-level tiles in
// registers / shared memory / matrix units; collectives cut into chunks paired with compute
// tiles, with synchronization inserted).
//
// Design, per workgroup (256 threads = 4 wave64s, 2 x 2 over the tile; 4 x 1 for fp8 tiles
// whose half width is not a multiple of 32; one workgroup per CU):
//   copy jobs first (the in-kernel producer): pieces of the remote chunks in arrival order,
//     the workgroup completing a chunk raising its flag; block 0 raises the local chunks' flags
//   loop:
//     claim a tile from this XCD's list (atomic counter), stealing from other XCDs' lists when
//       its own is exhausted; lists hold row tiles in arrival order, so early chunks are
//       computed first
//     wave 0 polls the flags of the chunks the tile's rows need (relaxed system-scope loads,
//       s_sleep back-off, bounded by a wall-clock limit), then an acquire fence where the
//       launch may have written the rows read
//     K loop: 64-byte-wide K slices (32 bf16 or 64 fp8) of the A rows (K contiguous) and of the
//       B rows (K x N, N contiguous) go straight from global memory to LDS (direct-to-LDS buffer
//       loads into swizzled stages or slice-pair regions below 128 KiB, one barrier per slice);
//       A fragments come from plain LDS reads, B fragments from gfx950's transposing LDS reads;
//       MFMA 16x16x32 bf16 or 32x32x64 f8f6f4 blocks accumulate in fp32
//     epilogue, by operation: AllGather -> bf16 (round to nearest even) rows of C; ReduceScatter
//       -> fp32 partial rows to `send` (non-local blocks; a per-chunk completion counter
//       releases the send flag) or to `out` (the local block); AllReduce -> the partial to
//       `send` with its send flag, then, once the peers' chunks of its rows have arrived, the
//       sum over ranks in ascending order to `out`; FFN chain -> SiLU and bf16 rows of h for
//       the first layer's tiles (which release the second layer's rows), the ReduceScatter
//       epilogue for the second layer's
//   ReduceScatter and the FFN chain then reduce the local block over the whole grid
//   the last workgroup to finish resets the counters for the next launch.
// A workgroup waits only on chunk flags or on tiles claimed before its own (split-K parts of a
// tile that all hold a workgroup; the FFN chain's second layer), so the grid never deadlocks.
//
// MFMA operand roles are swapped (the B tile feeds the instruction's first operand), so each
// lane ends with quads of 4 consecutive output columns of one row: 8-byte bf16 or 16-byte fp32
// stores.
#include "kernels.h"
#include "pipeline.h"

#include <hip/hip_ext.h>

#include <type_traits>
#include <utility>

namespace agg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaveLanes = 64;
constexpr int kThreads = 256;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle)
constexpr int kBufferFlags = 0x00020000;
// a buffer offset past every operand (operands are limited to 2^31 bytes)
constexpr uint32_t kOutOfRange = 0x80000000u;

// hardware register XCC_ID (id 20), bits [3:0]: which accelerator die runs this wave
__device__ inline int xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xF;
}

__device__ inline uint32_t wall_ticks() { return (uint32_t)wall_clock64(); }

__device__ inline uint32_t load_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---- operand pipeline: 64-byte K slices (32 bf16 or 64 fp8 elements) in LDS, filled by
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): four 64-byte stages (tiles below
// 64 x 64), regions of slice pairs with 128-byte rows (64 x 64 up to 128 x 128), or, for the
// 256-row tiles, A in slice-pair regions and B in four 64-byte stages. One wave instruction writes 1 KiB of
// LDS: 16 tile rows of 64 bytes, lane i landing at byte 16*i. Lane i therefore fetches row i/4
// of its 16-row group and the 16-byte chunk that the swizzle below puts at position i%4.
constexpr int kSliceBytes = 64;
constexpr int kStages = 4;

// byte offset of 16-byte chunk `g` (0..3) of LDS row `row` in a 64-byte-row stage: rows 2q and
// 2q+1 share a 128-byte bank line, so chunks rotate with row/2; a ds_read_b128 of 16
// consecutive rows at one chunk touches every bank once per 8 lanes
__device__ inline uint32_t lds64_off(int row, int g) {
  return (uint32_t)(row * kSliceBytes + ((g ^ ((row >> 1) & 3)) << 4));
}

// byte offset of 16-byte chunk `g` (0..7) of LDS row `row` in a 128-byte-row stage pair (two
// consecutive 64-byte K slices of one tile row side by side): rows 2q and 2q+1 share a 256-byte
// bank line, so chunks rotate with row/2; a ds_read_b128 of 16 consecutive rows at one chunk
// touches every bank once
__device__ inline uint32_t lds128_off(int row, int g) {
  return (uint32_t)(row * (2 * kSliceBytes) + ((g ^ ((row >> 1) & 7)) << 4));
}

// Wait until at most N of this wave's vector loads are in flight and its LDS reads are done,
// then meet the other waves. One asm block, so that no compiler fence drains every load.
template <int N>
__device__ inline void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// acc += B fragment x A fragment, one 16x16x32 bf16 MFMA. The asm ties the accumulator to its
// AGPRs: with the builtin's untied form the register allocator rotates the accumulators through
// copies every K slice. volatile keeps the MFMAs in program order with the LDS reads and
// barriers placed around them. The hardware does not interlock accumulator reads and writes by
// other instructions against these MFMAs, so the caller brackets them with acc_settle().
__device__ inline void mfma_bf16(f32x4& acc, const u32x4& b, const u32x4& a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// acc += B fragment x A fragment, one 32x32x64 MFMA on e4m3 operands (the instruction's
// default operand formats) with unit block scales (exponent 127 = 2^0); same rules as mfma_bf16.
__device__ inline void mfma_fp8(f32x16& acc, const i32x8& b, const i32x8& a) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
               : "+a"(acc) : "v"(b), "v"(a), "v"(127));
}

// The two above followed by one direct-to-LDS load (as lds_dma_load below), in one asm statement
// so that the MFMA sits between the M0 write and the load: the wait state the load needs after
// an M0 write, without an s_nop.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void mfma_bf16_dma(f32x4& acc, const u32x4& b, const u32x4& a, const u32x4& desc,
                                     uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %3\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
               "buffer_load_dwordx4 %4, %5, 0 offen lds"
               : "+a"(acc) : "v"(b), "v"(a), "s"(lds_base), "v"(voff), "s"(desc) : "memory", "m0");
}

__device__ inline void mfma_fp8_dma(f32x16& acc, const i32x8& b, const i32x8& a, const u32x4& desc,
                                    uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %3\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %6, %6 op_sel_hi:[0,0,0]\n\t"
               "buffer_load_dwordx4 %4, %5, 0 offen lds"
               : "+a"(acc) : "v"(b), "v"(a), "s"(lds_base), "v"(voff), "s"(desc), "v"(127)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 32 wait states: more than any MFMA result or operand hazard needs (about 20 for a 16-pass op).
// Every accumulator then passes through an empty asm placed after the nops, so that nothing the
// compiler emits touches an accumulator between the MFMAs and the nops.
template <typename V, int FM, int FN>
__device__ inline void acc_settle(V (&acc)[FM][FN]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Transposing LDS reads of 8 bytes per lane (gfx950 ds_read_b64_tr_b16 / _b8) at byte offset
// `off` of the LDS block starting at `base`; the lane permutation is described with the B
// layout (b_swizzle).
__device__ inline u32x2 lds_read_tr16(const uint8_t* base, uint32_t off) {
  typedef __attribute__((address_space(3))) i16x4* p_t;
  typedef __attribute__((address_space(3))) uint8_t* b_t;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((p_t)((b_t)base + off)));
}
__device__ inline u32x2 lds_read_tr8(const uint8_t* base, uint32_t off) {
  typedef __attribute__((address_space(3))) i32x2* p_t;
  typedef __attribute__((address_space(3))) uint8_t* b_t;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((p_t)((b_t)base + off)));
}

// Raw buffer descriptor (base, no stride, num_records bytes) in four scalar registers.
__device__ inline u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, bytes, (uint32_t)kBufferFlags};
}

// One direct-to-LDS load: 16 bytes per lane from desc + voff into LDS at lds_base + 16 * lane.
// Issued as asm so that the compiler neither waits for it nor reorders LDS accesses around it:
// the main loop accounts for these loads itself (stage_barrier / the final drain).
// M0 is reserved by the compiler, which in these kernels never holds a value in it (checked on
// the generated code), so the asm may set it; the s_nop is the wait state the hardware needs
// between an M0 write and the LDS-destination load that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma_load(const u32x4& desc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(desc) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)p);
}

// Two fp32 -> a packed bf16 pair (first value in the low half), rounded to nearest even: one
// gfx950 v_cvt_pk_bf16_f32 (finite inputs; a NaN stays a NaN)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Cache-policy bits of a buffer access on gfx950: sc0 | sc1 = system coherent. A store writes
// through to memory and is visible to every XCD once it completes, without writing back this
// XCD's whole L2 afterwards; a load bypasses the caches and returns what memory holds, so data
// read once after a flag needs no acquire fence (an L2 invalidate) before it.
constexpr int kStoreSystemCoherent = 1 | 16;

// Copy `bytes` (a multiple of 16, < 2 GiB) from src to dst with the whole workgroup: 16-byte
// vectors in groups of U per thread, software-pipelined over two register sets so that the
// loads of group g+1 are issued before the stores of group g (one counter tracks loads and
// stores in issue order, so a load wait never waits for the stores issued after it), then the
// partial last group with all its loads ahead of its stores. The
// source (a peer's block) is read once: non-temporal loads; the stores write through. On return
// every store of the calling thread has completed.
template <int NT, int U = 16>
__device__ inline void copy_piece(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
                                  int64_t bytes, int tid) {
  constexpr int64_t kStep = (int64_t)U * NT;
  const int64_t n16 = bytes >> 4;
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int)bytes, kBufferFlags);
  auto put = [&](int64_t e, const u32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, (int)(e * 16), 0, kStoreSystemCoherent);
  };
  auto load = [&](u32x4 (&v)[U], int64_t g) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(s + g + u * NT);
  };
  auto store = [&](const u32x4 (&v)[U], int64_t g) {
#pragma unroll
    for (int u = 0; u < U; ++u) put(g + u * NT, v[u]);
  };
  // G full groups (the same count for every thread), then a per-vector tail
  const int64_t G = n16 / kStep;
  int64_t i = tid;
  if (G > 0) {
    u32x4 va[U], vb[U];
    load(va, i);
    int64_t g = 1;
    for (; g + 1 < G; g += 2) {          // two groups per trip: loads run one group ahead
      load(vb, i + kStep);
      store(va, i);
      load(va, i + 2 * kStep);
      store(vb, i + kStep);
      i += 2 * kStep;
    }
    if (g < G) {                         // an even count: one more pair, without a look-ahead
      load(vb, i + kStep);
      store(va, i);
      store(vb, i + kStep);
      i += 2 * kStep;
    } else {
      store(va, i);
      i += kStep;
    }
  }
  // the tail: fewer than U vectors per thread are left; all their loads go out before the first
  // store (one load-to-store round trip, not one per vector)
  u32x4 vt[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i + (int64_t)u * NT < n16) vt[u] = __builtin_nontemporal_load(s + i + (int64_t)u * NT);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i + (int64_t)u * NT < n16) put(i + (int64_t)u * NT, vt[u]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ inline int64_t min_i64(int64_t x, int64_t y) { return x < y ? x : y; }
// x clamped to [0, hi]
__device__ inline int64_t clamp_bytes(int64_t x, int64_t hi) { return x < 0 ? 0 : (x > hi ? hi : x); }

// The in-kernel producer. Job j*pieces + q copies piece q of the chunk at arrival position j;
// the job that completes a chunk (all its pieces copied and released) stores the epoch into the
// chunk's flag. Jobs are taken from a shared counter in arrival order, so chunks complete
// roughly in arrival order and the jobs go to whichever workgroups are running (one that has not
// started yet holds none back). With delays, job j*pieces + q starts no earlier than the j-th
// cumulative delay after the first copying workgroup started.
template <int NT>
__device__ inline void produce_chunks(const GemmArgs& a, int tid, int* s_job, int static_rank) {
  const uint32_t* order = a.scratch + kScrOrder;
  // every value that decides a branch around a barrier is made visibly uniform
  // (readfirstlane): otherwise the compiler may treat the loop exit as divergent and lay the
  // loop out so that the lanes of one wave run different iterations, which misaligns the
  // barriers between the waves
  const uint32_t jobs = __builtin_amdgcn_readfirstlane(a.copy_jobs);
  // the next job comes from a shared counter; once it is past the last job a plain load says so
  // (one uncontended read per workgroup at the end of the copy instead of an atomic add)
  // (static_rank >= 0: this is copier static_rank of a.copy_wgs, which takes jobs static_rank,
  // + copy_wgs, ... without a counter; only where no tile waits for a copy)
  uint32_t fixed = static_rank >= 0 ? (uint32_t)static_rank : 0u;
  auto next_job = [&]() -> uint32_t {
    if (static_rank >= 0) {
      const uint32_t job = fixed;
      fixed += (uint32_t)a.copy_wgs;
      return job;
    }
    if (tid == 0) {
      uint32_t j = jobs;
      if (__hip_atomic_load(a.scratch + kScrCopyNext, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < jobs)
        j = atomicAdd(a.scratch + kScrCopyNext, 1u);
      s_job[0] = (int)j;
    }
    __syncthreads();
    const uint32_t job = (uint32_t)__builtin_amdgcn_readfirstlane(s_job[0]);
    __syncthreads();
    return job;
  };
  uint32_t t0 = 0;
  if (a.copy_delays && tid == 0) {
    const uint32_t now = wall_ticks() | 1u;   // never 0, which marks "unset"
    const uint32_t prev = atomicCAS(a.scratch + kScrCopyT0, 0u, now);
    t0 = prev ? prev : now;
  }
  const uint32_t jobs0 = __builtin_amdgcn_readfirstlane(a.cs[0].jobs);
  for (uint32_t job = next_job(); job < jobs; job = next_job()) {
    // the set this job belongs to (uniform): set 0's jobs come first
    const int set = job < jobs0 ? 0 : 1;
    const CopySet& cs = a.cs[set];
    const uint32_t pieces = __builtin_amdgcn_readfirstlane((uint32_t)cs.pieces);
    const uint32_t jj = job - (set ? jobs0 : 0u);
    const uint32_t j = jj / pieces, q = jj - j * pieces;
    const int c = (int)__builtin_amdgcn_readfirstlane(order[cs.order_off + j]);
    const int p = c / cs.cps, jl = c - p * cs.cps;
    if (set == 0 && a.copy_delays && tid == 0) {
      const uint32_t due = a.scratch[kScrDelay + j];
      while (wall_ticks() - t0 < due) __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
    const int64_t base = (int64_t)jl * cs.chunk_bytes;
    // the chunk's bytes that hold rows (all of them, except in an AllToAll's partly filled slots)
    const int64_t held = clamp_bytes(cs.valid_bytes[p] - base, cs.chunk_bytes);
    const int64_t lo = min_i64((int64_t)q * cs.piece_bytes, held);
    const int64_t hi = min_i64(lo + cs.piece_bytes, held);
    copy_piece<NT>(cs.sym + ((int64_t)p * cs.cps) * cs.chunk_bytes + base + lo,
               cs.peer[p] + base + lo, hi - lo, tid);
    // every thread's write-through stores have completed in memory (copy_piece waited for
    // them), so the count and the flag need no cache maintenance: a relaxed count per piece,
    // and the piece that completes the chunk writes its flag (a system-coherent store)
    __syncthreads();
    if (tid == 0) {
      // (a chunk in one piece needs no count: its only job raises the flag, a round trip sooner)
      const uint32_t prev = pieces == 1 ? 0u
                                        : __hip_atomic_fetch_add(a.scratch + kScrPieces + cs.piece_off + c, 1u,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev + 1 == pieces)
        __hip_atomic_store(cs.put_flags + c, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

struct Tile {
  int row_tile;   // index into the row tiles (AG: m-tile; RS: block * tpb + tile)
  int col_tile;
  int list, pos;
};

// Claim lists. The lists form a (L / list_cols) x list_cols grid: list x holds the row tiles at
// compute positions x / list_cols, + L / list_cols, ... (so every list follows the compute order)
// crossed with column tiles [xc*nc/list_cols, (xc+1)*nc/list_cols), xc = x % list_cols.
// Position k of list x is row tile (k / nx) of the list and column c_lo + k % nx.
struct ListGeom {
  int xr, c_lo, nx;
  uint32_t len;
};

__device__ inline ListGeom list_geom(const GemmArgs& a, int x) {
  const int L = a.n_lists, Lc = a.list_cols, Lr = L / Lc;
  ListGeom g;
  g.xr = x / Lc;
  const int xc = x - g.xr * Lc;
  g.c_lo = (int)((int64_t)xc * a.n_col_tiles / Lc);
  g.nx = (int)((int64_t)(xc + 1) * a.n_col_tiles / Lc) - g.c_lo;
  const int ny = g.xr < a.n_row_tiles ? (a.n_row_tiles - g.xr + Lr - 1) / Lr : 0;
  g.len = (x < L && g.nx > 0 && ny > 0) ? (uint32_t)ny * (uint32_t)g.nx : 0u;
  return g;
}

// The first `nstat` workgroups take their first tile without an atomic: workgroup b takes
// position b / L of list b % L (workgroups are dealt to the XCDs round robin, so that is its own
// XCD's list), if the list is that long. The counters then count only the later claims, which
// start past these positions.
__device__ inline uint32_t static_taken(const GemmArgs& a, int x, int nstat, uint32_t len) {
  const int L = a.n_lists;
  const uint32_t n = nstat > x ? (uint32_t)((nstat - 1 - x) / L + 1) : 0u;
  return n < len ? n : len;
}

__device__ inline void list_tile(const GemmArgs& a, int x, const ListGeom& g, uint32_t k, Tile& t) {
  const int Lr = a.n_lists / a.list_cols;
  t.row_tile = (int)a.scratch[kScrRowOrder + a.row_base + g.xr + (int)(k / (uint32_t)g.nx) * Lr];
  t.col_tile = g.c_lo + (int)(k % (uint32_t)g.nx);
  t.list = x;
  t.pos = (int)k;
}

// First tile of workgroup b < nstat (uniform on every lane); false if its list is too short.
__device__ inline bool claim_static(const GemmArgs& a, Tile& t) {
  const int L = a.n_lists, b = (int)blockIdx.x;
  const int x = b % L;
  const uint32_t k = (uint32_t)(b / L);
  const ListGeom g = list_geom(a, x);
  if (k >= g.len) return false;
  list_tile(a, x, g, k, t);
  return true;
}

// Claim the next tile: this XCD's list first, then the others in turn. Run by all lanes of one
// wave: an atomic add on the home list takes a tile while it has one; after that, lane d reads
// the counter of the d-th list in search order, so one round trip finds the first list with
// tiles left (and, at the end, that none has any); the lane owning that list takes a tile with
// an atomic add, retrying if another workgroup emptied the list in between. (Four tiles per
// workgroup, the 8192 x 7168 x 8192 fp8 AllGather+GEMM: 0.9% faster than reading the counters
// before every add.)
// Returns, on every lane, whether a tile was claimed (then in t).
__device__ inline bool claim(const GemmArgs& a, int home, int nstat, Tile& t) {
  const int L = a.n_lists;
  const int lane = threadIdx.x & 63;
  int x = home + lane;
  if (x >= L) x -= L;
  // recomputed per call: hoisted out of the tile loop, these would hold registers through the
  // main loop
  asm volatile("" : "+v"(x));
  const ListGeom g = list_geom(a, lane < L ? x : L);
  const uint32_t skip = static_taken(a, x, nstat, g.len);
  const uint32_t len = g.len - skip;
  // no list has tiles past its static positions: nothing to claim, no counter to read
  if (__ballot(len > 0) == 0) return false;
  uint32_t* ctr = a.scratch + kScrLists + x;
  // the home list first, with the atomic add alone (one round trip instead of a read and then
  // the add while the home list has tiles; a failed add leaves its counter past the list's
  // length, which every later read and add takes as empty)
  {
    const uint32_t len_home = (uint32_t)__shfl((int)len, 0);
    if (len_home > 0) {
      uint32_t k = 0;
      if (lane == 0) k = atomicAdd(ctr, 1u);
      k = (uint32_t)__shfl((int)k, 0);
      if (k < len_home) {
        if (lane == 0) list_tile(a, x, g, skip + k, t);
        t.row_tile = __shfl(t.row_tile, 0);
        t.col_tile = __shfl(t.col_tile, 0);
        t.list = __shfl(t.list, 0);
        t.pos = __shfl(t.pos, 0);
        return true;
      }
    }
  }
  for (;;) {
    const bool open = len > 0 && __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < len;
    const uint64_t m = __ballot(open);
    if (m == 0) return false;
    const int d = (int)__builtin_ctzll(m);
    uint32_t k = 0;
    if (lane == d) k = atomicAdd(ctr, 1u);
    k = (uint32_t)__shfl((int)k, d);
    if (k < (uint32_t)__shfl((int)len, d)) {
      if (lane == d) list_tile(a, x, g, skip + k, t);
      t.row_tile = __shfl(t.row_tile, d);
      t.col_tile = __shfl(t.col_tile, d);
      t.list = __shfl(t.list, d);
      t.pos = __shfl(t.pos, d);
      return true;
    }
  }
}

// FFN chain: task k of the launch is phase 1's tile k (k < tasks1: row tile k / N1-tiles of phase
// 1's order, column k % N1-tiles) or phase 2's tile k - tasks1. Workgroup b takes task b first
// (no atomic); later tasks come from one counter in increasing order, so a task is claimed only
// after every task before it, and the phase-1 tiles a phase-2 tile waits for are held by running
// workgroups that wait for nothing but chunk flags. Run by one wave; uniform result.
__device__ inline bool claim_chain(const GemmArgs& a, bool first, Tile& t) {
  const uint32_t t1 = (uint32_t)a.n_row_tiles1 * (uint32_t)a.n_col_tiles1;
  const uint32_t total = t1 + (uint32_t)a.n_row_tiles * (uint32_t)a.n_col_tiles;
  uint32_t k = blockIdx.x;
  if (!first) {
    uint32_t* ctr = a.scratch + kScrLists;
    k = total;
    if ((threadIdx.x & 63) == 0 &&
        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + gridDim.x < total)
      k = atomicAdd(ctr, 1u) + gridDim.x;
    k = (uint32_t)__shfl((int)k, 0);
  }
  if (k >= total) return false;
  if (k < t1) {
    t.row_tile = (int)a.scratch[kScrRowOrder + k / (uint32_t)a.n_col_tiles1];
    t.col_tile = (int)(k % (uint32_t)a.n_col_tiles1);
    t.list = 1;
  } else {
    const uint32_t k2 = k - t1;
    t.row_tile = (int)a.scratch[kScrRowOrder + a.n_row_tiles1 + k2 / (uint32_t)a.n_col_tiles];
    t.col_tile = (int)(k2 % (uint32_t)a.n_col_tiles);
    t.list = 2;
  }
  t.pos = (int)k;
  return true;
}

// Rows of a row tile: [lo, hi) in the A operand, and (RS) the block it belongs to. ReduceScatter
// row tiles (rs) are numbered block * tpb + tile within the block; others count from row 0.
template <int BM>
__device__ inline void tile_rows(const GemmArgs& a, int row_tile, bool rs, int64_t& lo, int64_t& hi,
                                 int& block, int& tile_in_block) {
  if (!rs) {
    lo = (int64_t)row_tile * BM;
    hi = lo + BM < a.M ? lo + BM : a.M;
    block = 0;
    tile_in_block = row_tile;
  } else {
    block = row_tile / a.tpb;
    tile_in_block = row_tile - block * a.tpb;
    const int64_t base = (int64_t)block * a.m_block;
    lo = base + (int64_t)tile_in_block * BM;
    const int64_t end = base + a.m_block;
    hi = lo + BM < end ? lo + BM : end;
  }
}

// Wave 0 waits until every flag the tile needs holds >= epoch: rows [lo, hi) of a buffer cut
// into chunks of `cr` rows, `cps` chunks per peer, flag p*cps + q for chunk q of peer p. ALL_PEERS
// false: the rows are gathered rows whose own chunks are needed (the local shard's need no wait);
// true: the rows are rows of every peer's block (the chunks of every peer but this rank). Returns
// false if the wait gave up (its own limit, or another workgroup's). Reports the smallest flag value
// seen: on success over all the tile's flags, on giving up the last value read of a flag still
// short of epoch.
template <bool ALL_PEERS>
__device__ bool wait_flags(const GemmArgs& a, const uint32_t* flags, int cr, int cps, int64_t lo,
                           int64_t hi, uint32_t& min_seen) {
  const int lane = threadIdx.x & 63;
  const int q_lo = (int)(lo / cr);
  const int nq = (int)((hi - 1) / cr) - q_lo + 1;
  const int count = ALL_PEERS ? (a.world - 1) * nq : nq;
  uint32_t seen = 0xFFFFFFFFu;
  for (int base_i = 0; base_i < count; base_i += 64) {
    const int i = base_i + lane;
    int f = -1;
    if (i < count) {
      if (!ALL_PEERS) {
        const int c = q_lo + i;
        if (c / cps != a.rank) f = c;
      } else {
        int p = i / nq;
        if (p >= a.rank) ++p;
        f = p * cps + q_lo + (i % nq);
      }
    }
    const uint32_t t0 = wall_ticks();
    uint32_t polls = 0;
    for (;;) {
      uint32_t v = 0xFFFFFFFFu;
      if (f >= 0) v = load_flag(flags + f);
      const bool ok = v >= a.epoch;
      if (__all(ok)) {
        seen = v < seen ? v : seen;
        break;
      }
      ++polls;
      const bool abort_seen = (polls & 15) == 0 &&
          __hip_atomic_load(a.scratch + kScrStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      const bool expired = (uint64_t)(wall_ticks() - t0) > a.timeout_ticks;
      if (abort_seen || expired) {
        if (expired && !ok) {
          atomicCAS(a.scratch + kScrFailed, 0xFFFFFFFFu, (uint32_t)f);
          atomicOr(a.scratch + kScrStatus, 1u);
        }
        uint32_t short_v = ok ? 0xFFFFFFFFu : v;
        for (int off = 32; off > 0; off >>= 1) {
          uint32_t o = __shfl_xor(short_v, off);
          short_v = o < short_v ? o : short_v;
        }
        min_seen = short_v;
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  // smallest value any lane saw
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(seen, off);
    seen = o < seen ? o : seen;
  }
  min_seen = seen;
  return true;
}

// The chunk waits of the three operations' tiles (rows [lo, hi) of the output; `block` is the
// ReduceScatter block): AllGather+GEMM waits for its gathered rows, the ReduceScatter local block
// and the AllReduce tiles for every peer's chunks of their rows.
template <int EPI>
__device__ bool wait_chunks(const GemmArgs& a, int64_t lo, int64_t hi, int block, uint32_t& min_seen) {
  if (EPI == kEpiAllGather) return wait_flags<false>(a, a.flags, a.chunk_rows, a.cps, lo, hi, min_seen);
  if (EPI == kEpiAllReduce) return wait_flags<true>(a, a.flags, a.chunk_rows, a.cps, lo, hi, min_seen);
  if (block != a.rank) return true;
  const int64_t base = (int64_t)block * a.m_block;
  return wait_flags<true>(a, a.flags, a.chunk_rows, a.cps, lo - base, hi - base, min_seen);
}

// Wave-uniform bounded wait until *ctr >= expect: relaxed agent-scope polls with s_sleep, giving
// up like the chunk waits (past the ctx limit, which sets the status word, or once another wait
// has given up). Returns false if it gave up.
__device__ bool wait_count(const GemmArgs& a, const uint32_t* ctr, uint32_t expect) {
  const uint32_t t0 = wall_ticks();
  for (uint32_t polls = 0;; ++polls) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= expect) return true;
    const bool abort_seen = (polls & 15) == 15 &&
        __hip_atomic_load(a.scratch + kScrStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    const bool expired = (uint64_t)(wall_ticks() - t0) > a.timeout_ticks;
    if (abort_seen || expired) {
      if (expired && (threadIdx.x & 63) == 0) atomicOr(a.scratch + kScrStatus, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The local block of a ReduceScatter (the owner sums the partial blocks; page "Triton-distributed
// is turning communication into compiler territory", section "The first move was to expose the
// overlap"): out = out + the incoming
// partial of every peer in ascending rank order, where `out` already holds this rank's own
// partial (stored by the local tiles). Run by every workgroup once no tile is left, over groups
// of kRedRows rows claimed from a shared counter, so the reduction is spread over the whole grid
// instead of the few workgroups holding local tiles. A group waits (wave 0, bounded) until the
// local tiles of its row tile have all stored their partials and until every peer's chunk of
// its rows has arrived; an abandoned group leaves its rows at the local partial. The sums are
// elementwise over 16-byte vectors, consecutive threads on consecutive addresses; `out` (written
// through by other workgroups of this launch) and the received blocks (written by the producer)
// are read with system-coherent loads, which bypass the caches: no acquire fence, whose L2
// invalidate costs more than these once-read lines.
template <int BM>
__device__ void reduce_local(const GemmArgs& a, int tid, int* s_item, int* s_ok) {
  constexpr int kRedRows = 4;              // divides every tile height: a group is in one row tile
  constexpr int U = 4;                     // vectors per thread in flight per peer
  const int64_t mb = a.m_block, N = a.N;
  if (mb == 0 || N == 0) return;
  const uint32_t items = (uint32_t)((mb + kRedRows - 1) / kRedRows);
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t blk = mb * N;              // floats per block
  const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, (int)(blk * 4), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rrecv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.recv), 0, (int)(a.world * blk * 4), kBufferFlags);
  const int world = __builtin_amdgcn_readfirstlane(a.world), rank = __builtin_amdgcn_readfirstlane(a.rank);
  for (;;) {
    if (tid == 0) {
      uint32_t it = items;
      if (__hip_atomic_load(a.scratch + kScrRedNext, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < items)
        it = atomicAdd(a.scratch + kScrRedNext, 1u);
      s_item[0] = (int)it;
    }
    __syncthreads();
    const uint32_t it = (uint32_t)__builtin_amdgcn_readfirstlane(s_item[0]);
    __syncthreads();
    if (it >= items) break;
    const int64_t r0 = (int64_t)it * kRedRows;
    const int64_t r1 = r0 + kRedRows < mb ? r0 + kRedRows : mb;
    if (wave == 0) {
      uint32_t seen = 0;
      const int64_t base = (int64_t)rank * mb;
      const bool ok = wait_count(a, a.scratch + kScrLocal + (int)(r0 / BM), (uint32_t)a.n_col_tiles) &&
                      wait_chunks<kEpiReduceScatter>(a, base + r0, base + r1, rank, seen);
      if (lane == 0) *s_ok = ok;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(*s_ok)) {
      __syncthreads();
      continue;
    }
    const int64_t v0 = r0 * N / 4, nv = (r1 - r0) * N / 4;   // the group's 16-byte vectors
    for (int64_t e0 = tid; e0 < nv; e0 += (int64_t)kThreads * U) {
      f32x4 v[U], in[U][AGG_MAX_WORLD - 1];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + (int64_t)u * kThreads;
        const bool live = e < nv;
        v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   rout, live ? (int)((v0 + e) * 16) : (int)kOutOfRange, 0, kStoreSystemCoherent));
#pragma unroll
        for (int q = 0; q < AGG_MAX_WORLD - 1; ++q) {
          const int p = q < rank ? q : q + 1;     // peers in ascending rank order
          const int off = (live && p < world) ? (int)((int64_t)p * blk * 4 + (v0 + e) * 16) : (int)kOutOfRange;
          in[u][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrecv, off, 0, kStoreSystemCoherent));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = e0 + (int64_t)u * kThreads;
        if (e >= nv) continue;
#pragma unroll
        for (int q = 0; q < AGG_MAX_WORLD - 1; ++q)
          if (q + 1 < world) v[u] += in[u][q];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[u]), rout, (int)((v0 + e) * 16), 0, 0);
      }
    }
    __syncthreads();
  }
}

// Split-K, every part of the tile running at once: part `part` of `ks` sums rows
// [part*BM/ks, (part+1)*BM/ks) of the tile over all parts' fp32 partials, in part order (the
// same sum, bit for bit, as one workgroup adding every part), scales (fp8), and stores bf16.
// Coalesced: consecutive threads take consecutive 16-byte column quads of a row; each thread's
// loads for E quads and G parts are in flight together (one round trip for E quads when ks <= G).
// The partial loads are system-coherent, like the partial stores.
template <int BM, int BN, bool FP8>
__device__ void sum_split_rows(const GemmArgs& a, int tid, int64_t lo, int64_t hi, int64_t n0, int part) {
  constexpr int Q = BN / 4;                       // column quads per tile row
  constexpr int G = 8;                            // parts whose loads are in flight together
  constexpr int E = 2;                            // quads per thread in flight together
  const int ks = __builtin_amdgcn_readfirstlane(a.ksplit);
  const int r0 = part * BM / ks, r1 = (part + 1) * BM / ks;
  const int n_el = (r1 - r0) * Q;
  const int64_t plane = a.M * a.N;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(a.ws, 0, (int)(ks * plane * 4), kBufferFlags);
  for (int e0 = tid; e0 < n_el; e0 += E * kThreads) {
    int64_t idx[E];                               // m * N + n of each quad
    bool live[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int e = e0 + u * kThreads;
      const int64_t m = lo + r0 + e / Q;
      const int64_t n = n0 + 4 * (e % Q);
      live[u] = e < n_el && m < hi && n < a.N;
      idx[u] = m * a.N + n;
    }
    f32x4 sum[E] = {};
    for (int q0 = 0; q0 < ks; q0 += G) {
      f32x4 v[E][G];
#pragma unroll
      for (int u = 0; u < E; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int o = (live[u] && q0 + g < ks) ? (int)(((q0 + g) * plane + idx[u]) * 4) : (int)kOutOfRange;
          v[u][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, kStoreSystemCoherent));
        }
#pragma unroll
      for (int u = 0; u < E; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (q0 + g >= ks) break;
          sum[u] = (q0 + g == 0) ? v[u][g] : sum[u] + v[u][g];
        }
    }
#pragma unroll
    for (int u = 0; u < E; ++u) {
      if (!live[u]) continue;
      f32x4 r = sum[u];
      if (FP8) r *= a.scale;
      u32x2 packed;
      packed[0] = bf16x2_rne(r[0], r[1]);
      packed[1] = bf16x2_rne(r[2], r[3]);
      *reinterpret_cast<u32x2*>(a.c + idx[u]) = packed;
    }
  }
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{}), in order
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BM, int BN, int DT, int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(const GemmArgs a) {
  constexpr int NW = kThreads / kWaveLanes, NT = kThreads;   // one wave per SIMD
  constexpr bool FP8 = (DT == AGG_FP8_E4M3);
  constexpr bool kSplitTiles = BM * BN <= 128 * 128;
  // 2 x 2 waves over 16x16x32 bf16 or 32x32x64 fp8 MFMA blocks (fp8: 4 x 1 when half the
  // tile's columns are not whole 32-column blocks)
  constexpr int WMW = (!FP8 || (BN / 2) % 32 == 0) ? 2 : 4;   // waves along M
  constexpr int WNW = NW / WMW;
  constexpr int WTM = BM / WMW, WTN = BN / WNW;        // wave tile
  constexpr int BLK = FP8 ? 32 : 16;                   // MFMA output block edge
  static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile");
  constexpr int F8M = WTM / 32 > 0 ? WTM / 32 : 1, F8N = WTN / 32 > 0 ? WTN / 32 : 1;
  // output quads (4 consecutive columns of one row per lane) of a wave: acc[FM][FN]; an fp8
  // 32x32 block holds 4 of them per lane
  constexpr int FM = WTM / BLK, FN = (WTN / BLK) * (FP8 ? 4 : 1);

  // 64-byte K slices filled by direct-to-LDS loads, in four stages or in regions of slice pairs
  constexpr int BNP = (BN + 63) / 64 * 64;                   // B rows held in LDS
  constexpr int DSTAGE = (BM + BNP) * kSliceBytes;
  // Tiles of 64 x 64 and larger load K slices in pairs: an LDS row holds two consecutive 64-byte
  // slices of a tile row, so that each load instruction fetches whole 128-byte lines (8 lanes per
  // row) and the L1 sends half as many requests for the same bytes. kRegions pair regions of
  // 2 x DSTAGE bytes each replace the four stages; slice stage sg lies in region sg / 2, half
  // sg % 2. The tiles up to 128 x 128 take four regions (a longer lead for their latency-bound
  // loads; split parts start on whole pairs). The big tiles (kMixed, both dtypes)
  // load only their A rows in pairs (two regions) and keep their B rows in the four 64-byte
  // stages, whose longer lead the B rows need (the XCD's L2 reuses them less; for fp8 this beat
  // two pair regions by ~5%); more regions do not fit the 128 KiB that direct-to-LDS loads were
  // seen to fill correctly. 64 x 64 tiles take pairs too (the decode AllReduce: 51.3 -> 45.8 us
  // against four 64-byte stages); a tile smaller than that would keep the four stages.
  constexpr bool kMixed = !kSplitTiles;
  constexpr bool kPairs = BM * BN >= 64 * 64 && !kMixed;
  constexpr int kRegions = 4;
  constexpr int AREG = BM * 2 * kSliceBytes;                 // mixed: one A pair region
  constexpr int BSTAGE = BNP * kSliceBytes;                  // mixed: one B slice stage
  constexpr int kStageBytes = kMixed ? 2 * AREG + 4 * BSTAGE : kPairs ? kRegions * 2 * DSTAGE : kStages * DSTAGE;
  // Direct-to-LDS loads take their LDS address from M0. Layouts whose destinations reached past
  // 128 KiB gave wrong results (and a copy staged there faulted), consistent with that address
  // wrapping at 128 KiB, so every destination stays below it: the operand stages come first in
  // the kernel's one LDS block, at offset 0, and end at or below 128 KiB.
  struct Smem {
    uint8_t stages[kStageBytes];
    int tile[4];
    int ok;
    int job;
    int acq;
  };
  static_assert(kStageBytes <= kLdsDmaLimit, "direct-to-LDS destinations must stay below 128 KiB");
  static_assert(__builtin_offsetof(Smem, stages) == 0, "the operand stages start the LDS block");
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto& stages = sm.stages;
  auto& s_tile = sm.tile;
  auto& s_ok = sm.ok;
  auto& s_acq = sm.acq;
  auto& s_job = sm.job;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  if (blockIdx.x == 0) {
#pragma unroll
    for (int f = 0; f < 3; ++f)
      for (int i = tid; i < a.mark_count[f]; i += NT)
        __hip_atomic_store(a.mark_flags[f] + i, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  // the list searched first: the one that gives this workgroup its static first tile. The
  // workgroups of one list share an XCD (they are dealt to the XCDs round robin), so its
  // tiles' operand rows stay in that XCD's L2.
  const int home = (int)blockIdx.x % a.n_lists;

  // workgroups whose first tile is taken statically (pull: all but the copiers at the end)
  const int nstat = (EPI == kEpiAllGather && (a.pull || a.copiers_last)) ? (int)gridDim.x - a.copy_wgs
                                                                        : (int)gridDim.x;
  auto claim_tile = [&](bool first) {
    if (wave == 0) {
      Tile t{};
      bool got;
      if constexpr (EPI == kEpiFfn) got = claim_chain(a, first, t);
      else got = (first && (int)blockIdx.x < nstat && claim_static(a, t)) || claim(a, home, nstat, t);
      if (lane == 0) {
        s_tile[0] = got ? t.row_tile : -1;
        s_tile[1] = t.col_tile; s_tile[2] = t.list; s_tile[3] = t.pos;
      }
    }
    __syncthreads();
  };

  // ---- the first tile is claimed at once, while the counters are quiet; then the first
  // copy_wgs workgroups move the remote chunks (so the claim is off the path from the end of
  // the copy to the first tile), and every workgroup computes tiles, claiming the next one after
  // each
  // (pull, and small pushed gathers: the copiers are the last copy_wgs workgroups and take no
  // tile before copying, so the tiles start at once on the others)
  const bool pull = EPI == kEpiAllGather && a.pull;
  const bool last = EPI == kEpiAllGather && (a.pull || a.copiers_last);
  const int first_copier = last ? (int)gridDim.x - a.copy_wgs : 0;
  const bool copier = a.copy_jobs && (int)blockIdx.x >= first_copier &&
                      (int)blockIdx.x < first_copier + a.copy_wgs;
  if (!(last && copier)) claim_tile(true);
  // (pulled: no tile waits for a copy, so the copiers may deal the jobs among themselves;
  // pushed, tiles wait for the copies, so any running copier takes the next job)
  if (copier) produce_chunks<NT>(a, tid, &s_job, pull ? (int)blockIdx.x - first_copier : -1);
  if (last && copier) claim_tile(false);

  for (;; claim_tile(false)) {   // (an abandoned tile returns early; the next claim follows)
    // uniform for the compiler too (see produce_chunks)
    const int row_tile = __builtin_amdgcn_readfirstlane(s_tile[0]);
    if (row_tile < 0) break;
    // the tile: one copy per FFN phase (compile-time), so that each keeps the registers of a
    // single-operation kernel
    auto tile_body = [&](auto ph1_) {
      const int vcol = __builtin_amdgcn_readfirstlane(s_tile[1]);
      const int col_tile = vcol / a.ksplit, part = vcol - col_tile * a.ksplit;
      // FFN chain: phase 1 (AllGather+GEMM into h) or phase 2 (GEMM+ReduceScatter of h); the
      // operands of this tile
      constexpr bool ph1 = EPI == kEpiFfn && decltype(ph1_)::value;
      const uint8_t* const opA = ph1 ? a.a1 : a.a;
      const uint8_t* const opB = ph1 ? a.b1 : a.b;
      const int64_t opN = ph1 ? a.N1 : a.N;
      const int64_t kbytes = (ph1 ? a.K1 : a.K) * (FP8 ? 1 : 2);
      int64_t lo, hi;
      int block, tib;
      tile_rows<BM>(a, row_tile, (EPI == kEpiReduceScatter || EPI == kEpiFfn) && !ph1, lo, hi, block, tib);
      const int64_t n0 = (int64_t)col_tile * BN;
      // this part's K slices [t_lo, t_hi) and the K byte where its loads stop (zeros past it)
      constexpr int kSlice = kSliceBytes;
      const int nk_all = (int)((kbytes + kSlice - 1) / kSlice);
      const int t_lo = part * a.kps;
      const int t_hi = t_lo + a.kps < nk_all ? t_lo + a.kps : nk_all;
      const uint32_t kend = (uint32_t)((int64_t)t_hi * kSlice < kbytes ? (int64_t)t_hi * kSlice : kbytes);
      uint32_t* trec = nullptr;
      if (a.trace && (uint32_t)(row_tile * a.n_col_tiles + vcol) < a.trace_tiles)
        trec = a.trace + 8 * ((int64_t)row_tile * a.n_col_tiles + vcol);
      if (tid == 0 && trec) {
        trec[0] = (uint32_t)s_tile[2]; trec[1] = (uint32_t)s_tile[3]; trec[2] = (uint32_t)xcc_id();
        trec[5] = wall_ticks();
      }

      // ---- wait for the chunks this tile's rows need
      if (wave == 0) {
        uint32_t seen = 0xFFFFFFFFu;
        // (ReduceScatter tiles need no chunk: the received partials are added by reduce_local;
        // AllReduce tiles wait for theirs in the epilogue, after the main loop)
        bool ok = true;
        if (EPI == kEpiAllGather && !pull) {
          ok = wait_chunks<EPI>(a, lo, hi, block, seen);
        } else if (EPI == kEpiFfn && ph1) {
          ok = wait_flags<false>(a, a.flags1, a.chunk_rows1, a.cps1, lo, hi, seen);
        } else if (EPI == kEpiFfn) {
          // phase 2: every phase-1 tile of these rows has stored its part of h
          for (int64_t r = lo / BM; ok && r <= (hi - 1) / BM; ++r)
            ok = wait_count(a, a.scratch + kScrSplit + (int)r, (uint32_t)a.n_col_tiles1);
        }
        // acquire only where this launch may have written what the tile reads: rows of a remote
        // chunk that can land during an overlapped call (not pulled: those come from the peers'
        // blocks), and the FFN chain's h, which its first layer writes in this very launch. An
        // acquire invalidates the XCD's L2, which costs the decode-sized launches ~10%.
        bool acq = false;
        if (EPI == kEpiAllGather && !pull && a.concurrent_producer) {
          const int64_t ms = (int64_t)a.cps * a.chunk_rows;
          acq = !(lo >= (int64_t)a.rank * ms && hi <= (int64_t)(a.rank + 1) * ms);
        } else if (EPI == kEpiFfn && ph1) {
          const int64_t ms = (int64_t)a.cps1 * a.chunk_rows1;
          acq = a.concurrent_producer && !(lo >= (int64_t)a.rank * ms && hi <= (int64_t)(a.rank + 1) * ms);
        } else if (EPI == kEpiFfn) {
          acq = true;
        }
        if (lane == 0) {
          s_ok = ok;
          s_acq = acq;
          if (trec) { trec[3] = seen; trec[6] = wall_ticks(); }
        }
      }
      __syncthreads();
      if (!__builtin_amdgcn_readfirstlane(s_ok)) {
        __syncthreads();
        return;  // abandoned (timeout): the tile's output is left as it was
      }
      if (__builtin_amdgcn_readfirstlane(s_acq)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");

      // ---- K loop: 64-byte K slices in LDS stages or pair regions, filled by direct-to-LDS loads
      // (out-of-range rows and the K tail read zeros through the buffer descriptor's range check)
      f32x4 acc[FM][FN];
      constexpr int NI = (BM + BNP) / (16 * NW);   // load instructions per wave per stage
      constexpr int NA = BM / (16 * NW);           // the first NA of them fetch A rows
      static_assert(BM % (16 * NW) == 0 && BNP % (16 * NW) == 0, "whole 16-row groups per wave");
      // pairs: NL load instructions per wave per slice pair, 8 rows x 128 bytes each, the first NAL
      // of them fetching A rows
      // mixed: NLA A loads per wave per pair (8 rows x 128 bytes), then NIB B loads per wave per
      // slice (16 rows x 64 bytes). NHB of a B slice's loads may go after the barrier of the slice
      // four before it, the rest before the barrier of the slice three before it: all of them
      // before (NHB = 0) measured 3% (bf16) and 6% (fp8) faster than half and half on the
      // workloads' data (9% and 12% with zero-valued remote rows, which draw less power), with the
      // same bits out.
      constexpr int NLA = BM / (8 * NW), NIB = BNP / (16 * NW), NHB = 0;
      // mixed: NLAP of an A pair's loads go after the barrier of an odd slice, the rest before the
      // barrier of the next even slice
      constexpr int NLAP = NLA / 2;
      constexpr int NL = kMixed ? NLA + NIB : kPairs ? 2 * NI : NI;
      constexpr int NAL = kMixed ? NLA : kPairs ? 2 * NA : NA;
      // four stages: NH of a slice's loads go after the barrier of the slice four before it, the
      // rest before the barrier of the slice three before it; pairs: NLP of a pair's loads go after
      // the barrier of an odd slice, the rest before the barrier of the next even slice
      constexpr int NH = NI / 2;
      constexpr int NLP = NL / 2;
      constexpr int EL = FP8 ? 1 : 2;
      constexpr int kRowsB = kSliceBytes / EL;              // K rows of B per slice
      constexpr int kChunksB = BNP * EL / 16;               // 16-byte chunks per B row
      constexpr int NBS = BNP / (16 * NW);                  // B loads per wave per slice
      static_assert(NL - NAL == (kPairs ? 2 : 1) * NBS, "B loads per slice");
      static_assert(!kPairs || (kRegions - 1) * NL < 64, "loads in flight within the vmcnt range");
      // lane's chunk: rows of a 16-row group are lane/4, chunk position lane%4 (pairs: rows of an
      // 8-row group are lane/8, chunk position lane%8)
      const uint32_t gk = (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) << 4);
      auto pair_row = [&](int j) { return (j * NW + wave) * 8 + (lane >> 3); };
      auto pair_gk = [&](int r) { return (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4); };
      // B (K x N, N contiguous): a slice's B block holds kRowsB K rows of kChunksB 16-byte chunks;
      // B load jb of a slice (NBS per wave) fills chunk positions (jb*NW + wave)*64 + lane, i.e. K row
      // b_load_row and column chunk b_load_chunk of the slice (whole rows per instruction, 2..16 of
      // them, so each request is a whole line for rows of 128 bytes and more). Pair tiles load two
      // slices of B per pair: B loads jb and jb + NBS fill the same positions of consecutive slices.
      auto b_pos = [&](int j) { return (((j - NAL) % NBS) * NW + wave) * 64 + lane; };
      uint32_t base[NL];
  #pragma unroll
      for (int j = 0; j < NL; ++j) {
        if (j < NAL) {
          const int r = (kPairs || kMixed) ? pair_row(j) : (j * NW + wave) * 16 + (lane >> 2);  // tile row
          const uint32_t g = (kPairs || kMixed) ? pair_gk(r) : gk;
          const int64_t gr = lo + r;
          base[j] = gr < a.M ? (uint32_t)gr * (uint32_t)kbytes + g : kOutOfRange;
        } else {
          const int q = b_pos(j);
          const int ncol = b_load_chunk(q, kChunksB, EL) * (16 / EL);
          const int64_t gn = n0 + ncol;
          base[j] = (ncol < BN && gn < opN)
                        ? (uint32_t)b_load_row(q, kChunksB) * (uint32_t)(opN * EL) + (uint32_t)gn * EL
                        : kOutOfRange;
        }
      }
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      // A operand: one descriptor for the tile, or (pull, tiles of up to 128 rows) one per A load,
      // whose 16-row group lies in one shard when shards are multiples of 16 rows
      constexpr bool kGroupPull = BM <= 128;
      u32x4 da = buffer_desc(opA, (uint32_t)(a.M * kbytes));
      u32x4 dag[kGroupPull ? NAL : 1];
  #pragma unroll
      for (int j = 0; j < (kGroupPull ? NAL : 1); ++j) dag[j] = da;
      if (pull) {
        // remote rows are read from the peer's block: rebase those A offsets from gather-buffer
        // rows to block rows
        const int64_t ms = (int64_t)a.chunk_rows * a.cps;
        if constexpr (kGroupPull) {
  #pragma unroll
          for (int j = 0; j < NAL; ++j) {
            const int64_t g0 = lo + (int64_t)(j * NW + wave_u) * (kPairs ? 8 : 16);  // first row of the group
            const int p = (int)(g0 / ms);
            if (g0 < a.M && p != a.rank) {
              dag[j] = buffer_desc(a.cs[0].peer[p], (uint32_t)(ms * kbytes));
              if (base[j] != kOutOfRange) base[j] -= (uint32_t)((int64_t)p * ms * kbytes);
            }
          }
        } else {
          // (a tile of more than 128 rows is pulled only when it lies inside one shard)
          const int p = (int)(lo / ms);
          if (p != a.rank) {
            da = buffer_desc(a.cs[0].peer[p], (uint32_t)(ms * kbytes));
            const uint32_t shift = (uint32_t)((int64_t)p * ms * kbytes);
  #pragma unroll
            for (int j = 0; j < NAL; ++j)
              if (base[j] != kOutOfRange) base[j] -= shift;
          }
        }
      }
      const u32x4 db = buffer_desc(opB, (uint32_t)(opN * kbytes));
      const uint32_t lds0 = lds_addr(stages) + (uint32_t)wave_u * 1024u;
      // Load j of a slice (j < NI; pairs: of a slice pair, j < NL): A rows for j < NA (NAL), else B
      // rows. The LDS stage of slice t is (t - t_lo) % 4 (pairs: region ((t - t_lo) / 2) % R); the
      // main loop runs four (pairs: 2R) slices per trip, so every stage and region is a constant.
      auto desc_of = [&](int j) -> const u32x4& {
        return j < NAL ? (kGroupPull ? dag[j < NAL ? j : 0] : da) : db;
      };
      auto m0_of = [&](int sg, int j) { return lds0 + (uint32_t)sg * DSTAGE + (uint32_t)j * (NW * 1024u); };
      // pairs: LDS address of load j into pair region rg
      auto m0p = [&](int rg, int j) { return lds0 + (uint32_t)rg * (2 * DSTAGE) + (uint32_t)j * (NW * 1024u); };
      // K byte offset of load j of slice t. Slices below t_safe lie wholly inside the part's K
      // range: a plain offset. Otherwise (`masked`) the offset's top bit is set past the K end
      // (out of range: reads zero), lane by lane, since a slice may straddle the end.
      const int t_safe = (int)(kend / kSlice);
      // B load j of slice t: row b_load_row of the slice's K rows, which start at K row t*kRowsB
      // (64 * N bytes per slice); masked: rows at or past the part's K end read zeros
      const uint32_t kend_rows = kend / EL;
      auto voff_b = [&](auto masked, int t, int j) -> uint32_t {
        const uint32_t tb = (uint32_t)t * (uint32_t)(kSliceBytes * opN);
        if constexpr (decltype(masked)::value) {
          const uint32_t row = (uint32_t)(t * kRowsB + b_load_row(b_pos(j), kChunksB));
          return (base[j] + tb) | (row >= kend_rows ? kOutOfRange : 0u);
        } else {
          return base[j] + tb;
        }
      };
      auto voff_of = [&](auto masked, int t, int j) -> uint32_t {
        if (j >= NAL) return voff_b(masked, t, j);
        const uint32_t tk = (uint32_t)t * kSliceBytes;
        if constexpr (decltype(masked)::value) {
          const uint32_t oob = (uint32_t)((int)(tk + gk - kend) >> 31) ^ 0xFFFFFFFFu;
          return (base[j] + tk) | (oob & kOutOfRange);
        } else {
          return base[j] + tk;
        }
      };
      // pairs: K byte offset of load j of slice pair pr (slices 2pr and 2pr+1), masked as above
      auto voffp = [&](auto masked, int pr, int j) -> uint32_t {
        if (j >= NAL) return voff_b(masked, 2 * pr + (j - NAL) / NBS, j);
        const uint32_t pk = (uint32_t)pr * (2 * kSliceBytes);
        if constexpr (decltype(masked)::value) {
          const uint32_t oob = (uint32_t)((int)(pk + pair_gk(pair_row(j)) - kend) >> 31) ^ 0xFFFFFFFFu;
          return (base[j] + pk) | (oob & kOutOfRange);
        } else {
          return base[j] + pk;
        }
      };
      // mixed: A load j into A region rg; B load j (>= NLA) into B stage sg
      auto m0ma = [&](int rg, int j) { return lds0 + (uint32_t)rg * AREG + (uint32_t)j * (NW * 1024u); };
      auto m0mb = [&](int sg, int j) {
        return lds0 + (uint32_t)(2 * AREG + sg * BSTAGE) + (uint32_t)(j - NLA) * (NW * 1024u);
      };
      auto issue_one = [&](auto masked, int t, int sg, int j) {
        lds_dma_load(desc_of(j), m0_of(sg, j), voff_of(masked, t, j));
      };
      // The loads a slice issues, as (load index, LDS address, offset). Four stages: in the first
      // half of slice t, loads NH.. of slice t+3 into stage (t+3)%4; in the second half, loads
      // 0..NH-1 of slice t+4 into stage t%4. Pairs: an even slice t issues, in its first half, the
      // second half of the loads of pair t/2+1 into the other region; an odd slice t, in its second
      // half, the first half of the loads of pair (t+1)/2+1 into its own region (whose pair every
      // wave has finished at the odd slice's barrier).
      struct Ld { int j; uint32_t m0, vo; };
      auto ld_first = [&](auto masked, auto u_, int t, int e) -> Ld {
        constexpr int U = decltype(u_)::value;
        if constexpr (kMixed) {
          // even slices: the second part of A pair t/2+1, then (all slices) the second part of B
          // slice t+3
          constexpr int EA = (U & 1) ? 0 : NLA - NLAP;
          if (e < EA) {
            const int j = NLAP + e;
            return Ld{j, m0ma(((U >> 1) + 1) & 1, j), voffp(masked, t / 2 + 1, j)};
          }
          const int j = NLA + NHB + (e - EA);
          return Ld{j, m0mb((U + 3) & 3, j), voff_of(masked, t + 3, j)};
        } else if constexpr (kPairs) {
          const int j = NLP + e;
          return Ld{j, m0p(((U >> 1) + kRegions - 1) % kRegions, j), voffp(masked, t / 2 + kRegions - 1, j)};
        } else {
          const int j = NH + e;
          return Ld{j, m0_of((U + 3) & 3, j), voff_of(masked, t + 3, j)};
        }
      };
      auto ld_second = [&](auto masked, auto u_, int t, int k) -> Ld {
        constexpr int U = decltype(u_)::value;
        if constexpr (kMixed) {
          // odd slices: the first part of A pair (t+1)/2+1, then (all slices) the first part of B
          // slice t+4
          constexpr int KA = (U & 1) ? NLAP : 0;
          if (k < KA) return Ld{k, m0ma(U >> 1, k), voffp(masked, (t + 1) / 2 + 1, k)};
          const int j = NLA + (k - KA);
          return Ld{j, m0mb(U, j), voff_of(masked, t + 4, j)};
        }
        if constexpr (kPairs) return Ld{k, m0p(U >> 1, k), voffp(masked, (t + 1) / 2 + kRegions - 1, k)};
        else return Ld{k, m0_of(U, k), voff_of(masked, t + 4, k)};
      };
      // The slice schedule, for both dtypes: RM x CN MFMA blocks per wave and slice, operand
      // fragments of type F read from LDS by lda(stage, block row) / ldb(stage, block column).
      // One K slice t in stage U, its B fragments in fbc and its first A fragment in fa (requested
      // during the previous slice). Stage U is refilled with slice t+4 by NI direct-to-LDS loads,
      // the first NH of them in the second half of slice t and the rest in the first half of slice
      // t+1, so that every half slice carries about NI/2 loads between its MFMAs and the load path
      // never takes a burst. First half of slice t: the remaining A fragments of slice t are
      // requested row by row, and the loads NH..NI-1 of slice t+3 go between the MFMAs. Then the
      // waves meet (slice t+1 has landed everywhere; every wave has read all of slice t), and the
      // second half spreads slice t+1's B fragments and first A fragment, then the loads 0..NH-1
      // of slice t+4, between its MFMAs. (Pairs: the same two halves carry the pair loads that
      // ld_first / ld_second describe.) A load that follows an MFMA shares its asm statement
      // (mma_dma), so the MFMA is the wait state between the M0 write and the load.
      auto run_slices = [&](auto& accs, auto fa, auto lda, auto ldb, auto mma, auto mma_dma,
                            auto rm_, auto cn_, auto lone_) {
        constexpr int RM = decltype(rm_)::value, CN = decltype(cn_)::value;
        constexpr bool kLone = decltype(lone_)::value;
        using F = decltype(fa);
        // block rows before the barrier: one more than half (when that leaves one after it), which
        // measured 1-3% faster than half
        constexpr int RB = (RM / 2 + 1 < RM) ? RM / 2 + 1 : RM / 2;
        constexpr int S1 = RB * CN, S2 = (RM - RB) * CN;
        static_assert(RM - RB - 1 <= RB, "the A fragments after the barrier are loaded before it");
        auto slice = [&](auto u_, auto masked, F (&fbc)[CN], F (&fbn)[CN], int t) {
          constexpr int U = decltype(u_)::value;
          constexpr int U1 = (U + 1) % (kPairs ? 2 * kRegions : 4);
          // loads issued in the first half (E1) and in the second half (ND) of this slice
          constexpr int E1 = kMixed ? ((U & 1) ? 0 : NLA - NLAP) + (NIB - NHB)
                             : kPairs ? ((U & 1) ? 0 : NL - NLP) : NI - NH;
          constexpr int ND = kMixed ? ((U & 1) ? NLAP : 0) + NHB : kPairs ? ((U & 1) ? NLP : 0) : NH;
          constexpr int E2 = CN + 1 + ND;
          F far[RM];
          far[0] = fa;
          if (S1 == 0) {                            // no MFMA before the barrier: issue plainly
  #pragma unroll
            for (int e = 0; e < E1; ++e) {
              const Ld l = ld_first(masked, u_, t, e);
              lds_dma_load(desc_of(l.j), l.m0, l.vo);
            }
          }
  #pragma unroll
          for (int i = 0; i < RB; ++i) {
            far[i + 1] = lda(U, i + 1);
            if (RB + 1 + i < RM) far[RB + 1 + i] = lda(U, RB + 1 + i);
  #pragma unroll
            for (int j = 0; j < CN; ++j) {
              const int q = i * CN + j;
              bool fused = false;
  #pragma unroll
              for (int e = 0; e < E1; ++e) {
                if (S1 == 0 || e * S1 / (E1 > 0 ? E1 : 1) != q) continue;
                const Ld l = ld_first(masked, u_, t, e);
                if (!fused) {
                  mma_dma(accs[i][j], fbc[j], far[i], desc_of(l.j), l.m0, l.vo);
                  fused = true;
                } else {
                  lds_dma_load(desc_of(l.j), l.m0, l.vo);
                }
              }
              if (!fused) mma(accs[i][j], fbc[j], far[i]);
            }
          }
          // slice t+1 has landed (four stages: all but the 2*NI loads issued since; pairs, odd t:
          // all of pair (t+1)/2, the last loads issued; even t: all but the NL of pair t/2+1)
          stage_barrier<kMixed ? mixed_barrier_count(U, NLA, NIB, NHB, NLAP)
                        : kPairs ? pair_barrier_count(U, kRegions, NL) : stage_barrier_count(NI)>();
  #pragma unroll
          for (int i = RB; i < RM; ++i) {
  #pragma unroll
            for (int j = 0; j < CN; ++j) {
              const int q = (i - RB) * CN + j;
              if (kLone) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
              // the first second-half load scheduled after this MFMA is fused with it
              int fuse_e = -1;
  #pragma unroll
              for (int e = CN + 1; e < E2; ++e)
                if (fuse_e < 0 && e * S2 / E2 == q) fuse_e = e;
              if (fuse_e >= 0) {
                const Ld l = ld_second(masked, u_, t, fuse_e - CN - 1);
                mma_dma(accs[i][j], fbc[j], far[i], desc_of(l.j), l.m0, l.vo);
              } else {
                mma(accs[i][j], fbc[j], far[i]);
              }
  #pragma unroll
              for (int e = 0; e < E2; ++e) {
                if (e * S2 / E2 != q || e == fuse_e) continue;   // request e goes after MFMA slot e*S2/E2
                if (e < CN) fbn[e] = ldb(U1, e);
                else if (e == CN) fa = lda(U1, 0);
                else {
                  const Ld l = ld_second(masked, u_, t, e - CN - 1);
                  lds_dma_load(desc_of(l.j), l.m0, l.vo);
                }
              }
            }
          }
        };
        if (t_hi > t_lo) {
          F fb0[CN], fb1[CN];
          acc_settle(accs);
          constexpr auto kPlain = std::integral_constant<bool, false>{};
          constexpr auto kMasked = std::integral_constant<bool, true>{};
          if constexpr (kMixed) {
            // A pair 0 whole and the first part of A pair 1; B slices 0..2 whole and the first part
            // of B slice 3 (the first slices issue the rest)
  #pragma unroll
            for (int j = 0; j < NLA; ++j) lds_dma_load(desc_of(j), m0ma(0, j), voffp(kMasked, t_lo / 2, j));
  #pragma unroll
            for (int j = 0; j < NLAP; ++j) lds_dma_load(desc_of(j), m0ma(1, j), voffp(kMasked, t_lo / 2 + 1, j));
  #pragma unroll
            for (int q = 0; q < 3; ++q)
  #pragma unroll
              for (int j = NLA; j < NLA + NIB; ++j) lds_dma_load(desc_of(j), m0mb(q, j), voff_of(kMasked, t_lo + q, j));
  #pragma unroll
            for (int j = NLA; j < NLA + NHB; ++j) lds_dma_load(desc_of(j), m0mb(3, j), voff_of(kMasked, t_lo + 3, j));
            stage_barrier<mixed_prologue_count(NLA, NIB, NHB, NLAP)>();
          } else if constexpr (kPairs) {
            // pairs 0 .. R-2 whole and the first half of pair R-1 (the first slice issues the rest)
  #pragma unroll
            for (int q = 0; q + 1 < kRegions; ++q)
  #pragma unroll
              for (int j = 0; j < NL; ++j) lds_dma_load(desc_of(j), m0p(q, j), voffp(kMasked, t_lo / 2 + q, j));
  #pragma unroll
            for (int j = 0; j < NLP; ++j)
              lds_dma_load(desc_of(j), m0p(kRegions - 1, j), voffp(kMasked, t_lo / 2 + kRegions - 1, j));
            stage_barrier<pair_prologue_count(kRegions, NL, NLP)>();
          } else {
  #pragma unroll
            for (int s = 0; s < 3; ++s)
  #pragma unroll
              for (int j = 0; j < NI; ++j) issue_one(kMasked, t_lo + s, s, j);
  #pragma unroll
            for (int j = 0; j < NH; ++j) issue_one(kMasked, t_lo + 3, 3, j);   // the first slice issues the rest
            stage_barrier<stage_prologue_count(NI, NH)>();
          }
  #pragma unroll
          for (int j = 0; j < CN; ++j) fb0[j] = ldb(0, j);
          fa = lda(0, 0);
          // four slices per trip (pairs: 2R), slice U of a trip in stage U (pairs: region U / 2).
          // A trip whose loads (up to slice t+7; pairs: t + 4R - 1) stay below t_safe needs no
          // K-end masks. The masked trips stop after the part's last slice (a uniform branch):
          // the loads already issued for later slices read zeros and are drained below.
          constexpr int TRIP = kPairs ? 2 * kRegions : 4;
          auto trip = [&](auto masked, int t) {
            bool live = true;
            static_for<TRIP>([&](auto u_) {
              constexpr int U = decltype(u_)::value;
              if (!live) return;
              if constexpr (U % 2 == 0) slice(u_, masked, fb0, fb1, t + U);
              else slice(u_, masked, fb1, fb0, t + U);
              if constexpr (decltype(masked)::value) live = t + U + 1 < t_hi;
            });
          };
          int t = t_lo;
          for (; t + (kPairs ? 4 * kRegions : 8) - 1 < t_safe; t += TRIP) trip(kPlain, t);
          for (; t < t_hi; t += TRIP) trip(kMasked, t);
          acc_settle(accs);
          // loads issued past the end land (as zeros) and every wave is done with LDS before the
          // next tile refills it
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
      };
      // LDS byte offset of 16-byte chunk g (0..3) of A row `row` of slice stage sg
      auto frag_off = [&](int sg, int row, int g) -> uint32_t {
        if constexpr (kMixed) {
          // A rows: pair region (sg/2) % 2, half sg % 2
          return (uint32_t)(((sg >> 1) & 1) * AREG) + lds128_off(row, (sg & 1) * 4 + g);
        } else if constexpr (kPairs) {
          return (uint32_t)((sg >> 1) * (2 * DSTAGE)) + lds128_off(row, (sg & 1) * 4 + g);
        } else {
          return (uint32_t)(sg * DSTAGE) + lds64_off(row, g);
        }
      };
      // LDS byte offset of the B block of slice stage sg (after the A rows of its stage or pair
      // region; mixed: the B stages after the two A regions)
      auto bblk = [&](int sg) -> uint32_t {
        if constexpr (kMixed) return (uint32_t)(2 * AREG + sg * BSTAGE);
        else if constexpr (kPairs)
          return (uint32_t)((sg >> 1) * (2 * DSTAGE) + BM * 2 * kSliceBytes + (sg & 1) * (BNP * kSliceBytes));
        else return (uint32_t)(sg * DSTAGE + BM * kSliceBytes);
      };
      // this lane's transposing B reads: byte offset of read 0 inside a B block for the fragment
      // whose first chunk is 0, and its rows' swizzle (read r adds r times 4 rows (bf16) or 8 rows
      // (fp8); the fragment's first chunk c0 (even) enters as (c0 ^ swizzle))
      const uint32_t boff0 = (uint32_t)b_read_base(lane, kChunksB, EL);
      const uint32_t bswz = (uint32_t)b_read_swizzle(lane, kChunksB, EL);
      constexpr uint32_t kReadRowStep = (uint32_t)b_read_step(kChunksB, EL);
      if constexpr (!FP8) {
        // ---- bf16: 16x16x32 MFMA blocks, one 16-byte fragment per lane
  #pragma unroll
        for (int i = 0; i < FM; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B fragment: 16 columns starting at chunk c0, K rows 8*(lane/16) .. +7 from two
        // transposing reads (rows +0..3 and +4..7)
        auto ldb = [&](int sg, int j) {
          const uint32_t c0 = (uint32_t)((wn * WTN + j * 16) >> 3);
          const uint32_t off = bblk(sg) + boff0 + 16u * (c0 ^ bswz);
          const u32x2 r0 = lds_read_tr16(stages, off);
          const u32x2 r1 = lds_read_tr16(stages, off + kReadRowStep);
          return u32x4{r0[0], r0[1], r1[0], r1[1]};
        };
        auto lda = [&](int sg, int i) {
          return *reinterpret_cast<const u32x4*>(stages + frag_off(sg, wm * WTM + i * 16 + (lane & 15), lane >> 4));
        };
        run_slices(acc, u32x4{}, lda, ldb,
                   [](f32x4& c, const u32x4& b, const u32x4& x) { mfma_bf16(c, b, x); },
                   [](f32x4& c, const u32x4& b, const u32x4& x, const u32x4& d, uint32_t m0v, uint32_t vo) {
                     mfma_bf16_dma(c, b, x, d, m0v, vo);
                   },
                   std::integral_constant<int, FM>{}, std::integral_constant<int, FN>{},
                   std::integral_constant<bool, false>{});
      } else {
        // ---- fp8 (e4m3): 32x32x64 MFMA blocks with unit block scales, one 32-byte fragment per
        // lane; the per-tensor scales are applied in the epilogue
        f32x16 acc8[F8M][F8N];
  #pragma unroll
        for (int i = 0; i < F8M; ++i)
  #pragma unroll
          for (int j = 0; j < F8N; ++j) acc8[i][j] = f32x16{};
        // a 32-row fp8 A fragment: row r + (lane & 31), K bytes 32*(lane/32) .. +31 of the slice
        auto lda = [&](int sg, int i) {
          const int row = wm * WTM + i * 32 + (lane & 31), g = (lane >> 5) * 2;
          const u32x4 lo4 = *reinterpret_cast<const u32x4*>(stages + frag_off(sg, row, g));
          const u32x4 hi4 = *reinterpret_cast<const u32x4*>(stages + frag_off(sg, row, g + 1));
          return i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                       (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        };
        // B fragment: 32 columns starting at chunk c0, K rows 32*(lane/32) .. +31 from four
        // transposing reads of 8 rows each
        auto ldb = [&](int sg, int j) {
          const uint32_t c0 = (uint32_t)((wn * WTN + j * 32) >> 4);
          const uint32_t off = bblk(sg) + boff0 + 16u * (c0 ^ bswz);
          const u32x2 r0 = lds_read_tr8(stages, off);
          const u32x2 r1 = lds_read_tr8(stages, off + kReadRowStep);
          const u32x2 r2 = lds_read_tr8(stages, off + 2 * kReadRowStep);
          const u32x2 r3 = lds_read_tr8(stages, off + 3 * kReadRowStep);
          return i32x8{(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1],
                       (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
        };
        // a wave with a single 32x32 block reuses its accumulator in the next slice's first
        // MFMA: give the previous one time to write it back
        run_slices(acc8, i32x8{}, lda, ldb,
                   [](f32x16& c, const i32x8& b, const i32x8& x) { mfma_fp8(c, b, x); },
                   [](f32x16& c, const i32x8& b, const i32x8& x, const u32x4& d, uint32_t m0v, uint32_t vo) {
                     mfma_fp8_dma(c, b, x, d, m0v, vo);
                   },
                   std::integral_constant<int, F8M>{}, std::integral_constant<int, F8N>{},
                   std::integral_constant<bool, (F8M * F8N < 3)>{});
        // the epilogue's view: quad q of block (i, j) is acc[i][4j + q]
  #pragma unroll
        for (int i = 0; i < F8M; ++i)
  #pragma unroll
          for (int j = 0; j < F8N; ++j)
  #pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][4 * j + q] = f32x4{acc8[i][j][4 * q], acc8[i][j][4 * q + 1], acc8[i][j][4 * q + 2],
                                        acc8[i][j][4 * q + 3]};
      }

      // ---- epilogue
      // quad (i, j) of this lane: row qrow(i), columns qcol(j) .. qcol(j)+3 of the tile
      auto qrow = [&](int i) {
        return FP8 ? wm * WTM + i * 32 + (lane & 31) : wm * WTM + i * 16 + (lane & 15);
      };
      auto qcol = [&](int j) {
        return FP8 ? wn * WTN + (j >> 2) * 32 + (j & 3) * 8 + (lane >> 5) * 4
                   : wn * WTN + j * 16 + (lane >> 4) * 4;
      };
      if (EPI == kEpiFfn && ph1) {
        // phase 1: h = silu(acc) as bf16, written through (phase-2 tiles on any XCD read it), then
        // the tile counts itself in its row tile once its stores have completed
        const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(a.h, 0, (int)(a.M * a.N1 * 2), kBufferFlags);
  #pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int64_t m = lo + qrow(i);
          if (m >= hi) continue;
  #pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + qcol(j);
            if (n >= a.N1) continue;
            f32x4 v = acc[i][j];
  #pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = v[e] / (1.0f + __expf(-v[e]));
            u32x2 packed;
            packed[0] = bf16x2_rne(v[0], v[1]);
            packed[1] = bf16x2_rne(v[2], v[3]);
            __builtin_amdgcn_raw_buffer_store_b64(packed, rh, (int)((m * a.N1 + n) * 2), 0, kStoreSystemCoherent);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
          __hip_atomic_fetch_add(a.scratch + kScrSplit + row_tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (EPI == kEpiAllGather) {
        bool finish = true;
        // split-K exists for tiles up to 128 x 128 only (the host never splits a larger one): the
        // partial and reduction code would cost the big tiles registers in their main loop
        if (kSplitTiles && a.ksplit > 1) {
          // split-K: every part writes its fp32 partial (write-through) and counts itself in; the
          // parts are summed in part order (so the sum does not depend on which part is last),
          // by all parts together or by the part that arrives last, then converted and stored.
          // The partial loads are system-coherent: a stale line of an earlier launch must not be
          // read.
          const int64_t plane = a.M * a.N;
          const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
              a.ws, 0, (int)(a.ksplit * plane * 4), kBufferFlags);
  #pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t m = lo + qrow(i);
            if (m >= hi) continue;
  #pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int64_t n = n0 + qcol(j);
              if (n >= a.N) continue;
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rw,
                                                     (int)(((int64_t)part * plane + m * a.N + n) * 4),
                                                     0, kStoreSystemCoherent);
            }
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          const int tile_id = row_tile * (a.n_col_tiles / a.ksplit) + col_tile;
          uint32_t* split_ctr = a.scratch + kScrSplit + tile_id;
          if (a.split_together) {
            // every part has its own workgroup in this launch: once all parts have stored, each
            // sums a row range of the tile. The counter is cleared by the launch's last
            // workgroup (not by the last part to finish its sum, which would cost every part
            // another atomic round trip before it is done)
            const uint32_t ks = (uint32_t)a.ksplit;
            if (tid == 0) __hip_atomic_fetch_add(split_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (wave == 0) {
              const bool ok = wait_count(a, split_ctr, ks);
              if (lane == 0) s_ok = ok;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(s_ok)) sum_split_rows<BM, BN, FP8>(a, tid, lo, hi, n0, part);
            finish = false;
          } else {
            if (tid == 0)
              s_ok = (__hip_atomic_fetch_add(split_ctr, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)a.ksplit - 1);
            __syncthreads();
            finish = __builtin_amdgcn_readfirstlane(s_ok) != 0;
            if (finish) {
              // parts in order, G at a time: the loads of G parts are in flight together (one round
              // trip per group instead of per part), then they are added one after another in part
              // order, so the sum does not depend on the grouping
              auto load_part = [&](f32x4 (&v)[FM][FN], int q) {
  #pragma unroll
                for (int i = 0; i < FM; ++i) {
                  const int64_t m = lo + qrow(i);
  #pragma unroll
                  for (int j = 0; j < FN; ++j) {
                    const int64_t n = n0 + qcol(j);
                    // rows / columns past the end, and parts past the last, read zeros (offset past
                    // the buffer)
                    const int off = (q < a.ksplit && m < hi && n < a.N)
                                        ? (int)(((int64_t)q * plane + m * a.N + n) * 4)
                                        : (int)kOutOfRange;
                    v[i][j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kStoreSystemCoherent));
                  }
                }
              };
              constexpr int G = FM * FN >= 32 ? 1 : (32 / (FM * FN) > 8 ? 8 : 32 / (FM * FN));
              const int ks = __builtin_amdgcn_readfirstlane(a.ksplit);
              for (int q0 = 0; q0 < ks; q0 += G) {
                f32x4 v[G][FM][FN];
  #pragma unroll
                for (int g = 0; g < G; ++g) load_part(v[g], q0 + g);
                __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
                for (int g = 0; g < G; ++g) {
                  if (q0 + g >= ks) break;
  #pragma unroll
                  for (int i = 0; i < FM; ++i)
  #pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = (q0 + g == 0) ? v[g][i][j] : acc[i][j] + v[g][i][j];
                }
              }
              if (tid == 0) __hip_atomic_store(split_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        if (finish) {
  #pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t m = lo + qrow(i);
            if (m >= hi) continue;
  #pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int64_t n = n0 + qcol(j);
              if (n >= a.N) continue;
              f32x4 v = acc[i][j];
              if (FP8) v *= a.scale;
              u32x2 packed;
              packed[0] = bf16x2_rne(v[0], v[1]);
              packed[1] = bf16x2_rne(v[2], v[3]);
              *reinterpret_cast<u32x2*>(a.c + m * a.N + n) = packed;
            }
          }
        }
      } else if (EPI == kEpiAllReduce) {
        // One-shot AllReduce, fused: this tile's partial goes to `send` (what every peer receives;
        // write-through, so it is visible everywhere once the stores complete) and the tile that
        // completes a chunk of `send` raises its send flag; then, once every peer's chunks of these
        // rows have arrived, out = partial + the peers' partials in ascending rank order (a fixed
        // order: `out` does not depend on arrival order).
        const int64_t MN = a.M * a.N;
        const __amdgpu_buffer_rsrc_t rsend = __builtin_amdgcn_make_buffer_rsrc(a.send, 0, (int)(MN * 4), kBufferFlags);
        const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, (int)(MN * 4), kBufferFlags);
        const __amdgpu_buffer_rsrc_t rrecv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.recv), 0, (int)(a.world * MN * 4), kBufferFlags);
  #pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int64_t m = lo + qrow(i);
          if (m >= hi) continue;
  #pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + qcol(j);
            if (n >= a.N) continue;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rsend,
                                                   (int)((m * a.N + n) * 4), 0, kStoreSystemCoherent);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // one lane per chunk of the tile's rows, so the counts are one round trip (the chunks'
        // counters are shared by every column tile, and one after another they cost the tile
        // several microseconds)
        if (wave == 0) {
          const int q_lo = (int)(lo / a.chunk_rows), q_hi = (int)((hi - 1) / a.chunk_rows);
          for (int q = q_lo + lane; q <= q_hi; q += kWaveLanes) {
            const int64_t clo = (int64_t)q * a.chunk_rows;
            const int64_t chi = clo + a.chunk_rows;
            const int t_first = (int)(clo / BM), t_last = (int)((chi - 1) / BM);
            const uint32_t expect = (uint32_t)(t_last - t_first + 1) * (uint32_t)a.n_col_tiles;
            const uint32_t prev = __hip_atomic_fetch_add(a.scratch + kScrRsCount + q, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (prev + 1 == expect)
              __hip_atomic_store(a.send_flags + q, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          }
        }
        if (wave == 0) {
          uint32_t seen = 0xFFFFFFFFu;
          const bool ok = wait_chunks<kEpiAllReduce>(a, lo, hi, 0, seen);
          if (lane == 0) {
            s_ok = ok;
            if (trec) { trec[3] = seen; trec[6] = wall_ticks(); }
          }
        }
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(s_ok)) {
          // the peers' partials: system-coherent loads (read once; no L2 invalidate)
          const int world = __builtin_amdgcn_readfirstlane(a.world), rank = __builtin_amdgcn_readfirstlane(a.rank);
  #pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t m = lo + qrow(i);
  #pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int64_t n = n0 + qcol(j);
              if (m >= hi || n >= a.N) continue;
              // every peer's quad in flight, then added in rank order
              f32x4 in[AGG_MAX_WORLD - 1];
  #pragma unroll
              for (int q = 0; q < AGG_MAX_WORLD - 1; ++q) {
                const int p = q < rank ? q : q + 1;
                const int off = p < world ? (int)(((int64_t)p * MN + m * a.N + n) * 4) : (int)kOutOfRange;
                in[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrecv, off, 0, kStoreSystemCoherent));
              }
              f32x4 v = acc[i][j];
  #pragma unroll
              for (int q = 0; q < AGG_MAX_WORLD - 1; ++q)
                if (q + 1 < world) v += in[q];
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rout, (int)((m * a.N + n) * 4), 0, 0);
            }
          }
        }
      } else {
        const int64_t base = (int64_t)block * a.m_block;
        const bool local = (block == a.rank);
        const int slot = block < a.rank ? block : block - 1;
        const int64_t blk = a.m_block * a.N;    // floats per block
        if (!local) {
          // a non-local block's partial goes to `send` with write-through stores, so it is visible
          // everywhere once they complete (no L2 writeback before the flag)
          const __amdgpu_buffer_rsrc_t rsend = __builtin_amdgcn_make_buffer_rsrc(
              a.send, 0, (int)((a.world - 1) * blk * 4), kBufferFlags);
  #pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t m = lo + qrow(i);
            if (m >= hi) continue;
  #pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int64_t n = n0 + qcol(j);
              if (n >= a.N) continue;
              __builtin_amdgcn_raw_buffer_store_b128(
                  __builtin_bit_cast(u32x4, acc[i][j]), rsend,
                  (int)(((int64_t)slot * blk + (m - base) * a.N + n) * 4), 0, kStoreSystemCoherent);
            }
          }
        } else {
          if (EPI == kEpiReduceScatter && a.fuse_local) {
            // the local block: once every peer's chunks of these rows have arrived, out = partial +
            // the peers' partials in ascending rank order. The partial goes through LDS (the operand
            // stages, free after the K loop) in passes of RP rows, so that all threads then read
            // whole rows of the peers' blocks (coalesced) while no accumulator is held beside them
            if (wave == 0) {
              uint32_t seen = 0xFFFFFFFFu;
              const bool ok = wait_chunks<EPI>(a, lo, hi, block, seen);
              if (lane == 0) s_ok = ok;
            }
            __syncthreads();
            const bool all_in = __builtin_amdgcn_readfirstlane(s_ok) != 0;
            constexpr int RP0 = (kStageBytes / (BN * 4)) / WTM * WTM;
            constexpr int RP = RP0 < BM ? RP0 : BM;
            static_assert(RP >= WTM && RP % WTM == 0 && RP * BN * 4 <= kStageBytes, "LDS passes");
            constexpr int Q4 = BN / 4, NE = RP * Q4, U = 2;
            float* const tl = reinterpret_cast<float*>(stages);
            const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
                a.out, 0, (int)(blk * 4), kBufferFlags);
            const __amdgpu_buffer_rsrc_t rrecv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.recv), 0, (int)(a.world * blk * 4), kBufferFlags);
            const int world = __builtin_amdgcn_readfirstlane(a.world), rank = __builtin_amdgcn_readfirstlane(a.rank);
            for (int p0 = 0; p0 < BM; p0 += RP) {
              if (wm * WTM >= p0 && wm * WTM < p0 + RP) {
    #pragma unroll
                for (int i = 0; i < FM; ++i)
    #pragma unroll
                  for (int j = 0; j < FN; ++j)
                    *reinterpret_cast<f32x4*>(tl + (qrow(i) - p0) * BN + qcol(j)) = acc[i][j];
              }
              __syncthreads();
              for (int e0 = tid; e0 < NE; e0 += NT * U) {
                f32x4 v[U], in[U][AGG_MAX_WORLD - 1];
                int64_t mo[U];
                bool ok[U];
    #pragma unroll
                for (int u = 0; u < U; ++u) {
                  const int e = e0 + u * NT;
                  const int r = e / Q4, c4 = e - (e / Q4) * Q4;
                  const int64_t m = lo + p0 + r, n = n0 + 4 * c4;
                  ok[u] = e < NE && m < hi && n < a.N;
                  mo[u] = (m - base) * a.N + n;
                  v[u] = ok[u] ? *reinterpret_cast<const f32x4*>(tl + r * BN + 4 * c4) : f32x4{};
    #pragma unroll
                  for (int q = 0; q < AGG_MAX_WORLD - 1; ++q) {
                    const int p = q < rank ? q : q + 1;
                    const int off = (ok[u] && all_in && p < world) ? (int)(((int64_t)p * blk + mo[u]) * 4) : (int)kOutOfRange;
                    in[u][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrecv, off, 0, kStoreSystemCoherent));
                  }
                }
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int u = 0; u < U; ++u) {
                  if (!ok[u]) continue;
                  if (all_in) {
    #pragma unroll
                    for (int q = 0; q < AGG_MAX_WORLD - 1; ++q)
                      if (q + 1 < world) v[u] += in[u][q];
                  }
                  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[u]), rout, (int)(mo[u] * 4), 0, 0);
                }
              }
              __syncthreads();
            }
          } else {
            // the local block: the tile's partial goes to `out` (write-through, like `send`); the
            // peers' partials are added after the last tile by reduce_local
            const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
                a.out, 0, (int)(blk * 4), kBufferFlags);
    #pragma unroll
            for (int i = 0; i < FM; ++i) {
              const int64_t m = lo + qrow(i);
              if (m >= hi) continue;
    #pragma unroll
              for (int j = 0; j < FN; ++j) {
                const int64_t n = n0 + qcol(j);
                if (n >= a.N) continue;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rout,
                                                       (int)(((m - base) * a.N + n) * 4), 0, kStoreSystemCoherent);
              }
            }
            // once the stores have completed, count the tile in its row tile
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
              __hip_atomic_fetch_add(a.scratch + kScrLocal + tib, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        if (!local) {
          // publish: once every thread's write-through stores have completed, this tile's rows of
          // `send` are final for its column range; the tile that completes a send chunk raises
          // its flag (a system-coherent store)
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (wave == 0) {
            // one lane per send chunk of the tile's rows: the counts in one round trip
            const int64_t rlo = lo - base, rhi = hi - base;
            const int q_lo = (int)(rlo / a.chunk_rows), q_hi = (int)((rhi - 1) / a.chunk_rows);
            for (int q = q_lo + lane; q <= q_hi; q += kWaveLanes) {
              // tiles overlapping chunk q of this block, times the column tiles
              const int64_t clo = (int64_t)q * a.chunk_rows;
              const int64_t chi = clo + a.chunk_rows;
              const int t_first = (int)(clo / BM), t_last = (int)((chi - 1) / BM);
              const uint32_t expect = (uint32_t)(t_last - t_first + 1) * (uint32_t)a.n_col_tiles;
              const int c = block * a.cps + q;
              const uint32_t prev = __hip_atomic_fetch_add(a.scratch + kScrRsCount + c, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
              if (prev + 1 == expect)
                __hip_atomic_store(a.send_flags + c, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
          }
        }
      }
      if (tid == 0 && trec) {
        trec[7] = wall_ticks();
        atomicAdd(trec + 4, 1u);
      }
      // s_tile / s_ok are rewritten by the next claim only after every thread passed here
      __syncthreads();
    };
    if (EPI == kEpiFfn && __builtin_amdgcn_readfirstlane(s_tile[2]) == 1) tile_body(std::true_type{});
    else tile_body(std::false_type{});
  }

  // (only a launch that computes the tiles reduces: a copy-only launch leaves `out` alone)
  if (((EPI == kEpiReduceScatter && !a.fuse_local) || EPI == kEpiFfn) && a.n_row_tiles > 0)
    reduce_local<BM>(a, tid, &s_job, &s_ok);

  // ---- the last workgroup resets the counters for the next launch. No fence: every counter
  // reset here was last touched by the other workgroups through atomics whose returned values
  // they used, i.e. that had completed, before they counted themselves done (the local row-tile
  // counts were read to their final values by the reduction's waits, the split-K counts by every
  // part's wait).
  if (tid == 0) {
    const uint32_t prev = atomicAdd(a.scratch + kScrDone, 1u);
    s_ok = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_ok)) {
    if (tid < kMaxLists) __hip_atomic_store(a.scratch + kScrLists + tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.copy_jobs) {
      if (tid == 0) {
        __hip_atomic_store(a.scratch + kScrCopyNext, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.scratch + kScrCopyT0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int set = 0; set < 2; ++set) {
        const CopySet& cs = a.cs[set];
        for (uint32_t i = tid; i * (uint32_t)cs.pieces < cs.jobs; i += NT)
          __hip_atomic_store(a.scratch + kScrPieces + cs.piece_off + a.scratch[kScrOrder + cs.order_off + i], 0u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (EPI == kEpiAllReduce) {
      for (int i = tid; i < a.cps; i += NT)
        __hip_atomic_store(a.scratch + kScrRsCount + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (EPI == kEpiFfn) {
      for (int i = tid; i < a.n_row_tiles1; i += NT)
        __hip_atomic_store(a.scratch + kScrSplit + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (EPI == kEpiAllGather && kSplitTiles && a.ksplit > 1) {
      // split-K tile counters (a launch whose parts all ran together leaves them at ksplit)
      for (int i = tid; i < a.n_row_tiles * (a.n_col_tiles / a.ksplit); i += NT)
        __hip_atomic_store(a.scratch + kScrSplit + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (EPI == kEpiReduceScatter || EPI == kEpiFfn) {
      for (int i = tid; i < a.world * a.cps; i += NT)
        __hip_atomic_store(a.scratch + kScrRsCount + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = tid; i < a.tpb; i += NT)
        __hip_atomic_store(a.scratch + kScrLocal + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) __hip_atomic_store(a.scratch + kScrRedNext, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.scratch + kScrDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The producer as a kernel of its own: every workgroup is one wave that takes copy jobs (set 0's,
// then set 1's, in arrival order) from the shared counter until none is left, copying each piece
// with a few vectors per lane in flight (so that it fits in the registers the GEMM kernel leaves
// free on each SIMD); the wave that completes a chunk releases its flag. Workgroup 0 first raises
// the local slots' flags. The last workgroup to finish clears the counters for the next launch.
__global__ void __launch_bounds__(64) copy_kernel(const GemmArgs a) {
  const int lane = threadIdx.x;
  if (blockIdx.x == 0) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
      for (int i = lane; i < a.mark_count[f]; i += 64)
        __hip_atomic_store(a.mark_flags[f] + i, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  const uint32_t* order = a.scratch + kScrOrder;
  const uint32_t jobs = __builtin_amdgcn_readfirstlane(a.copy_jobs);
  const uint32_t jobs0 = __builtin_amdgcn_readfirstlane(a.cs[0].jobs);
  // The next job, taken with no lane-dependent branch: every lane joins the add (lane 0 adds 1,
  // the others 0) and lane 0's result, the count before its own 1, is the job. (A fetch under
  // `if (lane == 0)` followed by a cross-lane read lets the compiler lay the loop out as two
  // nested loops, lane 0 in the outer one, and the cross-lane read then misses lane 0.)
  auto next_job = [&]() -> uint32_t {
    const uint32_t cur = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(a.scratch + kScrCopyNext, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (cur >= jobs) return jobs;
    return __builtin_amdgcn_readfirstlane(atomicAdd(a.scratch + kScrCopyNext, lane == 0 ? 1u : 0u));
  };
  for (uint32_t job = next_job(); job < jobs; job = next_job()) {
    const int set = job < jobs0 ? 0 : 1;
    const CopySet& cs = a.cs[set];
    const uint32_t pieces = __builtin_amdgcn_readfirstlane((uint32_t)cs.pieces);
    const uint32_t jj = job - (set ? jobs0 : 0u);
    const uint32_t j = jj / pieces, q = jj - j * pieces;
    const int c = (int)__builtin_amdgcn_readfirstlane(order[cs.order_off + j]);
    const int p = c / cs.cps, jl = c - p * cs.cps;
    const int64_t base = (int64_t)jl * cs.chunk_bytes;
    const int64_t held = clamp_bytes(cs.valid_bytes[p] - base, cs.chunk_bytes);
    const int64_t lo = min_i64((int64_t)q * cs.piece_bytes, held);
    const int64_t hi = min_i64(lo + cs.piece_bytes, held);
    copy_piece<64, 2>(cs.sym + ((int64_t)p * cs.cps) * cs.chunk_bytes + base + lo, cs.peer[p] + base + lo,
                      hi - lo, lane);
    // the wave's write-through stores have completed (copy_piece waited for them)
    if (lane == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(a.scratch + kScrPieces + cs.piece_off + c, 1u,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev + 1 == pieces)
        __hip_atomic_store(cs.put_flags + c, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  // the last wave out clears the job counter and every chunk's piece count (the same
  // branch-free count as the job fetch)
  const uint32_t done = __builtin_amdgcn_readfirstlane(atomicAdd(a.scratch + kScrCopyDone, lane == 0 ? 1u : 0u));
  if (done == gridDim.x - 1) {
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      const CopySet& cs = a.cs[set];
      for (uint32_t i = lane; i * (uint32_t)cs.pieces < cs.jobs; i += 64)
        __hip_atomic_store(a.scratch + kScrPieces + cs.piece_off + a.scratch[kScrOrder + cs.order_off + i], 0u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) {
      __hip_atomic_store(a.scratch + kScrCopyNext, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.scratch + kScrCopyDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_copy(const GemmArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(64), 0, stream, args);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* dst, size_t words, uint32_t value) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

// With timing events, the launch carries them (the dispatch's own start and end timestamps), so
// timing adds no packets to the stream between launches.
template <int BM, int BN, int DT, int EPI>
static hipError_t launch_one(const GemmArgs& args, int grid, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (t0 || t1)
    hipExtLaunchKernelGGL((gemm_kernel<BM, BN, DT, EPI>), dim3(grid), dim3(kThreads), 0, stream, t0, t1, 0, args);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, DT, EPI>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

__global__ void copy_kernel(const GemmArgs a);

template <int BM, int BN, int DT, int EPI>
static int regs_one() {
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(gemm_kernel<BM, BN, DT, EPI>)) != hipSuccess)
    return -1;
  return attr.numRegs;
}

template <int DT, int EPI>
static int regs_shape(int bm, int bn) {
  if (bm == 256 && bn == 256) return regs_one<256, 256, DT, EPI>();
  if (bm == 256 && bn == 224) return regs_one<256, 224, DT, EPI>();
  if (bm == 128 && bn == 128) return regs_one<128, 128, DT, EPI>();
  if (bm == 128 && bn == 64) return regs_one<128, 64, DT, EPI>();
  if (bm == 64 && bn == 64) return regs_one<64, 64, DT, EPI>();
  return -1;
}

int kernel_regs(int bm, int bn, int dtype, int epilogue) {
  if (epilogue == kEpiAllGather) {
    if (dtype == AGG_BF16) return regs_shape<AGG_BF16, kEpiAllGather>(bm, bn);
    if (dtype == AGG_FP8_E4M3) return regs_shape<AGG_FP8_E4M3, kEpiAllGather>(bm, bn);
  } else if (epilogue == kEpiReduceScatter && dtype == AGG_BF16) {
    return regs_shape<AGG_BF16, kEpiReduceScatter>(bm, bn);
  } else if (epilogue == kEpiAllReduce && dtype == AGG_BF16) {
    return regs_shape<AGG_BF16, kEpiAllReduce>(bm, bn);
  } else if (epilogue == kEpiFfn && dtype == AGG_BF16 && bm == 256 && bn == 256) {
    return regs_one<256, 256, AGG_BF16, kEpiFfn>();
  }
  return -1;
}

int copy_kernel_regs() {
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(copy_kernel)) != hipSuccess) return -1;
  return attr.numRegs;
}

template <int BM, int BN, int DT, int EPI>
static int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_kernel<BM, BN, DT, EPI>, kThreads, 0) != hipSuccess)
    return 0;
  return n;
}

template <int DT, int EPI>
static int occupancy_shape(int bm, int bn) {
  if (bm == 256 && bn == 256) return occupancy_one<256, 256, DT, EPI>();
  if (bm == 256 && bn == 224) return occupancy_one<256, 224, DT, EPI>();
  if (bm == 128 && bn == 128) return occupancy_one<128, 128, DT, EPI>();
  if (bm == 128 && bn == 64) return occupancy_one<128, 64, DT, EPI>();
  if (bm == 64 && bn == 64) return occupancy_one<64, 64, DT, EPI>();
  return 0;
}

int max_blocks_per_cu(int bm, int bn, int dtype, int epilogue) {
  if (epilogue == kEpiAllGather) {
    if (dtype == AGG_BF16) return occupancy_shape<AGG_BF16, kEpiAllGather>(bm, bn);
    if (dtype == AGG_FP8_E4M3) return occupancy_shape<AGG_FP8_E4M3, kEpiAllGather>(bm, bn);
  } else if (epilogue == kEpiReduceScatter && dtype == AGG_BF16) {
    return occupancy_shape<AGG_BF16, kEpiReduceScatter>(bm, bn);
  } else if (epilogue == kEpiAllReduce && dtype == AGG_BF16) {
    return occupancy_shape<AGG_BF16, kEpiAllReduce>(bm, bn);
  } else if (epilogue == kEpiFfn && dtype == AGG_BF16 && bm == 256 && bn == 256) {
    return occupancy_one<256, 256, AGG_BF16, kEpiFfn>();
  }
  return 0;
}

template <int DT, int EPI>
static hipError_t launch_shape(const GemmArgs& args, int bm, int bn, int grid, hipStream_t s, hipEvent_t t0,
                               hipEvent_t t1) {
  if (bm == 256 && bn == 256) return launch_one<256, 256, DT, EPI>(args, grid, s, t0, t1);
  if (bm == 256 && bn == 224) return launch_one<256, 224, DT, EPI>(args, grid, s, t0, t1);
  if (bm == 128 && bn == 128) return launch_one<128, 128, DT, EPI>(args, grid, s, t0, t1);
  if (bm == 128 && bn == 64) return launch_one<128, 64, DT, EPI>(args, grid, s, t0, t1);
  if (bm == 64 && bn == 64) return launch_one<64, 64, DT, EPI>(args, grid, s, t0, t1);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& args, int bm, int bn, int dtype, int epilogue, int grid,
                       hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (epilogue == kEpiAllGather) {
    if (dtype == AGG_BF16) return launch_shape<AGG_BF16, kEpiAllGather>(args, bm, bn, grid, stream, t0, t1);
    if (dtype == AGG_FP8_E4M3)
      return launch_shape<AGG_FP8_E4M3, kEpiAllGather>(args, bm, bn, grid, stream, t0, t1);
  } else if (epilogue == kEpiReduceScatter && dtype == AGG_BF16) {
    return launch_shape<AGG_BF16, kEpiReduceScatter>(args, bm, bn, grid, stream, t0, t1);
  } else if (epilogue == kEpiAllReduce && dtype == AGG_BF16) {
    return launch_shape<AGG_BF16, kEpiAllReduce>(args, bm, bn, grid, stream, t0, t1);
  } else if (epilogue == kEpiFfn && dtype == AGG_BF16 && bm == 256 && bn == 256) {
    return launch_one<256, 256, AGG_BF16, kEpiFfn>(args, grid, stream, t0, t1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fill_u32(uint32_t* dst, size_t words, uint32_t value, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, words, value);
  return hipGetLastError();
}

}  // namespace agg
