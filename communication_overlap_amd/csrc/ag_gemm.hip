// AllGather -> GEMM with tile-level producer/consumer overlap
// ("Triton-distributed Semantics", Kernel Design Patterns, "AllGather and
// GEMM Overlapping"; Producer-Consumer Model; Threadblock Swizzling).
//
// One persistent launch.  All workgroups first copy, together, the units the
// first round of consumer tiles needs; then workgroups [0, P) are producers:
// they take the remaining flag units in the caller's producer order, copy
// each unit's rows and K-range from its shard into the gathered buffer with
// 16-byte vectors, and publish the unit's flag (agent-scope release).  Workgroups [P, P + C) are
// consumers: each computes output tiles in arrival order; before the K-step
// that enters a new K-batch it waits (wave-level acquire) on every unit that
// covers the tile's rows in that batch, then loads the A tile from the
// gathered buffer.  Tiles whose rows are all the own rank's read the own
// shard directly and never wait.
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "device.h"
#include "gemm_core.h"
#include "host.h"

namespace ovl {

constexpr int kMaxRanks = 16;
constexpr int kMaxUnitProducers = 16;
constexpr int kMaxRowTiles = 1024;  // consumer-order table held in LDS
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies, each with its own L2

struct AgArgs {
  const uint16_t* shards[kMaxRanks];
  const uint16_t* b;
  uint16_t* g;
  float* c;
  int64_t* flags;
  ErrRec* err;
  const int32_t* order;
  int64_t shard_m, m, k, n;
  int64_t flag_stride;  // in int64 slots
  int64_t epoch;
  uint64_t spin_limit;
  int32_t ranks, rank;
  int32_t unit_rows, panels, batches, batch_cols;
  int32_t num_units;
  int32_t producers, consumers;
  int32_t tiles_m, tiles_n;
  // Split K: each output tile is computed as `splits` column ranges of A
  // (split_cols wide); each range's fp32 product goes to partial[s], and C
  // is their sum in range order.  With split_sync (every range of the launch
  // runs in its first round, so the ranges of a tile run at the same time)
  // the ranges wait for each other on counters[2 * tile] and each sums one
  // stripe of rows; otherwise the last range to arrive sums the whole tile.
  int32_t splits, split_cols, split_sync;
  float* partial;     // [splits][m][n]
  int64_t* counters;  // [tiles][2], zero between launches
  int64_t* trace;     // optional timestamps: [num_units] publishes, then [items][kTraceItem]
  uint32_t jitter;    // producers sleep up to this many intervals before each unit (test aid)
  int32_t unit_producers;  // W: workgroups that move one unit together (1: one publisher)
  int64_t* arrivals;       // [num_units] monotone arrival counters (W > 1)
};

constexpr int kTraceItem = 6;  // int64 per traced work item

constexpr int kMaxSplits = 8;

enum { kModeFused = 0, kModeBarrier = 1, kModeGemmOnly = 2 };

// The consumer tile configurations: BM x BN output tile, K step BK, NS LDS
// stages, NW wavefronts; SPLIT marks the one that carries the split-K
// epilogue (the others keep their registers for the main loop).
//  - big: 256 x 256, 8 waves in a 2 x 4 grid, two per SIMD (one's MFMAs
//    cover the other's LDS reads; measured faster than 4);
//  - small: 128 x 128, 4 waves;
//  - split (skinny, bandwidth-bound shapes, K split over workgroups): short
//    K steps through a deep ring, so that more of B is in flight when a
//    step waits for its stage.
template <int BM_, int BN_, int BK_, int NS_, int NW_, bool SPLIT_, int NL_ = NW_>
struct AgTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_, NW = NW_;
  static constexpr bool SPLIT = SPLIT_;
  static constexpr int NL = NL_;  // waves that issue the stage loads (gemm_tile)
};
using TileBig = AgTile<256, 256, 64, 2, 8, false>;
using TileSmall = AgTile<128, 128, 64, 2, 4, false>;
// Eight waves (two per SIMD): skinny 128x7168x8192 fused 50.3-50.4 -> 49.1-49.7 us,
// GEMM only the same within 2%.
constexpr int kSplitBN = 128, kSplitBK = 64, kSplitStages = 4, kSplitWaves = 8;
using TileSplit = AgTile<128, kSplitBN, kSplitBK, kSplitStages, kSplitWaves, true>;
constexpr int kMaxWaves = 8;

}  // namespace ovl

// The allocation-free variant's workspace (ag_gemm_run_noalloc): a file-scope
// device array, one copy per GPU, kept until the process ends.  A plan with
// one producer per unit always fits: a K split runs at most 224 tile ranges
// of 128 x 128 fp32 partials (14 MiB), and an unsplit plan needs only the
// 256-byte error record; several producers per unit add 8 bytes per unit.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace ovl {

// ---------------------------------------------------------------- producer

// Copies rows x cols bf16 (cols a multiple of 8) between two row-major
// matrices of row pitch ld, 16 bytes per lane, in blocks of U vectors per
// lane; the (row, vector) position advances incrementally, without a
// division per vector.  The loads of block i+1 are issued before the stores
// of block i, so that a lane always has a block in flight (vector memory
// counters complete in order: waiting for the loads does not wait for the
// stores issued after them).  Loads and stores are buffer operations with
// no branch around them (a vector past the end gets an offset past the
// buffer: the load returns zeros, the store is dropped): guarded one by one,
// they made the compiler wait for every load in flight before each store.
template <int NT, bool AGENT = false>
__device__ inline void copy_block(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t rows,
                                  int64_t cols, int64_t ld) {
  constexpr int U = 8;
  const rsrc_t sr = make_rsrc(src, rows * ld * 2);
  const rsrc_t dr = make_rsrc(dst, rows * ld * 2);
  const uint32_t vpr = (uint32_t)(cols / 8);
  const uint32_t total = (uint32_t)(rows * vpr);
  const uint32_t step_r = NT / vpr, step_c = NT % vpr;
  uint32_t r = threadIdx.x / vpr, c = threadIdx.x % vpr;  // next vector to load
  const uint32_t blocks = (total + NT * U - 1) / (NT * U);
  struct Blk {
    u32x4 v[U];
    uint32_t off[U];  // byte offset, or kOOB past the end
  };
  auto load = [&](uint32_t bi, Blk& b) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const bool in = bi * NT * U + j * NT + threadIdx.x < total;
      b.off[j] = in ? (r * (uint32_t)ld + c * 8) * 2 : kOOB;
      b.v[j] = __builtin_amdgcn_raw_buffer_load_b128(sr, (int)b.off[j], 0, 0);
      c += step_c;
      r += step_r;
      if (c >= vpr) {
        c -= vpr;
        ++r;
      }
    }
  };
  auto store = [&](const Blk& b) {
#pragma unroll
    for (int j = 0; j < U; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(b.v[j], dr, (int)b.off[j], 0, AGENT ? kAuxAgent : 0);
  };
  Blk x, y;
  if (blocks > 0) load(0, x);
  for (uint32_t bi = 0; bi < blocks; bi += 2) {
    if (bi + 1 < blocks) load(bi + 1, y);
    store(x);
    if (bi + 1 >= blocks) break;
    if (bi + 2 < blocks) load(bi + 2, x);
    store(y);
  }
}

// What every workgroup knows of the schedule (tables in LDS, built by
// build_schedule): the row tiles in consumer order, each row tile's position
// in it, and the bootstrap: the panels (sp = shard * panels + panel) that the
// first round of consumer tiles reads, whose units all workgroups move
// together before anything else.
struct Sched {
  int* sorted;         // [tiles_m] row tiles in consumer order
  int* pos;            // [tiles_m] position of each row tile in `sorted`
  int* boot;           // [n_boot] bootstrap panels, ascending
  int* bidx;           // [ranks * panels] index in `boot`, or -1
  uint32_t* present;   // bit i * batches + bt: unit (boot[i], bt) occurs in the producer order
  int n_boot;
  int rows1;           // row-tile positions [0, rows1) are read by the first round
};

constexpr int kBootBits = 2048 * 32;  // presence bitmap: n_boot * batches <= this

// Geometry of flag unit u: rows [r0, r0 + rows) of shard s, columns
// [c0, c0 + cols).
struct UnitBox {
  int s;
  int64_t r0, rows, c0, cols;
};

__device__ inline UnitBox unit_box(const AgArgs& a, int u) {
  const int bt = u % a.batches;
  const int sp = u / a.batches;
  const int p = sp % a.panels;
  UnitBox x;
  x.s = sp / a.panels;
  x.r0 = (int64_t)p * a.unit_rows;
  x.rows = min((int64_t)a.unit_rows, a.shard_m - x.r0);
  x.c0 = (int64_t)bt * a.batch_cols;
  x.cols = min((int64_t)a.batch_cols, a.k - x.c0);
  return x;
}

// Copies rows [r0, r0 + rows) of unit box x (agent: with agent-scope stores).
template <int NT>
__device__ inline void copy_unit_rows(const AgArgs& a, const UnitBox& x, int64_t r0, int64_t rows, bool agent) {
  const uint16_t* src = a.shards[x.s] + r0 * a.k + x.c0;
  uint16_t* dst = a.g + ((int64_t)x.s * a.shard_m + r0) * a.k + x.c0;
  if (agent)
    copy_block<NT, true>(src, dst, rows, x.cols, a.k);
  else
    copy_block<NT>(src, dst, rows, x.cols, a.k);
}

// Copies one flag unit into the gathered buffer and publishes its flag (NT
// threads per workgroup).
// `agent`: the unit is written with agent-scope stores and published
// without the release fence.  Used for the bootstrap units (moved by every
// workgroup at once), small units (at most 64 KiB) and the copy-only
// launch: there the per-die serialised L2 writebacks of the fences, not the
// bytes, bound the copy (skinny 128x7168x8192 fused 61.0 -> 58.6 us; the
// 8192 x 4096 copy alone 41 -> 33 us).  Large units of the fused launch's
// producers keep plain stores and the fence: with agent-scope stores there
// the copy ran beside the GEMM's traffic slower (last unit published at
// 146 against 127 us) and the fused launch took 250-253 against 240-242 us.
// With several producers per unit (unit_producers = W > 1) a unit moved
// whole by one workgroup also adds W to its arrival counter, which keeps the
// counter at a multiple of W after every run.
template <int NT>
__device__ inline void move_unit(const AgArgs& a, int u, bool agent_hint = false) {
  const UnitBox x = unit_box(a, u);
  const bool agent = agent_hint || x.rows * x.cols * 2 <= 64 * 1024;
  int64_t* flag = a.flags + (int64_t)u * a.flag_stride;
  copy_unit_rows<NT>(a, x, x.r0, x.rows, agent);
  if (agent) {
    wave_drain();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    wg_publish(flag, a.epoch);
  }
  if (threadIdx.x == 0) {
    if (a.unit_producers > 1)
      __hip_atomic_fetch_add(a.arrivals + u, (int64_t)a.unit_producers, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.trace) a.trace[u] = now_ticks();
  }
}

// Piece `piece` of W of unit u (rows split evenly; a piece may be empty):
// the split-unit signal ADD ("Triton-distributed Semantics", Runtime
// Implementation of Communication Primitives: signal SET and ADD).  The
// workgroup copies its rows, then arrives once on the unit's counter; the
// counter is never reset (it only grows, by exactly W per run), so the
// arrival that brings it to a multiple of W is the unit's last, whatever
// the epoch, and that workgroup publishes the flag.  Ordering: plain stores
// are released by an agent-scope fence before the add and the last
// arriver acquires the others' releases before its release store of the
// flag; agent-scope stores are complete once drained, so those pieces add
// and publish without fences (as move_unit's agent path).
template <int NT>
__device__ inline void move_piece(const AgArgs& a, int u, int piece, bool agent_hint) {
  const UnitBox x = unit_box(a, u);
  const int W = a.unit_producers;
  const int64_t lo = x.r0 + x.rows * piece / W, hi = x.r0 + x.rows * (piece + 1) / W;
  const bool agent = agent_hint || (hi - lo) * x.cols * 2 <= 64 * 1024;
  copy_unit_rows<NT>(a, x, lo, hi - lo, agent);
  wave_drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t* flag = a.flags + (int64_t)u * a.flag_stride;
    if (!agent) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int64_t old = __hip_atomic_fetch_add(a.arrivals + u, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old % W == W - 1) {
      if (agent) {
        __hip_atomic_store(flag, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(flag, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (a.trace) a.trace[u] = now_ticks();
    }
  }
  // Separates this thread-0 branch from the caller's next one.
  __syncthreads();
}

// Test aid: a pause of h(u, epoch) mod (jitter + 1) sleeps of about 64
// clocks before unit u (or piece u of the split units' pieces) is moved, h
// a fixed integer hash, so that units land in an uneven, shuffled order.
__device__ inline void jitter_pause(const AgArgs& a, int u) {
  uint32_t h = (uint32_t)u * 0x9E3779B1u ^ (uint32_t)a.epoch * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t n = uniform((int)(h % (a.jitter + 1)));
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
}

// Moves the units at producer-order positions w, w + P, ..., skipping the
// bootstrap panels' units when sc is given (those were moved already).  With
// W producers per unit the work items are (position, piece) pairs, the W
// pieces of a unit consecutive, so that W producers move a unit at once.
template <int NT>
__device__ inline void produce(const AgArgs& a, int w, int P, const Sched* sc, bool agent = false) {
  const int W = a.unit_producers;
  const int items = a.num_units * W;
  for (int i = w; i < items; i += P) {
    const int pos = W == 1 ? i : i / W;
    const int u = uniform(a.order ? a.order[pos] : pos);
    if (u < 0 || u >= a.num_units) continue;  // not a unit index: nothing to move
    // Bootstrap units were moved already.  The bootstrap is off (n_boot = 0)
    // when the panels outnumber the bidx table, which then holds no entry for
    // most panels.
    if (sc && sc->n_boot > 0 && uniform(sc->bidx[u / a.batches]) >= 0) continue;
    if (a.jitter) jitter_pause(a, W == 1 ? u : u * W + i % W);
    if (W == 1)
      move_unit<NT>(a, u, agent);
    else
      move_piece<NT>(a, u, i % W, agent);
  }
}

// Bootstrap: workgroup w of G moves the bootstrap units number w, w + G, ...
// (every K-batch of every bootstrap panel, panel-major) that occur in the
// producer order; a unit the order omits stays unmoved.
template <int NT>
__device__ inline void produce_boot(const AgArgs& a, int w, int G, const Sched& sc) {
  // A loop around barriers: its bound and counter are scalars to the compiler.
  const int items = uniform(sc.n_boot * a.batches);
  for (int i = w; uniform(i) < items; i += G)
    if (uniform((sc.present[i >> 5] >> (i & 31)) & 1u))
      move_unit<NT>(a, uniform(sc.boot[i / a.batches]) * a.batches + i % a.batches, true);
}

__global__ __launch_bounds__(kThreads) void ag_produce_kernel(AgArgs a) {
  produce<kThreads>(a, blockIdx.x, gridDim.x, nullptr, true);
}

// ---------------------------------------------------------------- consumer order

// Row tile rt covers gathered rows [rt*BM, min((rt+1)*BM, m)).  It is "own"
// when all of them belong to the own rank's shard.
__device__ inline bool row_tile_own(const AgArgs& a, int BM, int rt) {
  const int64_t lo = (int64_t)rt * BM, hi = min(lo + BM, a.m);
  return lo >= (int64_t)a.rank * a.shard_m && hi <= (int64_t)(a.rank + 1) * a.shard_m;
}

// True when a consumer of the first round reads panel sp from the gathered
// buffer: some row tile that the panel's rows fall in is in the first round
// and is not an own tile (own tiles read the own shard directly).
__device__ inline bool panel_is_boot(const AgArgs& a, int BM, const int* pos, int rows1, int sp) {
  const int p = sp % a.panels, s = sp / a.panels;
  const int64_t r_lo = (int64_t)s * a.shard_m + (int64_t)p * a.unit_rows;
  const int64_t r_hi = min(r_lo + a.unit_rows, (int64_t)(s + 1) * a.shard_m);
  for (int rt = (int)(r_lo / BM); rt <= (int)((r_hi - 1) / BM); ++rt)
    if (pos[rt] < rows1 && !row_tile_own(a, BM, rt)) return true;
  return false;
}

// LDS the schedule tables take: the consumer order sits after the GEMM
// stages (consumers read it throughout); the tables only the bootstrap and
// the producers use alias the start of the stage area, which consumers
// overwrite once the bootstrap is done.
constexpr int kOrderBytes = kMaxRowTiles * (int)sizeof(int);
constexpr int kBootTabBytes = (3 * kMaxRowTiles + kBootBits / 32) * (int)sizeof(int);

// Builds the schedule tables in LDS at `tab` (identical in every
// workgroup).  The consumer order puts the own row tiles first (ascending),
// then the others by the latest producer-order position among the
// first-K-batch units that cover their rows (ties by index).  The bootstrap
// is left empty when `with_boot` is false or the panels outnumber the
// table, and keeps only as many panels as the presence bitmap holds.
__device__ Sched build_schedule(const AgArgs& a, int BM, int* sorted, int* tab, bool with_boot) {
  __shared__ int s_nboot;
  __shared__ int s_wave[kMaxWaves];
  int* key = tab;  // reused as bidx once the order is known
  int* pos = tab + kMaxRowTiles;
  int* boot = pos + kMaxRowTiles;
  uint32_t* present = reinterpret_cast<uint32_t*>(boot + kMaxRowTiles);
  const int T = a.tiles_m;
  for (int rt = threadIdx.x; rt < T; rt += blockDim.x) key[rt] = row_tile_own(a, BM, rt) ? -1 : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < a.num_units; i += blockDim.x) {
    const int u = a.order ? a.order[i] : i;
    if (u < 0 || u >= a.num_units || u % a.batches != 0) continue;
    const int sp = u / a.batches;
    const int p = sp % a.panels, s = sp / a.panels;
    const int64_t r_lo = (int64_t)s * a.shard_m + (int64_t)p * a.unit_rows;
    const int64_t r_hi = min(r_lo + a.unit_rows, (int64_t)(s + 1) * a.shard_m);
    for (int rt = (int)(r_lo / BM); rt <= (int)((r_hi - 1) / BM); ++rt)
      if (key[rt] >= 0) atomicMax(&key[rt], i);
  }
  __syncthreads();
  for (int rt = threadIdx.x; rt < T; rt += blockDim.x) {
    const int k0 = key[rt];
    int rank = 0;
    for (int q = 0; q < T; ++q) {
      const int kq = key[q];
      rank += (kq < k0) || (kq == k0 && q < rt);
    }
    sorted[rank] = rt;
    pos[rt] = rank;
  }
  const int64_t round1 =
      min((int64_t)a.tiles_m * a.tiles_n, ((int64_t)a.consumers + a.splits - 1) / a.splits);  // tiles
  const int rows1 = (int)((round1 + a.tiles_n - 1) / a.tiles_n);
  const int SP = a.ranks * a.panels;
  const bool boot_on = with_boot && SP <= kMaxRowTiles;
  if (threadIdx.x == 0) s_nboot = 0;
  __syncthreads();  // key is no longer needed: it becomes bidx
  int* bidx = key;
  if (boot_on) {
    // Ordered compaction of the bootstrap panels: a ballot prefix per wave,
    // then the waves in order, so every workgroup builds the same list.
    const int wv = threadIdx.x / 64, ln = lane_id();
    const int cap = kBootBits / a.batches;  // panels whose presence bits fit
    for (int base = 0; base < SP; base += blockDim.x) {
      const int sp = base + threadIdx.x;
      const bool b = sp < SP && panel_is_boot(a, BM, pos, rows1, sp);
      const uint64_t m = __ballot(b);
      if (ln == 0) s_wave[wv] = __popcll(m);
      __syncthreads();
      int off = s_nboot;
      for (int q = 0; q < wv; ++q) off += s_wave[q];
      off += __popcll(m & ((1ull << ln) - 1));
      if (sp < SP) bidx[sp] = (b && off < cap) ? off : -1;
      if (b && off < cap) boot[off] = sp;
      __syncthreads();
      if (threadIdx.x == 0) {
        int t = 0;
        for (int q = 0; q < (int)(blockDim.x / 64); ++q) t += s_wave[q];
        s_nboot = min(s_nboot + t, cap);
      }
      __syncthreads();
    }
    const int words = (s_nboot * a.batches + 31) / 32;
    for (int i = threadIdx.x; i < words; i += blockDim.x) present[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < a.num_units; i += blockDim.x) {
      const int u = a.order ? a.order[i] : i;
      if (u < 0 || u >= a.num_units) continue;
      const int bi = bidx[u / a.batches];
      if (bi < 0) continue;
      const int bit = bi * a.batches + u % a.batches;
      atomicOr(&present[bit >> 5], 1u << (bit & 31));
    }
  } else {
    for (int sp = threadIdx.x; sp < min(SP, kMaxRowTiles); sp += blockDim.x) bidx[sp] = -1;
  }
  __syncthreads();
  Sched sc;
  sc.sorted = sorted;
  sc.pos = pos;
  sc.boot = boot;
  sc.bidx = bidx;
  sc.present = present;
  sc.n_boot = uniform(s_nboot);
  sc.rows1 = rows1;
  return sc;
}

// ---------------------------------------------------------------- consumer

// Tile rows [lo, hi) of a split tile: C = ((P_0 + P_1) + ...) over the
// partial products in range order, 16 bytes per lane, two row groups of
// every partial loaded before the first add.
template <int BM, int BN, int NT>
__device__ void reduce_splits(const AgArgs& a, int64_t m0, int64_t n0, int64_t lo, int64_t hi) {
  constexpr int VPR = BN / 4;           // 16-byte vectors per tile row
  constexpr int RPP = NT / VPR;         // rows per pass
  constexpr int U = 2;
  const int64_t rows = min(hi, a.m - m0);
  const int64_t cols = min((int64_t)BN, a.n - n0);
  const int vc = threadIdx.x % VPR, r0 = threadIdx.x / VPR;
  if (vc * 4 >= cols) return;  // n is a multiple of 8: a vector is all in or all out
  const int64_t slice = a.m * a.n;
  for (int64_t r = lo + r0; r < rows; r += RPP * U) {
    f32x4 v[U][kMaxSplits];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r + (int64_t)u * RPP;
      if (row >= rows) continue;
      const float* src = a.partial + (m0 + row) * a.n + n0 + vc * 4;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < a.splits) v[u][sp] = *reinterpret_cast<const f32x4*>(src + sp * slice);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r + (int64_t)u * RPP;
      if (row >= rows) continue;
      f32x4 sum = v[u][0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplits; ++sp)
        if (sp < a.splits) sum += v[u][sp];
      *reinterpret_cast<f32x4*>(a.c + (m0 + row) * a.n + n0 + vc * 4) = sum;
    }
  }
}

template <class T, int MODE>
__device__ void consume(const AgArgs& a, int cidx, const int* sorted, uint16_t* lds) {
  constexpr int BM = T::BM, BN = T::BN, NW = T::NW;

  bool timed_out = false;
  if (MODE == kModeBarrier) {
    // Every unit must have landed before any tile starts.
    for (int u = lane_id(); u < a.num_units; u += 64) {
      const int64_t* f = a.flags + (int64_t)u * a.flag_stride;
      uint64_t polls = 0;
      int64_t v;
      while ((v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < a.epoch) {
        if (++polls > a.spin_limit) {
          report_error(a.err, OVL_ETIMEOUT, kSiteAgBarrier, u, v, a.epoch);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      check_epoch(a.err, kSiteAgBarrier, u, v, a.epoch);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }

  // Work items (tile, K range) in consumer order are dealt out in rounds of
  // C; inside a round, consecutive items go to consumers on the same die
  // (workgroup ids are dispatched round-robin over the dies), so that items
  // sharing A rows or B columns share an L2.  When a round is whole rows of
  // unsplit tiles, each die takes a block of it instead (gr x gc dies over
  // the round's row tiles x column tiles, the split that needs the fewest A
  // and B panels per die): 4 row tiles x 7 column tiles at 224 consumers
  // and 14 column tiles, i.e. 11 operand panels per die and round where
  // 2 whole rows of tiles need 16.
  const int Cn = a.consumers;
  const int groups = (Cn % kXcds == 0) ? kXcds : 1;
  const int per = Cn / groups;
  const int x = cidx % groups, q = cidx / groups;
  const int64_t items = (int64_t)a.tiles_m * a.tiles_n * a.splits;
  const int own_lo = a.rank;  // shard index of the own rank
  __shared__ int s_last;

  int gr = 0, gc = 0;
  if (a.splits == 1 && groups == kXcds && Cn % a.tiles_n == 0) {
    const int rr = Cn / a.tiles_n;
    int best = 1 << 30;
    for (int c = 1; c <= kXcds; c *= 2) {
      const int r = kXcds / c;
      if (rr % r == 0 && a.tiles_n % c == 0 && rr / r + a.tiles_n / c < best) {
        best = rr / r + a.tiles_n / c;
        gr = r;
        gc = c;
      }
    }
  }
  for (int64_t w = 0;; ++w) {
    int64_t j = deal_item(w, x, q, groups, per, items);
    if (j < 0) break;
    if (gr && (w + 1) * Cn <= items) {
      const int rr = Cn / a.tiles_n, rpd = rr / gr, cpd = a.tiles_n / gc;
      j = (w * rr + (x / gc) * rpd + q / cpd) * a.tiles_n + (x % gc) * cpd + q % cpd;
    }
    const int64_t tl = j / a.splits;
    const int sp = (int)(j % a.splits);
    const int rt = uniform(sorted[tl / a.tiles_n]);
    const int nt = (int)(tl % a.tiles_n);
    const int64_t m0 = (int64_t)rt * BM, n0 = (int64_t)nt * BN;
    const int64_t k_lo = (int64_t)sp * a.split_cols;
    const int64_t k_hi = min(a.k, k_lo + a.split_cols);
    const int64_t m_end = min(m0 + BM, a.m);
    const bool own = row_tile_own(a, BM, rt);

    Operands op;  // A and B shifted to the item's K range
    op.b = a.b + k_lo * a.n;
    op.ldb = a.n;
    op.n0 = n0;
    op.n_valid = a.n;
    op.k = k_hi - k_lo;
    op.lda = a.k;
    int64_t m0_op;
    if (own) {
      op.a = a.shards[own_lo] + k_lo;
      op.m_valid = a.shard_m;
      m0_op = m0 - (int64_t)a.rank * a.shard_m;
    } else {
      op.a = a.g + k_lo;
      op.m_valid = a.m;
      m0_op = m0;
    }

    // Batches (ready, last] of this item's K range are the ones still to be
    // acquired.  Waiting is done by wave 0 one K-step ahead (see gemm_tile).
    // One round trip reads every flag of every remaining batch of the item,
    // lanes in parallel, so that a producer that runs ahead costs one poll
    // per item instead of one per batch; the item then knows all batches
    // up to the first missing unit are there.
    int ready = (int)(k_lo / a.batch_cols) - 1;
    const int last = (int)((k_hi - 1) / a.batch_cols);
    // covered: the columns of the item's K range (from k_lo) up to which this
    // wave checks no flag.  For wave 0 of a fused item that reads the gathered
    // operand, what the acquired batches cover (grown as batches are
    // acquired); for every other wave and item, all of them.  Wave-uniform,
    // so a step costs one scalar compare.  (A 64-bit division per step to
    // find its batch took a few hundred instructions of wave 0 per K-step.)
    const bool polls_flags = MODE == kModeFused && !own && uniform((int)threadIdx.x) < 64;
    int covered = polls_flags ? (int)((int64_t)(ready + 1) * a.batch_cols - k_lo) : INT32_MAX;
    // The (shard, row panel) pairs that cover the tile's rows are consecutive
    // in unit numbering (unit = (shard * panels + panel) * batches + batch):
    // panel ids sp_lo .. sp_lo + npan - 1.  Computed once per item, so that a
    // poll costs no 64-bit division.
    const int s_lo = (int)(m0 / a.shard_m), s_hi = (int)((m_end - 1) / a.shard_m);
    const int sp_lo = s_lo * a.panels + (int)((m0 - (int64_t)s_lo * a.shard_m) / a.unit_rows);
    const int npan =
        s_hi * a.panels + (int)((m_end - 1 - (int64_t)s_hi * a.shard_m) / a.unit_rows) - sp_lo + 1;
    const int64_t t_item = a.trace ? now_ticks() : 0;
    const int64_t c_item = a.trace ? now_cycles() : 0;
    int64_t waited = 0;  // ticks wave 0 spent polling for this item (traced runs)
    auto before_step = [&](int64_t, int64_t k1) {
      if (MODE != kModeFused || (int)k1 <= covered) return;  // wave 0 waits for the workgroup (see gemm_tile)
      const int need = (int)((k_lo + k1 - 1) / a.batch_cols);  // > ready
      const int64_t t_wait = a.trace ? now_ticks() : 0;
      const int lane = lane_id();
      for (uint64_t polls = 0;; ++polls) {
        // One round trip reads the units of every remaining batch (numbered
        // batch-major: i -> batch ready + 1 + i / npan, panel i % npan),
        // lanes in parallel; miss = the first i whose unit is not there yet,
        // seen holding the flag value it read.
        int miss = INT32_MAX;
        int64_t seen = 0;
        const int cnt = npan * (last - ready);
        for (int i = lane; i < cnt; i += 64) {
          const int bt = ready + 1 + i / npan;
          const int64_t u = (int64_t)(sp_lo + i % npan) * a.batches + bt;
          const int64_t v = __hip_atomic_load(a.flags + u * a.flag_stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v < a.epoch && i < miss) {
            miss = i;
            seen = v;
          }
          check_epoch(a.err, kSiteAgUnit, u, v, a.epoch);
        }
        int first = miss;
        for (int d = 1; d < 64; d <<= 1) first = min(first, __shfl_xor(first, d, 64));
        first = uniform(first);
        const int bad = first == INT32_MAX ? last + 1 : ready + 1 + first / npan;  // first batch not complete
        if (bad > need) {
          ready = bad - 1;
          break;
        }
        if (polls >= a.spin_limit) {
          // Name the first missing unit in the error record: the lane that
          // read it reports, with no further load (polls or error reports in
          // a loop here made the compiler wait for every load in flight at
          // the top of each K-step).
          if (miss == first)
            report_error(a.err, OVL_ETIMEOUT, kSiteAgUnit,
                         (int64_t)(sp_lo + first % npan) * a.batches + ready + 1 + first / npan, seen, a.epoch);
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      wave_acquire();  // one acquire for all the units seen
      covered = uniform(timed_out ? INT32_MAX : (int)((int64_t)(ready + 1) * a.batch_cols - k_lo));
      if (a.trace) waited += now_ticks() - t_wait;
    };
    // Thread 0 (in wave 0, which holds `waited`) records the item.
    auto trace_item = [&]() {
      if (!a.trace || threadIdx.x != 0) return;
      int64_t* rec = a.trace + a.num_units + kTraceItem * j;
      rec[0] = t_item;
      rec[1] = now_ticks();
      rec[2] = waited;
      rec[3] = cidx;
      rec[4] = c_item;
      rec[5] = now_cycles();
    };

    Acc<BM, BN, NW> acc;
    gemm_tile<BM, BN, T::BK, T::NS, false, NW, T::NL>(acc, op, m0_op, lds, before_step);
    if (!T::SPLIT || a.splits == 1) {
      acc_store<BM, BN, 0, NW>(acc, a.c, a.n, m0, n0, a.m, a.n);
      trace_item();
      continue;
    }
    // The range's partial goes out with agent-scope stores (complete at the
    // device's point of coherence once drained), so its arrival is a drain,
    // a barrier and a relaxed add: no release fence, whose L2 writeback of
    // the die (about 0.5 us, serialised per die) cost two per item here
    // (skinny 128x7168x8192 GEMM only: 50 us with the fences, 30 us with no
    // epilogue at all).
    acc_store<BM, BN, kAuxAgent, NW>(acc, a.partial + (int64_t)sp * a.m * a.n, a.n, m0, n0, a.m, a.n);
    int64_t* cnt = a.counters + 2 * tl;
    // The count before the add (thread 0's, in every lane of wave 0) is used
    // on both paths below: an atomic whose returned value stays pending into
    // the next item makes the compiler wait for every load in flight at the
    // top of each K-step.
    const int64_t before = uniform64(wg_arrive_agent(cnt));
    if (a.split_sync) {
      // Wait for the tile's other ranges (the last to arrive has seen them
      // all), then sum stripe sp of its rows.
      if (threadIdx.x < 64 && !timed_out) {
        if (before + 1 < a.splits && !wave_poll(cnt, a.splits, a.spin_limit, a.err, kSiteAgSplit, tl))
          timed_out = true;
        wave_acquire();
      }
      __syncthreads();
      const int64_t rs = (BM + a.splits - 1) / a.splits;
      reduce_splits<BM, BN, 64 * NW>(a, m0, n0, sp * rs, min((int64_t)BM, (sp + 1) * rs));
      // The last range out returns both counters to zero for the next launch
      // (bookkeeping only: this arrival publishes no data, so it needs no
      // release; every range has passed its wait on cnt before it arrives).
      __syncthreads();
      int64_t out = 0;
      if (threadIdx.x == 0)
        out = __hip_atomic_fetch_add(cnt + 1, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (threadIdx.x == 0 && out == a.splits - 1) {
        __hip_atomic_store(cnt, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(cnt + 1, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      trace_item();
      continue;
    }
    if (threadIdx.x == 0) {
      const bool last = before == a.splits - 1;
      if (last) {
        wave_acquire();  // the other ranges' partials
        __hip_atomic_store(cnt, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_last = last;
    }
    __syncthreads();
    if (uniform(s_last)) reduce_splits<BM, BN, 64 * NW>(a, m0, n0, 0, BM);
    trace_item();
  }
}

// Fused launch.  Every workgroup derives the schedule from the producer
// order.  In FUSED and BARRIER modes all workgroups first move, together, the
// units the first round of consumer tiles reads (the bootstrap: the whole
// chip copies what is needed first); then producers move the remaining units
// in the caller's order while consumers compute.
template <class T, int MODE>
__global__ __launch_bounds__(64 * T::NW, 1) void ag_gemm_kernel(AgArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  constexpr int NW = T::NW;
  using C = TileCfg<T::BM, T::BN, T::BK, T::NS, NW>;
  static_assert(kBootTabBytes <= C::LDS_BYTES, "bootstrap tables alias the stage area");
  int* sorted = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(lds) + C::LDS_BYTES);
  const Sched sc = build_schedule(a, T::BM, sorted, reinterpret_cast<int*>(lds), MODE != kModeGemmOnly);
  if (MODE != kModeGemmOnly) produce_boot<64 * NW>(a, blockIdx.x, gridDim.x, sc);
  if ((int)blockIdx.x < a.producers) {
    produce<64 * NW>(a, blockIdx.x, a.producers, &sc);
    return;
  }
  __syncthreads();  // every read of the bootstrap tables is done: the stages may be written
  consume<T, MODE>(a, (int)blockIdx.x - a.producers, sc.sorted, lds);
}

template <class T>
constexpr int ag_lds_bytes() {
  return TileCfg<T::BM, T::BN, T::BK, T::NS, T::NW>::LDS_BYTES + kOrderBytes;
}

}  // namespace ovl

using namespace ovl;

struct ag_gemm_plan_s {
  ag_gemm_desc d;
  int64_t m;
  int32_t unit_rows, panels, batches, batch_cols;
  int64_t num_units;
  int bm, bn;
  int tiles_m, tiles_n;
  int splits, split_cols;  // K split (1: none)
  int unit_producers;      // W >= 1
};

namespace {

template <class T, int MODE>
ovl_status launch_fused(const AgArgs& a, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&ag_gemm_kernel<T, MODE>);
  const int lds = ag_lds_bytes<T>();
  ovl_status st = allow_lds(fn, lds);
  if (st) return st;
  hipLaunchKernelGGL((ag_gemm_kernel<T, MODE>), dim3(a.producers + a.consumers), dim3(64 * T::NW), lds, stream, a);
  OVL_HIP_TRY(hipGetLastError());
  return OVL_OK;
}

template <class T>
ovl_status occupancy(int* out) {
  const int lds = ag_lds_bytes<T>();
  ovl_status st = allow_lds(reinterpret_cast<const void*>(&ag_gemm_kernel<T, kModeFused>), lds);
  if (st) return st;
  OVL_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(out, ag_gemm_kernel<T, kModeFused>, 64 * T::NW, lds));
  return OVL_OK;
}

template <class T>
ovl_status dispatch_mode(const AgArgs& a, uint32_t mode, hipStream_t stream) {
  switch (mode) {
    case OVL_MODE_FUSED: return launch_fused<T, kModeFused>(a, stream);
    case OVL_MODE_BARRIER: return launch_fused<T, kModeBarrier>(a, stream);
    case OVL_MODE_GEMM_ONLY: return launch_fused<T, kModeGemmOnly>(a, stream);
    default: return OVL_EINVAL;
  }
}

// The three tile configurations (TileBig, TileSmall, TileSplit above).
enum TileKind { kBig = 0, kSmall = 1, kSplit = 2 };

inline TileKind tile_kind(const ag_gemm_plan_s* p) {
  return p->bm == 256 ? kBig : (p->splits > 1 ? kSplit : kSmall);
}

// Compute units the plan assumes (MI355X); a device with fewer runs the
// same work items in more rounds.
constexpr int kPlanCus = 256;

}  // namespace

extern "C" ovl_status ag_gemm_plan(const ag_gemm_desc* d, ag_gemm_plan_t* out) {
  if (!d || !out) return OVL_EINVAL;
  *out = nullptr;
  if (d->ranks < 1 || d->rank < 0 || d->rank >= d->ranks) return OVL_EINVAL;
  if (d->ranks > kMaxRanks) return OVL_EUNSUPPORTED;
  if (d->shard_m < 1 || d->k < 8 || d->n < 8 || d->tile_m < 1 || d->tile_n < 8 || d->tiles_per_flag < 0)
    return OVL_ESHAPE;
  if (d->unit_producers < 0 || d->unit_producers > kMaxUnitProducers) return OVL_EINVAL;
  if (d->k % 8 || d->n % 8 || d->tile_n % 8) return OVL_EALIGN;
  if (d->flag_stride < 8 || d->flag_stride % 8) return OVL_EALIGN;
  const int64_t m = (int64_t)d->ranks * d->shard_m;
  // Every operand below 1 GiB and rows below 2^20 elements: buffer offsets stay in 32 bits.
  if (m > (1 << 20) || d->k > (1 << 20) || d->n > (1 << 20) || m * d->k * 2 > (1ll << 30) ||
      d->k * d->n * 2 > (1ll << 30) || m * d->n * 4 > (1ll << 30))
    return OVL_EUNSUPPORTED;

  ag_gemm_plan_s* p = new (std::nothrow) ag_gemm_plan_s();
  if (!p) return OVL_EINVAL;
  p->d = *d;
  p->m = m;
  p->unit_rows = (int32_t)std::min<int64_t>(d->tile_m, d->shard_m);
  p->panels = (int32_t)ceil_div(d->shard_m, p->unit_rows);
  const int64_t width = d->tiles_per_flag ? (int64_t)d->tiles_per_flag * d->tile_n : d->k;
  p->batch_cols = (int32_t)std::min<int64_t>(width, d->k);
  p->batches = (int32_t)ceil_div(d->k, p->batch_cols);
  p->num_units = (int64_t)d->ranks * p->panels * p->batches;
  p->unit_producers = std::max(1, d->unit_producers);
  if (p->num_units > (1 << 24)) {
    delete p;
    return OVL_EUNSUPPORTED;
  }
  // Large problems use 256x256 tiles; small ones 128x128 so that more
  // workgroups get work (half of MI355X's 256 compute units at least).
  const int64_t big_tiles = ceil_div(m, 256) * ceil_div(d->n, 256);
  if (m >= 256 && d->n >= 256 && big_tiles >= 128) {
    p->bm = 256;
    p->bn = 256;
  } else {
    p->bm = 128;
    p->bn = 128;
  }
  p->tiles_m = (int)ceil_div(m, p->bm);
  p->tiles_n = (int)ceil_div(d->n, p->bn);
  if (p->tiles_m > kMaxRowTiles) {
    delete p;
    return OVL_EUNSUPPORTED;
  }
  // Split K when the 128x128 tiles fill less than half of the consumers and
  // K is long: each range at least 4 K-steps of 64, at most kMaxSplits.
  p->splits = 1;
  p->split_cols = (int32_t)d->k;
  const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
  const int64_t consumers = kPlanCus - std::max(kXcds, kPlanCus / 8);
  if (p->bm == 128) {
    int64_t s = std::min<int64_t>({consumers / tiles, ceil_div(d->k, 256), kMaxSplits});
    if (s >= 2) {
      // The split tile may be wider: recount its tiles and ranges.
      p->bn = kSplitBN;
      p->tiles_n = (int)ceil_div(d->n, p->bn);
      const int64_t split_tiles = (int64_t)p->tiles_m * p->tiles_n;
      s = std::min<int64_t>({consumers / split_tiles, ceil_div(d->k, 256), kMaxSplits});
      if (s < 2) s = 2;
      p->split_cols = (int32_t)(ceil_div(ceil_div(d->k, s), 64) * 64);
      p->splits = (int)ceil_div(d->k, p->split_cols);
    }
  }
  *out = p;
  return OVL_OK;
}

extern "C" ovl_status ag_gemm_consumer_order(ag_gemm_plan_t p, const int32_t* order, int32_t* out) {
  if (!p || !out) return OVL_EINVAL;
  const ag_gemm_desc& d = p->d;
  const int T = p->tiles_m;
  const int64_t lo_own = (int64_t)d.rank * d.shard_m, hi_own = lo_own + d.shard_m;
  std::vector<int64_t> key(T);
  for (int rt = 0; rt < T; ++rt) {
    const int64_t lo = (int64_t)rt * p->bm, hi = std::min<int64_t>(lo + p->bm, p->m);
    key[rt] = (lo >= lo_own && hi <= hi_own) ? -1 : 0;
  }
  for (int64_t i = 0; i < p->num_units; ++i) {
    const int64_t u = order ? order[i] : i;
    if (u < 0 || u >= p->num_units) return OVL_EINVAL;
    if (u % p->batches) continue;
    const int64_t sp = u / p->batches;
    const int64_t pn = sp % p->panels, s = sp / p->panels;
    const int64_t r_lo = s * d.shard_m + pn * p->unit_rows;
    const int64_t r_hi = std::min<int64_t>(r_lo + p->unit_rows, (s + 1) * d.shard_m);
    for (int64_t rt = r_lo / p->bm; rt <= (r_hi - 1) / p->bm; ++rt)
      if (key[rt] >= 0) key[rt] = std::max<int64_t>(key[rt], i);
  }
  std::vector<int32_t> idx(T);
  for (int rt = 0; rt < T; ++rt) idx[rt] = rt;
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return key[x] < key[y]; });
  for (int rt = 0; rt < T; ++rt) out[rt] = idx[rt];
  return OVL_OK;
}

extern "C" int32_t ag_gemm_row_tiles(ag_gemm_plan_t p) { return p ? p->tiles_m : 0; }
extern "C" int32_t ag_gemm_tile_rows(ag_gemm_plan_t p) { return p ? p->bm : 0; }

extern "C" ovl_status ag_gemm_plan_destroy(ag_gemm_plan_t p) {
  delete p;
  return OVL_OK;
}

extern "C" int64_t ag_gemm_num_units(ag_gemm_plan_t p) { return p ? p->num_units : 0; }

extern "C" size_t ag_gemm_flags_bytes(ag_gemm_plan_t p) {
  return p ? (size_t)p->num_units * (size_t)p->d.flag_stride : 0;
}

// Error record (256 bytes reserved); with a K split, two arrival counters
// per tile (padded to 256 bytes); with several producers per unit, one
// arrival counter per unit (padded to 256 bytes); then, with a K split, the
// fp32 partial products [splits][m][n].
static size_t ag_counters_offset() { return 256; }
static size_t ag_arrivals_offset(const ag_gemm_plan_s* p) {
  return ag_counters_offset() +
         (p->splits > 1 ? (size_t)ceil_div((int64_t)p->tiles_m * p->tiles_n * 16, 256) * 256 : 0);
}
static size_t ag_partial_offset(const ag_gemm_plan_s* p) {
  return ag_arrivals_offset(p) + (p->unit_producers > 1 ? (size_t)ceil_div(p->num_units * 8, 256) * 256 : 0);
}

extern "C" size_t ag_gemm_workspace_bytes(ag_gemm_plan_t p) {
  if (!p) return 0;
  return ag_partial_offset(p) + (p->splits > 1 ? (size_t)p->splits * p->m * p->d.n * 4 : 0);
}

extern "C" int32_t ag_gemm_splits(ag_gemm_plan_t p) { return p ? p->splits : 0; }

// Publish times of the units, then four records per work item.
extern "C" size_t ag_gemm_trace_bytes(ag_gemm_plan_t p) {
  if (!p) return 0;
  return 8 * ((size_t)p->num_units + kTraceItem * (size_t)p->tiles_m * (size_t)p->tiles_n * (size_t)p->splits);
}

namespace {

// Bytes at the start of a plan's workspace that the allocation-free call
// clears before each run: the error record, the split counters and the unit
// arrival counters (the partial products need no clearing).  Arrival
// counters that start at zero count as if the workspace had just been reset.
size_t ag_state_bytes(const ag_gemm_plan_s* p) { return ag_partial_offset(p); }

// ag_gemm_run, and its allocation-free variant: clear_state zeroes the
// workspace's run state with a fill kernel on `stream` once every argument
// has been accepted, right before the launch.
ovl_status ag_gemm_launch(ag_gemm_plan_t p, const void* const* shards, const void* b, void* gathered, float* c,
                          int64_t* flags, void* workspace, bool clear_state, int64_t epoch,
                          const int32_t* producer_order, const ovl_opts* opts, hipStream_t stream) {
  if (!p || !shards || !workspace) return OVL_EINVAL;
  const uint32_t mode = opts ? opts->mode : OVL_MODE_FUSED;
  if (mode > OVL_MODE_BARRIER) return OVL_EINVAL;
  const bool needs_copy = mode != OVL_MODE_GEMM_ONLY;
  const bool needs_gemm = mode != OVL_MODE_COPY_ONLY;
  const ag_gemm_desc& d = p->d;
  if (!gathered) return OVL_EINVAL;
  if (!aligned16(gathered) || !aligned16(workspace)) return OVL_EALIGN;
  for (int s = 0; s < d.ranks; ++s) {
    if (!needs_copy && s != d.rank) continue;
    if (!shards[s]) return OVL_EINVAL;
    if (!aligned16(shards[s])) return OVL_EALIGN;
  }
  if (needs_gemm) {
    if (!b || !c) return OVL_EINVAL;
    if (!aligned16(b) || !aligned16(c)) return OVL_EALIGN;
  }
  if (needs_copy || mode == OVL_MODE_BARRIER) {
    if (!flags) return OVL_EINVAL;
    if (reinterpret_cast<uintptr_t>(flags) & 7u) return OVL_EALIGN;
  }
  if (producer_order && (reinterpret_cast<uintptr_t>(producer_order) & 3u)) return OVL_EALIGN;
  if (opts && opts->trace && (reinterpret_cast<uintptr_t>(opts->trace) & 7u)) return OVL_EALIGN;

  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;

  AgArgs a = {};
  for (int s = 0; s < d.ranks; ++s) a.shards[s] = static_cast<const uint16_t*>(shards[s]);
  a.b = static_cast<const uint16_t*>(b);
  a.g = static_cast<uint16_t*>(gathered);
  a.c = c;
  a.flags = flags;
  a.err = static_cast<ErrRec*>(workspace);
  a.order = producer_order;
  a.trace = opts ? opts->trace : nullptr;
  a.jitter = opts ? opts->jitter : 0;
  a.shard_m = d.shard_m;
  a.m = p->m;
  a.k = d.k;
  a.n = d.n;
  a.flag_stride = d.flag_stride / 8;
  a.epoch = epoch;
  a.spin_limit = spin_limit_of(opts);
  a.ranks = d.ranks;
  a.rank = d.rank;
  a.unit_rows = p->unit_rows;
  a.panels = p->panels;
  a.batches = p->batches;
  a.batch_cols = p->batch_cols;
  a.num_units = (int32_t)p->num_units;
  a.tiles_m = p->tiles_m;
  a.tiles_n = p->tiles_n;
  a.splits = p->splits;
  a.split_cols = p->split_cols;
  a.counters = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + ag_counters_offset());
  a.unit_producers = p->unit_producers;
  a.arrivals = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + ag_arrivals_offset(p));
  a.partial = p->splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ag_partial_offset(p))
                            : nullptr;

  const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
  const uint32_t req_prod = opts ? opts->producers : 0;

  if (mode == OVL_MODE_COPY_ONLY) {
    ovl_status st = epoch_accept(flags, epoch);
    if (st) return st;
    int P = req_prod ? (int)req_prod : di.cus * 4;
    P = (int)std::max<int64_t>(1, std::min<int64_t>(P, (int64_t)a.num_units * a.unit_producers));
    a.producers = P;
    a.consumers = 0;
    if (clear_state && (st = zero_async(workspace, ag_state_bytes(p), stream))) return st;
    hipLaunchKernelGGL(ag_produce_kernel, dim3(P), dim3(kThreads), 0, stream, a);
    OVL_HIP_TRY(hipGetLastError());
    return OVL_OK;
  }

  int occ = 0;
  const TileKind kind = tile_kind(p);
  st = kind == kBig ? occupancy<TileBig>(&occ)
                    : (kind == kSmall ? occupancy<TileSmall>(&occ) : occupancy<TileSplit>(&occ));
  if (st) return st;
  const int64_t resident = (int64_t)std::max(occ, 1) * di.cus;
  int P = 0;
  if (needs_copy) {
    P = req_prod ? (int)req_prod : std::max(kXcds, di.cus / 8);
    P = (int)std::min<int64_t>(P, (int64_t)a.num_units * a.unit_producers);
    if (P >= resident) return OVL_EINVAL;
  }
  // Consumers: the fewest that finish the items in as few rounds as the
  // resident ones allow, in whole die groups (448 tiles of 256 x 256 on 256
  // resident workgroups: 224 consumers in two whole rounds ran the GEMM alone
  // in 204 us, 256 consumers with a partial second round in 208-223 us).
  const int64_t items = tiles * p->splits, room = resident - P;
  int64_t Cn = std::min<int64_t>(items, room);
  Cn = (items + (items + Cn - 1) / Cn - 1) / ((items + Cn - 1) / Cn);
  const int64_t whole = (Cn + kXcds - 1) / kXcds * kXcds;
  if (Cn > kXcds && whole <= room) Cn = whole;
  a.producers = P;
  a.consumers = (int32_t)Cn;
  a.split_sync = p->splits > 1 && tiles * p->splits <= Cn;  // every range in the first round
  if (needs_copy) {
    st = epoch_accept(flags, epoch);
    if (st) return st;
  }
  if (clear_state && (st = zero_async(workspace, ag_state_bytes(p), stream))) return st;
  return kind == kBig ? dispatch_mode<TileBig>(a, mode, stream)
                      : (kind == kSmall ? dispatch_mode<TileSmall>(a, mode, stream)
                                        : dispatch_mode<TileSplit>(a, mode, stream));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

namespace ovl {

// The array's name is a host-side stand-in in host code; its device address
// on the current device comes from the runtime, once per device, with that
// device current.
ovl_status noalloc_scratch(void** out) {
  int dev = 0;
  OVL_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return OVL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return OVL_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return OVL_OK;
}

}  // namespace ovl

extern "C" ovl_status ag_gemm_run(ag_gemm_plan_t p, const void* const* shards, const void* b, void* gathered,
                                  float* c, int64_t* flags, void* workspace, int64_t epoch,
                                  const int32_t* producer_order, const ovl_opts* opts, hipStream_t stream) {
  return ag_gemm_launch(p, shards, b, gathered, c, flags, workspace, false, epoch, producer_order, opts, stream);
}

extern "C" ovl_status ag_gemm_run_noalloc(ag_gemm_plan_t p, const void* const* shards, const void* b,
                                          void* gathered, float* c, int64_t* flags, int64_t epoch,
                                          const int32_t* producer_order, const ovl_opts* opts, hipStream_t stream) {
  if (!p) return OVL_EINVAL;
  if (ag_gemm_workspace_bytes(p) > kScratchBytes) return OVL_EUNSUPPORTED;
  void* ws = nullptr;
  const ovl_status st = noalloc_scratch(&ws);
  if (st) return st;
  return ag_gemm_launch(p, shards, b, gathered, c, flags, ws, true, epoch, producer_order, opts, stream);
}
