// All-to-all dispatch of routed tokens, then a grouped expert GEMM, with
// slice-level overlap (the Aboleth README's all-to-all with one program per
// peer: put the slice at an offset indexed by the sender's rank, then set
// the receiver's flag for that sender; "Triton-distributed Semantics",
// Producer-Consumer Model).
//
// Two launches on the caller's stream:
//  1. Layout, one workgroup per (source s, local expert e): the number of
//     (token, choice) pairs of s routed to e and, for each pair, its row in
//     slice s, ordered by (e, token id).  Integer block scans only, so the
//     layout is bit-exact and does not depend on timing.  It also zeroes the
//     slice arrival counters of this run.
//  2. Fused: 32-row chunks of every slice (the own slice first, then
//     rank+1, rank+2, ...) are handed out from a ticket counter; a workgroup
//     that takes one copies the chunk's rows from the source's token rows,
//     then arrives on its slice's counter, and the workgroup that completes
//     a slice publishes the slice flag (signal ADD for the arrivals, signal
//     SET for the flag).  Producer workgroups take tickets until none is
//     left.  Consumer workgroups run 256x256 tiles of the grouped GEMM,
//     expert-major: an m-tile takes 256 consecutive rows of one expert's
//     rows (its segments in slice order, gathered through a per-tile row
//     table), so only each expert's last m-tile is partial; m-tiles go in
//     the order their last slice arrives.  Before a tile whose slices are
//     not all acquired, a consumer takes tickets while the flag it waits
//     for is not set (helping the copy instead of idling), then waits, and
//     runs the MFMA GEMM of the rows against that expert's weight.
#include <algorithm>

#include "device.h"
#include "gemm_core.h"
#include "gemm_fp8.h"
#include "host.h"

namespace ovl {

namespace {

constexpr int kA2aMaxRanks = 16;
constexpr int kA2aMaxExperts = 64;
constexpr int kChunkRows = 32;
constexpr int kGbm = 256, kGbn = 256;  // grouped GEMM tile
// The FP8 tile: 256 x 256 over eight waves, each wave's share (128 x 64) as
// in the four-wave 256 x 128 tile it replaced (a four-wave 256 x 256 tile
// spilled: its scaled epilogue moved all 256 accumulators out at once).
constexpr int kGbn8 = 256;
constexpr int kA2aMaxMTiles = 1024;    // m-tiles whose consumer order is sorted in LDS
constexpr int kA2aXcds = 8;
// Trace layout (int64): [R] slice publish times, [kA2aTraceProducers]
// producer finish times, then kA2aTraceItem values per work item.
constexpr int kA2aTraceProducers = 64;
constexpr int kA2aTraceItem = 8;
// Wavefronts per workgroup of the fused launch: both tiles run as a 2 x 4
// grid of waves, two per SIMD (one's MFMAs cover the other's LDS reads;
// measured faster than 4 for both).
constexpr int a2a_waves(bool) { return 8; }
// LDS of a grouped-GEMM tile, bf16 or FP8 (the geometry follows it).
constexpr int kA2aGemmLds = TileCfg<kGbm, kGbn>::LDS_BYTES > F8Cfg<kGbm, kGbn8>::LDS_BYTES
                                ? TileCfg<kGbm, kGbn>::LDS_BYTES
                                : F8Cfg<kGbm, kGbn8>::LDS_BYTES;

struct A2aArgs {
  const uint8_t* x[kA2aMaxRanks];        // token rows of row_bytes (bf16 or FP8 codes)
  const float* x_scale[kA2aMaxRanks];    // FP8: per-token scales (else null)
  const uint8_t* x_own;                  // x[rank] and x_scale[rank] (read in place by own-slice tiles)
  const float* x_scale_own;
  const int32_t* topk[kA2aMaxRanks];
  const uint8_t* w;        // bf16 [E][hidden][n], or FP8 codes [E][n][hidden]
  const float* w_scale;    // FP8: [E][n]
  uint8_t* recv_x;
  float* recv_scale;       // FP8: [R][cap]
  int32_t* recv_src;
  int32_t* recv_count;
  float* y;
  int64_t* flags;
  int64_t* counters;  // [R] slice arrival counters (workspace)
  int64_t* trace;     // optional timestamps (a2a_trace_bytes), or null
  int64_t* ticket;    // [0] next chunk to copy, [1] next shared tile, in the fused launch (workspace)
  ErrRec* err;
  int64_t tokens, hidden, n, cap;
  int64_t row_bytes;    // bytes of one token row: hidden * 2 (bf16) or hidden (FP8)
  int64_t flag_stride;  // int64 slots
  int64_t epoch;
  uint64_t spin_limit;
  int32_t ranks, rank, topk_n, experts;  // experts = experts per rank
  int32_t producers, consumers;
};

// ---------------------------------------------------------------- layout

__device__ inline int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Sum of v over the wavefront (every lane gets it).
__device__ inline int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// One workgroup per (source s, local expert e).  Wave w takes a contiguous
// range of the source's (token, choice) entries and reads it 64 entries at a
// time, lane l the l-th (coalesced; eight loads in flight).  Pass 1 counts
// the entries routed to local experts below e (which place expert e's
// segment in the slice) and to e; the wave totals give each wave's share of
// the segment; pass 2 reads the range again and writes expert e's rows in
// entry order, each matching lane at its wave's running count plus the
// matches of the lanes below it (a ballot).  Rows of a slice are thus
// ordered by (expert, token, choice), as the layout defines.
// Sixteen waves per (source, expert) workgroup: at the MoE workload (4096
// tokens x top-2) each wave then reads its 512 entries in one round of loads
// per pass.
constexpr int kLayoutThreads = 1024;

__global__ __launch_bounds__(kLayoutThreads) void a2a_layout_kernel(A2aArgs a) {
  constexpr int NWV = kLayoutThreads / 64;
  constexpr int B = 8;  // 64-entry groups loaded before they are looked at
  __shared__ int smem[2 * NWV];
  const int s = blockIdx.x / a.experts, e = blockIdx.x % a.experts;
  const int32_t* idx = a.topk[s];
  const int e_lo = a.rank * a.experts;
  const int lane = lane_id(), wave = uniform(threadIdx.x >> 6);
  const int64_t NE = a.tokens * a.topk_n;
  const int64_t per_w = ((NE + NWV - 1) / NWV + 63) / 64 * 64;
  const int64_t w0 = min(NE, wave * per_w), w1 = min(NE, w0 + per_w);
  int lt = 0, eq = 0;
  for (int64_t i = w0; i < w1; i += 64 * B) {
    int32_t v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int64_t k = i + 64 * q + lane;
      v[q] = k < w1 ? idx[k] : -1;
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int ex = v[q] - e_lo;
      lt += (ex >= 0) & (ex < e);
      eq += ex == e;
    }
  }
  lt = wave_sum(lt);
  eq = wave_sum(eq);
  if (lane == 0) {
    smem[wave] = eq;
    smem[NWV + wave] = lt;
  }
  __syncthreads();
  int base_total = 0, cnt_total = 0, before = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    base_total += smem[NWV + w];
    cnt_total += smem[w];
    if (w < wave) before += smem[w];
  }
  // A slice holds at most cap rows.  Only routing rows that repeat a local
  // expert (which the call's contract excludes) can ask for more; then the
  // rows past cap are dropped, the counts are clipped so that every later
  // step stays inside the slice, and the run reports OVL_ESHAPE.
  const int64_t end = min((int64_t)base_total + cnt_total, a.cap);
  const int cnt = (int)max((int64_t)0, end - base_total);
  if (eq) {
    int32_t* dst = a.recv_src + (int64_t)s * a.cap;
    int64_t run = (int64_t)base_total + before;  // next row of this wave
    for (int64_t i = w0; i < w1; i += 64 * B) {
      int32_t v[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int64_t k = i + 64 * q + lane;
        v[q] = k < w1 ? idx[k] : -1;
      }
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const bool hit = v[q] - e_lo == e;
        const uint64_t m = __ballot(hit);
        const int64_t pos = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (hit && pos < end) dst[pos] = (int32_t)((i + 64 * q + lane) / a.topk_n);
        run += __popcll(m);
      }
    }
  }
  if (threadIdx.x == 0) {
    if (cnt < cnt_total) report_error(a.err, OVL_ESHAPE, kSiteA2aCap, s, (int64_t)base_total + cnt_total, a.cap);
    a.recv_count[s * a.experts + e] = cnt;
    if (e == 0) a.counters[s] = 0;
    if (blockIdx.x == 0) {
      a.ticket[0] = 0;
      a.ticket[1] = 0;
    }
  }
}

// ---------------------------------------------------------------- shared schedule

// Per-run geometry, rebuilt by every workgroup from recv_count.
//
// The grouped GEMM runs expert-major: expert e's rows are the rows of its
// segments in slice order (own slice first), and its m-tiles cut that list
// into kGbm-row pieces, so a tile may take rows from two slices and only the
// expert's last m-tile is partial.  M-tiles are taken in the order the data
// arrives: by the slice position of their last row, then by expert, then by
// m-tile (n-tiles of one m-tile are consecutive).
struct Geometry {
  int32_t count[kA2aMaxRanks * kA2aMaxExperts];  // recv_count, by (slice, expert)
  int32_t slice_rows[kA2aMaxRanks];   // by slice
  int32_t chunk_base[kA2aMaxRanks + 1];  // by position in slice order
  int32_t seg_start[kA2aMaxRanks * kA2aMaxExperts];  // by (position, expert): segment start in the slice
  int32_t exp_pre[kA2aMaxExperts * (kA2aMaxRanks + 1)];  // by (expert, position): expert rows before it
  int32_t mt_base[kA2aMaxExperts + 1];  // m-tiles of experts before e
  int32_t n_mt;                         // m-tiles in all
  int32_t mt_order[kA2aMaxMTiles];      // m-tiles in consumer order (e << 20 | mt), if n_mt fits
};

__device__ inline int slice_at(const A2aArgs& a, int pos) { return (a.rank + pos) % a.ranks; }

// Slice position of expert row r of expert e (rows of earlier positions come first).
__device__ inline int pos_of_row(const A2aArgs& a, const Geometry* g, int e, int r) {
  const int32_t* pre = g->exp_pre + e * (kA2aMaxRanks + 1);
  int pos = 0;
  while (pos + 1 < a.ranks && uniform(pre[pos + 1]) <= r) ++pos;
  return pos;
}

__device__ void build_geometry(const A2aArgs& a, Geometry* g) {
  __shared__ int32_t s_key[kA2aMaxMTiles];
  for (int i = threadIdx.x; i < a.ranks * a.experts; i += blockDim.x) g->count[i] = a.recv_count[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    int chunks = 0;
    for (int pos = 0; pos < a.ranks; ++pos) {
      const int s = slice_at(a, pos);
      int rows = 0;
      g->chunk_base[pos] = chunks;
      for (int e = 0; e < a.experts; ++e) {
        g->seg_start[pos * a.experts + e] = rows;
        rows += g->count[s * a.experts + e];
      }
      g->slice_rows[s] = rows;
      chunks += (rows + kChunkRows - 1) / kChunkRows;
    }
    g->chunk_base[a.ranks] = chunks;
    int mts = 0;
    for (int e = 0; e < a.experts; ++e) {
      int32_t* pre = g->exp_pre + e * (kA2aMaxRanks + 1);
      int r = 0;
      for (int pos = 0; pos < a.ranks; ++pos) {
        pre[pos] = r;
        r += g->count[slice_at(a, pos) * a.experts + e];
      }
      pre[a.ranks] = r;
      g->mt_base[e] = mts;
      mts += (r + kGbm - 1) / kGbm;
    }
    g->mt_base[a.experts] = mts;
    g->n_mt = mts;
  }
  __syncthreads();
  // Consumer order of the m-tiles: a rank sort on (last row's position,
  // expert, m-tile), identical in every workgroup.
  const int n_mt = uniform(g->n_mt);
  if (n_mt <= kA2aMaxMTiles) {
    for (int q = threadIdx.x; q < n_mt; q += blockDim.x) {
      int e = 0;
      while (g->mt_base[e + 1] <= q) ++e;
      const int mt = q - g->mt_base[e];
      const int32_t* pre = g->exp_pre + e * (kA2aMaxRanks + 1);
      const int last = min((mt + 1) * kGbm, pre[a.ranks]) - 1;
      int pos = 0;
      while (pos + 1 < a.ranks && pre[pos + 1] <= last) ++pos;
      s_key[q] = (pos * kA2aMaxExperts + e) * kA2aMaxMTiles + mt;  // distinct keys
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n_mt; q += blockDim.x) {
      const int32_t k = s_key[q];
      int rank = 0;
      for (int o = 0; o < n_mt; ++o) rank += s_key[o] < k;
      const int e = (k / kA2aMaxMTiles) % kA2aMaxExperts;
      g->mt_order[rank] = (e << 20) | (k % kA2aMaxMTiles);
    }
  }
  __syncthreads();
}

// Expert and m-tile of the q-th m-tile in consumer order (expert-major
// when there are more m-tiles than the order table holds).
__device__ inline void mtile_at(const A2aArgs& a, const Geometry* g, int q, int* e, int* mt) {
  if (uniform(g->n_mt) <= kA2aMaxMTiles) {
    const int v = uniform(g->mt_order[q]);
    *e = v >> 20;
    *mt = v & ((1 << 20) - 1);
    return;
  }
  int x = 0;
  while (uniform(g->mt_base[x + 1]) <= q) ++x;
  *e = x;
  *mt = q - uniform(g->mt_base[x]);
}

// ---------------------------------------------------------------- producer

// Copies rows [r0, r1) of slice s: row r of the slice is token recv_src[r]
// of source s.  A wave moves 8 KiB slots, two per step, each lane 16-byte
// vectors lane, lane + 64, ... of a slot: a slot is one row (in passes, for
// rows longer than 8 KiB), or several whole rows when rows are shorter (a
// power-of-two count of at least 1 KiB: FP8 tokens), so that every lane
// always has work.  Wave w of W takes slots w, w + W (a pair), then w + 2W, ....
// The loads of the next step are issued before the stores of the current
// one, so that a wave always has a slot pair in flight (vector memory
// counters complete in order: waiting for the loads then does not wait for
// the stores issued after them).
__device__ inline void copy_rows(const A2aArgs& a, int s, int r0, int r1) {
  constexpr int V = 8;  // vectors per lane per slot: 8 KiB
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int W = (int)(blockDim.x >> 6);
  const int vpr = (int)(a.row_bytes / 16);
  const uint8_t* src = a.x[s];
  uint8_t* dst = a.recv_x + (int64_t)s * a.cap * a.row_bytes;
  const float* xs = a.x_scale[s];
  const int32_t* srow = a.recv_src + (int64_t)s * a.cap;
  // rows per slot: 64 * V / vpr for rows of 1 KiB .. 4 KiB (a power of two)
  const bool multi = vpr >= 64 && vpr < 64 * V && (vpr & (vpr - 1)) == 0;
  const int lg_qpr = multi ? __builtin_ctz(vpr / 64) : 0;  // log2(vectors per lane per row)
  const int rps = multi ? (64 * V) / vpr : 1;
  const int units = (r1 - r0 + rps - 1) / rps;
  // Steps: (slot pair, column pass); a pair is slots u, u + W of this wave.
  const int passes = multi ? 1 : (vpr + 64 * V - 1) / (64 * V);
  const int pairs = units > wave ? (units - wave + 2 * W - 1) / (2 * W) : 0;
  const int steps = pairs * passes;
  u32x4 cur[2][V], nxt[2][V];
  // Buffer loads and stores with no branch around them: a vector that does
  // not exist gets an offset past its buffer (the load returns zeros, the
  // store is dropped).  Guarded per vector, the compiler lost count of the
  // loads in flight and waited for all of them before every store.
  const rsrc_t rsrc = make_rsrc(src, a.tokens * a.row_bytes);
  const rsrc_t rdst = make_rsrc(dst, a.cap * a.row_bytes);
  const uint32_t rb = (uint32_t)a.row_bytes;
  auto load = [&](int st, u32x4 (&v)[2][V]) {
    const int u = wave + (st / passes) * 2 * W, c0 = (st % passes) * 64 * V;
    // every vector's source token first (all lanes read the same entries),
    // then the data loads: one wait for the table, not one per row
    int32_t tok[2][V];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const int rr = r0 + (u + W * h) * rps + (multi ? q >> lg_qpr : 0);
        tok[h][q] = rr < r1 ? srow[rr] : -1;
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const int c = multi ? ((q & ((1 << lg_qpr) - 1)) << 6) + lane : c0 + q * 64 + lane;
        const uint32_t off = (tok[h][q] >= 0 && c < vpr) ? (uint32_t)tok[h][q] * rb + (uint32_t)c * 16 : kOOB;
        v[h][q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
      }
    }
  };
  auto store = [&](int st, const u32x4 (&v)[2][V]) {
    const int u = wave + (st / passes) * 2 * W, c0 = (st % passes) * 64 * V;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const int rr = r0 + (u + W * h) * rps + (multi ? q >> lg_qpr : 0);
        const int c = multi ? ((q & ((1 << lg_qpr) - 1)) << 6) + lane : c0 + q * 64 + lane;
        const uint32_t off = (rr < r1 && c < vpr) ? (uint32_t)rr * rb + (uint32_t)c * 16 : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(v[h][q], rdst, (int)off, 0, 0);
      }
    }
    // FP8: each row's scale travels with it, read with scalar loads after
    // the data stores: a vector load here would make every later store
    // wait for all the loads in flight (vector memory counters complete in
    // order).
    if (xs) {
      typedef const __attribute__((address_space(4))) int32_t* ctok_t;
      typedef const __attribute__((address_space(4))) float* cscale_t;
      const ctok_t ctok = (ctok_t)srow;
      const cscale_t cxs = (cscale_t)xs;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        for (int k = 0; k < rps; ++k) {
          const int rr = uniform(r0 + (u + W * h) * rps + k);
          if (rr < r1 && lane == 0) a.recv_scale[(int64_t)s * a.cap + rr] = cxs[ctok[rr]];
        }
    }
  };
  if (steps > 0) load(0, cur);
  for (int st = 0; st < steps; st += 2) {
    if (st + 1 < steps) load(st + 1, nxt);
    store(st, cur);
    if (st + 1 >= steps) break;
    if (st + 2 < steps) load(st + 2, cur);
    store(st + 1, nxt);
  }
}

// Position (in slice order) of the slice chunk ch belongs to.
__device__ inline int chunk_pos(const Geometry* g, int ch) {
  int pos = 0;
  while (uniform(g->chunk_base[pos + 1]) <= ch) ++pos;
  return pos;
}

// Copies the rows of chunk ch (kChunkRows rows of the slice at `pos`, in
// slice order).
__device__ inline void a2a_copy_chunk_rows(const A2aArgs& a, const Geometry* g, int ch, int pos) {
  const int s = slice_at(a, pos);
  const int r0 = (ch - uniform(g->chunk_base[pos])) * kChunkRows;
  copy_rows(a, s, r0, min(r0 + kChunkRows, uniform(g->slice_rows[s])));
}

// Arrives for n chunks of the slice at `pos` that this workgroup copied:
// one release (an L2 writeback of this die, the costly part) for all of
// them.  The workgroup that completes the slice acquires the other arrivals
// and publishes the slice flag.
__device__ inline void a2a_arrive(const A2aArgs& a, const Geometry* g, int pos, int n) {
  const int s = slice_at(a, pos);
  const int need = uniform(g->chunk_base[pos + 1]) - uniform(g->chunk_base[pos]);
  const int64_t old = wg_arrive(a.counters + s, n);
  if (threadIdx.x == 0 && old + n == need) {
    // Acquire the other arrivals, then release them on with the flag.
    wave_acquire();
    __hip_atomic_store(a.flags + (int64_t)s * a.flag_stride, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (a.trace) a.trace[s] = now_ticks();
  }
  // A barrier after the thread-0 branch: callers loop over chunks and take
  // the next ticket in another thread-0 branch; with nothing between the two
  // the compiler joins them into one path for thread 0 and lets the other
  // lanes of its wave run on to the next barrier without it.
  __syncthreads();
}

// Chunk ch, then its arrival at once (a consumer that helps copy goes back
// to its flag after each chunk).
__device__ inline void a2a_copy_chunk(const A2aArgs& a, const Geometry* g, int ch) {
  const int pos = chunk_pos(g, ch);
  a2a_copy_chunk_rows(a, g, ch, pos);
  a2a_arrive(a, g, pos, 1);
}

// Chunk ch for a producer that defers its arrivals: chunks of one slice
// copied back to back arrive together, when the producer moves on to
// another slice or runs out of chunks (*pend_n chunks of the slice at
// *pend_pos are pending).  A slice cannot complete before the producer's
// current chunk of it is copied, so the deferral delays no flag.
__device__ inline void a2a_copy_chunk_deferred(const A2aArgs& a, const Geometry* g, int ch, int* pend_pos,
                                               int* pend_n) {
  const int pos = chunk_pos(g, ch);
  if (*pend_n && pos != *pend_pos) {
    a2a_arrive(a, g, *pend_pos, *pend_n);
    *pend_n = 0;
  }
  a2a_copy_chunk_rows(a, g, ch, pos);
  *pend_pos = pos;
  ++*pend_n;
}

// Chunks [c0, c1), workgroup w of P taking a contiguous share (mostly of
// one slice, so that its arrivals go out together).
__device__ void a2a_produce(const A2aArgs& a, const Geometry* g, int w, int P, int c0, int c1) {
  // Slices that receive nothing are complete at once.
  if (w == 0 && c0 == 0 && threadIdx.x < a.ranks && g->slice_rows[threadIdx.x] == 0)
    __hip_atomic_store(a.flags + (int64_t)threadIdx.x * a.flag_stride, a.epoch, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
  const int per = (c1 - c0 + P - 1) / P;
  const int lo = min(c1, c0 + w * per), hi = min(c1, lo + per);
  int pend_pos = 0, pend_n = 0;
  for (int ch = lo; ch < hi; ++ch) a2a_copy_chunk_deferred(a, g, ch, &pend_pos, &pend_n);
  if (pend_n) a2a_arrive(a, g, pend_pos, pend_n);
}

// Fused launch: chunks are handed out in slice order from one ticket
// counter.  Thread 0 takes the next ticket; every thread returns it (or
// `total` once none is left).
__device__ inline int take_chunk(const A2aArgs& a, int total, int* sh) {
  if (threadIdx.x == 0) {
    const int64_t t = __hip_atomic_fetch_add(a.ticket, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sh = t < total ? (int)t : total;
  }
  __syncthreads();
  const int ch = uniform(*sh);
  __syncthreads();  // *sh is rewritten by the next call
  return ch;
}

// Copy-only producers run eight waves (FP8 rows: dispatch alone 88 -> 81.5
// us; bf16 rows: the same 133 us as with four).
constexpr int kProduceThreads = 512;

__global__ __launch_bounds__(kProduceThreads) void a2a_produce_kernel(A2aArgs a) {
  __shared__ Geometry g;
  build_geometry(a, &g);
  a2a_produce(a, &g, blockIdx.x, gridDim.x, 0, uniform(g.chunk_base[a.ranks]));
}

// ---------------------------------------------------------------- consumer

// Waits for slice s; while its flag is not set and chunks are left, the
// workgroup copies chunks itself, rechecking the flag after each (the first
// consumers thus copy the first slices together, and no consumer idles
// while copying work remains: measured better than helping only with the
// chunks up to s).  Ends with the acquire done by wave 0 and a workgroup
// barrier.  Returns false on timeout.
// The result is the same in every wave: wave 0's poll result goes through
// LDS, because callers loop over this call and every barrier in it.
__device__ bool wait_slice_helping(const A2aArgs& a, const Geometry* g, int s, int* sh, int* helped) {
  const int total = uniform(g->chunk_base[a.ranks]);
  const int64_t* flag = a.flags + (int64_t)s * a.flag_stride;
  int st;
  for (;;) {
    if (threadIdx.x == 0) {
      int v = 2;  // 0 ready, 1 help, 2 wait
      const int64_t f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f >= a.epoch) {
        v = 0;
        check_epoch(a.err, kSiteA2aSlice, s, f, a.epoch);
      } else if (__hip_atomic_load(a.ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < total) {
        v = 1;
      }
      sh[1] = v;
    }
    __syncthreads();
    st = uniform(sh[1]);
    __syncthreads();
    if (st != 1) break;
    const int ch = take_chunk(a, total, sh);
    if (ch < total) {
      a2a_copy_chunk(a, g, ch);
      ++*helped;
    }
  }
  if (threadIdx.x < 64) {
    const bool ok = st != 2 || wave_poll(flag, a.epoch, a.spin_limit, a.err, kSiteA2aSlice, s);
    wave_acquire();
    if (threadIdx.x == 0) sh[1] = ok;
  }
  __syncthreads();
  const int ok = uniform(sh[1]);
  __syncthreads();  // sh[1] is rewritten by the next call
  return ok != 0;
}

// The next tile of the shared tail (fused launch): every thread returns it.
// The barrier before the thread-0 branch keeps it apart from the previous
// tile's thread-0 trace record.
__device__ inline int take_tile(const A2aArgs& a, int* sh) {
  __syncthreads();
  if (threadIdx.x == 0)
    *sh = (int)__hip_atomic_fetch_add(a.ticket + 1, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = uniform(*sh);
  __syncthreads();  // *sh is rewritten by the next call
  return t;
}

// Tiles of one workgroup.  Consumer cidx (cidx >= 0) first takes its static
// share of `srounds` whole rounds (tiles w * Cn + x * per + q: dies take
// consecutive tiles); the tiles after those rounds form a tail that every
// workgroup takes from a ticket counter once it is free: consumers after
// their static share, producers (cidx < 0) once the copy is handed out, so
// no compute unit idles at the end.
template <bool WAIT, bool F8>
__device__ void a2a_consume(const A2aArgs& a, const Geometry* g, int cidx, uint16_t* lds, int64_t srounds) {
  __shared__ int sh[2];
  // Per tile (double-buffered): [0] the y row of each tile row (s * cap +
  // slice row; also the A row in recv_x), or -1; [1] for own-slice tiles,
  // the token row of x[rank] each tile row reads.
  __shared__ int32_t rowtab[2][2][kGbm];
  __shared__ float scaletab[F8 ? 2 : 1][F8 ? kGbm : 1];  // FP8: the scale of each tile row
  constexpr int TBN = F8 ? kGbn8 : kGbn;
  const int ntn = (int)((a.n + TBN - 1) / TBN);
  const int total = uniform(g->n_mt) * ntn;
  const int Cn = a.consumers;
  const int groups = (Cn % kA2aXcds == 0) ? kA2aXcds : 1;
  const int per = Cn / groups;
  const int x = cidx % groups, q = cidx / groups;
  int waited_hi = -1;  // slice positions [0, waited_hi] are acquired
  bool timed_out = false;
  const int64_t tail = srounds * Cn;  // first tile of the shared tail
  for (int64_t wv = 0;; ++wv) {
    const int64_t j = (cidx >= 0 && wv < srounds) ? wv * Cn + (int64_t)x * per + q : tail + take_tile(a, sh);
    if (j >= total) break;
    int e, mt;
    mtile_at(a, g, (int)(j / ntn), &e, &mt);
    const int nt = (int)(j % ntn);
    const int32_t* pre = g->exp_pre + e * (kA2aMaxRanks + 1);
    const int r0 = mt * kGbm, rows_e = uniform(pre[a.ranks]);
    const int nrows = min(kGbm, rows_e - r0);
    const int pos_hi = pos_of_row(a, g, e, r0 + nrows - 1);
    // A tile whose rows all lie in the own slice reads them from the own
    // tokens in place (recv_src, from the layout kernel, names each row's
    // token): the same bits as the slice's copy, with nothing to wait for,
    // so the first consumers compute while the others copy.  Its row table
    // holds token ids (< tokens) or -1 (no row: an out-of-range offset), so
    // the A resource keeps the ranks * cap row bound of the received rows
    // (>= tokens) and is never read past x[rank]'s rows; a bound selected
    // per tile made the compiler reserve scratch.
    const bool local = WAIT && pos_hi == 0;
    const int64_t t_item = a.trace ? now_ticks() : 0;
    int helped = 0;
    if (WAIT && !local) {
      while (waited_hi < pos_hi && !timed_out) {
        ++waited_hi;
        if (!wait_slice_helping(a, g, slice_at(a, waited_hi), sh, &helped)) timed_out = true;
      }
    }
    const int64_t t_ready = a.trace ? now_ticks() : 0;
    // Row table of the tile: expert row r0 + i lies in the slice at the
    // first position whose expert prefix exceeds it.
    int32_t* tab = rowtab[wv & 1][0];
    int32_t* tokrow = rowtab[wv & 1][1];
    for (int i = threadIdx.x; i < kGbm; i += blockDim.x) {
      int32_t v = -1;
      if (i < nrows) {
        const int r = r0 + i;
        int pos = 0;
        while (pos + 1 < a.ranks && pre[pos + 1] <= r) ++pos;
        const int s = slice_at(a, pos);
        v = s * (int32_t)a.cap + g->seg_start[pos * a.experts + e] + (r - pre[pos]);
      }
      tab[i] = v;
      const int32_t tk = (local && v >= 0) ? a.recv_src[v] : -1;
      if (local) tokrow[i] = tk;
      if constexpr (F8)
        scaletab[wv & 1][i] = local ? (tk >= 0 ? a.x_scale_own[tk] : 0.f) : (v >= 0 ? a.recv_scale[v] : 0.f);
    }
    __syncthreads();
    constexpr int NW = a2a_waves(F8);
    Acc<kGbm, TBN, NW> acc;
    if constexpr (F8) {
      Operands8 op;
      op.a = a.recv_x;
      op.lda = a.hidden;
      op.m_valid = (int64_t)a.ranks * a.cap;
      if (local) op.a = a.x_own;  // rows: token ids < tokens <= ranks * cap (see above)
      op.rows = rowtab[wv & 1][local ? 1 : 0];
      op.bt = a.w + (int64_t)e * a.n * a.hidden;
      op.ldb = a.hidden;
      op.n0 = (int64_t)nt * TBN;
      op.n_valid = a.n;
      op.k = a.hidden;
      if (a.n - op.n0 <= TBN / 2) {
        // A last column block at most half a tile wide: a half-width tile
        // (the same K order per element, so the same bits).
        Acc<kGbm, TBN / 2, NW> acc2;
        gemm_tile_fp8<kGbm, TBN / 2, true, NW>(acc2, op, reinterpret_cast<uint8_t*>(lds));
        acc_store_rows_scaled<kGbm, TBN / 2, NW>(acc2, a.y, a.n, (int64_t)a.ranks * a.cap, tab, scaletab[wv & 1],
                                                 a.w_scale + (int64_t)e * a.n, op.n0, a.n);
      } else {
        gemm_tile_fp8<kGbm, TBN, true, NW>(acc, op, reinterpret_cast<uint8_t*>(lds));
        acc_store_rows_scaled<kGbm, TBN, NW>(acc, a.y, a.n, (int64_t)a.ranks * a.cap, tab, scaletab[wv & 1],
                                             a.w_scale + (int64_t)e * a.n, op.n0, a.n);
      }
    } else {
      Operands op;
      op.a = reinterpret_cast<const uint16_t*>(a.recv_x);
      op.lda = a.hidden;
      op.m_valid = (int64_t)a.ranks * a.cap;
      if (local) op.a = reinterpret_cast<const uint16_t*>(a.x_own);  // rows: token ids (see above)
      op.rows = rowtab[wv & 1][local ? 1 : 0];
      op.b = reinterpret_cast<const uint16_t*>(a.w) + (int64_t)e * a.hidden * a.n;
      op.ldb = a.n;
      op.n0 = (int64_t)nt * TBN;
      op.n_valid = a.n;
      op.k = a.hidden;
      if (a.n - op.n0 <= TBN / 2) {
        // The last column block is at most half a tile wide (1408 = 5.5 x
        // 256): a half-width tile does half the MFMA work, with the same
        // K order per element (so the same bits).
        Acc<kGbm, TBN / 2, NW> acc2;
        gemm_tile<kGbm, TBN / 2, 64, 0, true, NW>(acc2, op, 0, lds, [](int64_t, int64_t) {});
        acc_store_rows<kGbm, TBN / 2, NW>(acc2, a.y, a.n, (int64_t)a.ranks * a.cap, tab, op.n0, a.n);
      } else {
        gemm_tile<kGbm, TBN, 64, 0, true, NW>(acc, op, 0, lds, [](int64_t, int64_t) {});
        acc_store_rows<kGbm, TBN, NW>(acc, a.y, a.n, (int64_t)a.ranks * a.cap, tab, op.n0, a.n);
      }
    }
    if (a.trace && threadIdx.x == 0) {
      int64_t* rec = a.trace + a.ranks + kA2aTraceProducers + kA2aTraceItem * j;
      rec[0] = t_item;
      rec[1] = now_ticks();
      rec[2] = t_ready - t_item;  // waiting for slices, copying chunks meanwhile
      rec[3] = helped;
      rec[4] = cidx;
      rec[5] = e;
      rec[6] = mt;
      rec[7] = nt;
    }
  }
}

// Whole rounds of the fused launch's tiles dealt statically to the
// consumers: one round fewer than all workgroups would fill, so that the
// tail (at least one round) is shared with the producers.
__device__ inline int64_t a2a_static_rounds(const A2aArgs& a, const Geometry* g, bool f8) {
  const int tbn = f8 ? kGbn8 : kGbn;
  const int64_t total = (int64_t)uniform(g->n_mt) * ((a.n + tbn - 1) / tbn);
  const int64_t r = total / (a.consumers + a.producers) - 1;
  return r > 0 ? r : 0;
}

// Fused launch.  Producer workgroups take chunk tickets until none is
// left; consumers take tickets too whenever the slice of their next tile is
// not complete yet, so the first consumers copy the first slices together
// and the copy keeps ahead of the GEMM.
template <int MODE, bool F8>  // MODE 0 fused, 2 GEMM only; F8: FP8 rows and grouped GEMM
__global__ __launch_bounds__(64 * a2a_waves(F8), 1) void a2a_fused_kernel(A2aArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int sh;
  Geometry* g = reinterpret_cast<Geometry*>(reinterpret_cast<uint8_t*>(lds) + kA2aGemmLds);
  build_geometry(a, g);
  if (MODE == 0) {
    // Slices that receive nothing are complete at once.
    if (blockIdx.x == 0 && threadIdx.x < a.ranks && g->slice_rows[threadIdx.x] == 0)
      __hip_atomic_store(a.flags + (int64_t)threadIdx.x * a.flag_stride, a.epoch, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    if ((int)blockIdx.x < a.producers) {
      const int total = uniform(g->chunk_base[a.ranks]);
      int pend_pos = 0, pend_n = 0;
      for (int ch; (ch = take_chunk(a, total, &sh)) < total;) a2a_copy_chunk_deferred(a, g, ch, &pend_pos, &pend_n);
      if (pend_n) a2a_arrive(a, g, pend_pos, pend_n);
      // No copy load may stay pending into the GEMM below: the compiler would
      // otherwise wait for them at the top of every K-step.
      wave_drain();
      if (a.trace && threadIdx.x == 0 && blockIdx.x < kA2aTraceProducers) a.trace[a.ranks + blockIdx.x] = now_ticks();
      // The copy is handed out: take tiles of the shared tail.
      a2a_consume<true, F8>(a, g, -1, lds, a2a_static_rounds(a, g, F8));
      return;
    }
  }
  a2a_consume<MODE == 0, F8>(a, g, (int)blockIdx.x - a.producers, lds,
                             MODE == 0 ? a2a_static_rounds(a, g, F8) : (int64_t)1 << 40);
}

constexpr int a2a_lds_bytes() { return kA2aGemmLds + (int)sizeof(Geometry); }

}  // namespace

}  // namespace ovl

using namespace ovl;

extern "C" size_t a2a_flags_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1 || d->flag_stride < 8) return 0;
  return (size_t)d->ranks * (size_t)d->flag_stride;
}

// Slice publish times, producer finish times, then a record per work item:
// at most (R * cap / 256 + experts) m-tiles times the n-tiles of the
// narrower (FP8) tile.
extern "C" size_t a2a_trace_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1 || d->experts_per_rank < 1 || d->n < 1 || d->tokens < 0) return 0;
  const int64_t cap = d->tokens * std::min<int64_t>(d->topk, d->experts_per_rank);
  const int64_t mts = ((int64_t)d->ranks * cap + kGbm - 1) / kGbm + d->experts_per_rank;
  const int64_t nts = (d->n + kGbn8 - 1) / kGbn8;
  return 8 * ((size_t)d->ranks + kA2aTraceProducers + (size_t)kA2aTraceItem * (size_t)(mts * nts));
}

// Error record, slice arrival counters, chunk and tile tickets.
extern "C" size_t a2a_workspace_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1) return 0;
  return OVL_ERROR_RECORD_BYTES + 8 * (size_t)kA2aMaxRanks + 16;
}

namespace ovl {
namespace {

// Both dispatch entry points: f8 selects FP8 rows (hidden bytes, a scale
// each) and the FP8 grouped GEMM (weights [E][n][hidden] codes, a scale per
// output column).
ovl_status a2a_run(const a2a_desc* d, bool f8, const void* const* x, const float* const* x_scale,
                   const int32_t* const* topk_idx, const void* w, const float* w_scale, void* recv_x,
                   float* recv_scale, int32_t* recv_src, int32_t* recv_count, float* y, int64_t* flags,
                   void* workspace, int64_t epoch, const ovl_opts* opts, hipStream_t stream) {
  if (!d) return OVL_EINVAL;
  // The grouped-GEMM tile: the default or the one implemented for the row type.
  const int32_t tile_n = f8 ? kGbn8 : kGbn;
  if (!((d->tile_m == 0 && d->tile_n == 0) || (d->tile_m == kGbm && d->tile_n == tile_n))) return OVL_EUNSUPPORTED;
  if (!recv_count || !flags || !workspace) return OVL_EINVAL;
  const bool empty = d->tokens == 0;  // nothing to read or write but counts and flags
  if (!empty && (!x || !topk_idx || !recv_x || !recv_src || (f8 && (!x_scale || !recv_scale)))) return OVL_EINVAL;
  if (d->ranks < 1 || d->rank < 0 || d->rank >= d->ranks) return OVL_EINVAL;
  if (d->ranks > kA2aMaxRanks || d->experts_per_rank > kA2aMaxExperts) return OVL_EUNSUPPORTED;
  if (d->experts_per_rank < 1 || d->topk < 1 || d->topk > 8 || d->tokens < 0 ||
      d->num_experts != d->ranks * d->experts_per_rank)
    return OVL_ESHAPE;
  const int64_t hid_mult = f8 ? 16 : 8;  // a row moves in 16-byte vectors
  if (d->hidden < hid_mult || d->n < 8 || d->hidden % hid_mult || d->n % 8 || d->flag_stride < 8 ||
      d->flag_stride % 8)
    return OVL_EALIGN;
  const int64_t cap = d->tokens * std::min<int64_t>(d->topk, d->experts_per_rank);
  const int64_t esz = f8 ? 1 : 2;
  // Every operand below 1 GiB and rows below 2^20 elements: buffer offsets stay in 32 bits.
  if (d->tokens > (1 << 20) || d->hidden > (1 << 20) || d->n > (1 << 20) ||
      (int64_t)d->ranks * cap * d->hidden * esz > (1ll << 30) || (int64_t)d->ranks * cap * d->n * 4 > (1ll << 30) ||
      (int64_t)d->experts_per_rank * d->hidden * d->n * esz > (1ll << 30))
    return OVL_EUNSUPPORTED;
  const uint32_t mode = opts ? opts->mode : OVL_MODE_FUSED;
  if (mode != OVL_MODE_FUSED && mode != OVL_MODE_GEMM_ONLY && mode != OVL_MODE_COPY_ONLY) return OVL_EINVAL;
  const bool gemm = mode != OVL_MODE_COPY_ONLY;
  if (gemm && !empty && (!w || !y || (f8 && !w_scale))) return OVL_EINVAL;
  if (!aligned16(recv_x) || !aligned16(workspace) || (gemm && (!aligned16(w) || !aligned16(y))) ||
      (reinterpret_cast<uintptr_t>(flags) & 7u) || (reinterpret_cast<uintptr_t>(recv_src) & 3u) ||
      (reinterpret_cast<uintptr_t>(recv_count) & 3u) || (reinterpret_cast<uintptr_t>(recv_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(w_scale) & 3u))
    return OVL_EALIGN;
  for (int s = 0; s < d->ranks; ++s) {
    if (mode == OVL_MODE_GEMM_ONLY || empty) break;
    if (!x[s] || !topk_idx[s] || (f8 && !x_scale[s])) return OVL_EINVAL;
    if (!aligned16(x[s]) || (reinterpret_cast<uintptr_t>(topk_idx[s]) & 3u) ||
        (f8 && (reinterpret_cast<uintptr_t>(x_scale[s]) & 3u)))
      return OVL_EALIGN;
  }
  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;

  A2aArgs a = {};
  for (int s = 0; s < d->ranks; ++s) {
    if (mode == OVL_MODE_GEMM_ONLY || empty) break;
    a.x[s] = static_cast<const uint8_t*>(x[s]);
    a.x_scale[s] = f8 ? x_scale[s] : nullptr;
    a.topk[s] = topk_idx[s];
  }
  a.x_own = a.x[d->rank];
  a.x_scale_own = a.x_scale[d->rank];
  a.w = static_cast<const uint8_t*>(w);
  a.w_scale = f8 ? w_scale : nullptr;
  a.recv_x = static_cast<uint8_t*>(recv_x);
  a.recv_scale = f8 ? recv_scale : nullptr;
  a.recv_src = recv_src;
  a.recv_count = recv_count;
  a.y = y;
  a.flags = flags;
  a.err = static_cast<ErrRec*>(workspace);
  a.counters = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + OVL_ERROR_RECORD_BYTES);
  a.ticket = a.counters + kA2aMaxRanks;
  a.trace = opts ? opts->trace : nullptr;
  a.tokens = d->tokens;
  a.hidden = d->hidden;
  a.n = d->n;
  a.cap = cap;
  a.row_bytes = d->hidden * esz;
  a.flag_stride = d->flag_stride / 8;
  a.epoch = epoch;
  a.spin_limit = spin_limit_of(opts);
  a.ranks = d->ranks;
  a.rank = d->rank;
  a.topk_n = d->topk;
  a.experts = d->experts_per_rank;

  const int lds = a2a_lds_bytes();
  auto fk = f8 ? (mode == OVL_MODE_GEMM_ONLY ? a2a_fused_kernel<2, true> : a2a_fused_kernel<0, true>)
               : (mode == OVL_MODE_GEMM_ONLY ? a2a_fused_kernel<2, false> : a2a_fused_kernel<0, false>);
  st = allow_lds(reinterpret_cast<const void*>(fk), lds);
  if (st) return st;
  int occ = 0;
  const int threads = 64 * a2a_waves(f8);
  OVL_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fk, threads, lds));
  const int64_t resident = (int64_t)std::max(occ, 1) * di.cus;
  const uint32_t req = opts ? opts->producers : 0;

  if (mode != OVL_MODE_GEMM_ONLY) {
    st = epoch_accept(flags, epoch);
    if (st) return st;
    hipLaunchKernelGGL(a2a_layout_kernel, dim3(d->ranks * d->experts_per_rank), dim3(kLayoutThreads), 0, stream, a);
    OVL_HIP_TRY(hipGetLastError());
  }
  if (mode == OVL_MODE_COPY_ONLY) {
    // One producer per compute unit, each with a contiguous share of the
    // chunks (measured: 175 us against 195 with four per unit).
    const int P = req ? (int)req : di.cus;
    a.producers = P;
    a.consumers = 0;
    hipLaunchKernelGGL(a2a_produce_kernel, dim3(P), dim3(kProduceThreads), 0, stream, a);
    OVL_HIP_TRY(hipGetLastError());
    return OVL_OK;
  }
  int P = 0;
  if (mode == OVL_MODE_FUSED) {
    // Few dedicated producers: consumers take chunks themselves whenever
    // the slice they need is behind, and the producers take tiles of the
    // shared tail once the copy is handed out.  Measured with 256x256
    // tiles and the shared tail (one box, same run): 48 producers (bf16
    // fused 586-587 us, FP8 433-434) beat 32 (603-646, 431-460), 40, 56,
    // 64 (608, 456) and 96 or more; without the tail, 32 had been best
    // (600-628, 455-473), as a producer's compute unit then idled after
    // the copy.
    P = req ? (int)req : 6 * kA2aXcds;
    if (P >= resident) return OVL_EINVAL;
  }
  int64_t Cn = resident - P;
  if (Cn > kA2aXcds) Cn -= Cn % kA2aXcds;
  a.producers = P;
  a.consumers = (int32_t)Cn;
  hipLaunchKernelGGL(fk, dim3(P + Cn), dim3(threads), lds, stream, a);
  OVL_HIP_TRY(hipGetLastError());
  return OVL_OK;
}

}  // namespace
}  // namespace ovl

extern "C" ovl_status a2a_dispatch_grouped_gemm_run(const a2a_desc* d, const void* const* x,
                                                    const int32_t* const* topk_idx, const void* w, void* recv_x,
                                                    int32_t* recv_src, int32_t* recv_count, float* y,
                                                    int64_t* flags, void* workspace, int64_t epoch,
                                                    const ovl_opts* opts, hipStream_t stream) {
  return a2a_run(d, false, x, nullptr, topk_idx, w, nullptr, recv_x, nullptr, recv_src, recv_count, y, flags,
                 workspace, epoch, opts, stream);
}

extern "C" ovl_status a2a_dispatch_grouped_gemm_fp8_run(const a2a_desc* d, const void* const* x8,
                                                        const float* const* x_scale, const int32_t* const* topk_idx,
                                                        const void* w8, const float* w_scale, void* recv_x8,
                                                        float* recv_scale, int32_t* recv_src, int32_t* recv_count,
                                                        float* y, int64_t* flags, void* workspace, int64_t epoch,
                                                        const ovl_opts* opts, hipStream_t stream) {
  return a2a_run(d, true, x8, x_scale, topk_idx, w8, w_scale, recv_x8, recv_scale, recv_src, recv_count, y, flags,
                 workspace, epoch, opts, stream);
}
