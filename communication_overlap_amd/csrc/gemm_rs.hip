// GEMM -> ReduceScatter with tile-level overlap ("Triton-distributed
// Semantics", Kernel Design Patterns, "GEMM and ReduceScatter Overlapping").
//
// One persistent launch of GEMM workgroups.  The local product's rows split
// into R blocks.  The own block's tiles come first, then the blocks destined
// for peers, starting at block rank+1 (the mirror of the all-gather's
// swizzle).
//   - Own tile: the fp32 accumulator is stored to `out` and an own-tile flag
//     in the workspace is published.
//   - Peer tile: the fp32 tile is stored to that peer's partial buffer and
//     its out flag is published (put + signal).  Then the workgroup runs one
//     reduce job: the own block's tile rows are split evenly over all peer
//     tiles, and job j, for its share of rows, waits for the own tiles and
//     the peers' partials it covers (own-tile flags, in flags), sums the
//     partials in ascending peer order, S = P_a + P_b + ..., and writes
//     out = acc + S over the stored accumulator.  This spreads the reading of
//     the R-1 partials over the whole launch, and nothing waits at its end.
// Every output element is therefore acc + ((P_a + P_b) + ...) in fp32, in
// this fixed order, whatever the timing.
#include <algorithm>

#include "device.h"
#include "gemm_core.h"
#include "host.h"

namespace ovl {

namespace {

constexpr int kRsMaxRanks = 16;
constexpr int kRsXcds = 8;
// Tiles: 256 x 256 (the default) or 128 x 128.  Wavefronts per workgroup:
// the 256 x 256 tile as a 2 x 4 grid of waves, two per SIMD (one's MFMAs
// cover the other's LDS reads; measured faster than 4); the 128 x 128 tile
// as 2 x 2.
template <int TILE>
constexpr int rs_waves() { return TILE == 256 ? 8 : 4; }

struct RsArgs {
  float* peer_out[kRsMaxRanks];
  const float* peer_in[kRsMaxRanks];
  const uint16_t* a;
  const uint16_t* b;
  float* out;
  int64_t* out_flags;
  const int64_t* in_flags;
  int64_t* own_flags;  // [tiles per block] in the workspace
  ErrRec* err;
  int64_t m, n, k, bm;  // bm = rows per block
  int64_t flag_stride;  // int64 slots
  int64_t epoch;
  uint64_t spin_limit;
  int32_t ranks, rank;
  int32_t tr, tc;       // row / column tiles per block
  int32_t workers;
  int32_t sync;         // 0: no in/out flag traffic (measurement of the work alone)
};

// Own-row space: own tile t owns rows [t*TILE, t*TILE + TILE) of it (tile
// row trow*TILE + r of the block, columns of tile column tcol), cut into
// lines of 64 lanes x 4 columns: one row of a 256-wide tile, two rows of a
// 128-wide one.  Job j of J covers lines [j*OL/J, (j+1)*OL/J), OL =
// tiles_per_block * TILE / rows per line.
__device__ inline int64_t job_begin(int64_t j, int64_t J, int64_t OL) { return j * OL / J; }

// 16 bytes per lane from global memory straight into LDS at lds_block +
// 16 * lane (gfx950's global load to LDS; no registers hold the data).
__device__ inline void gload16_to_lds(const void* g, uint32_t lds_block) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_block), "v"(g) : "memory", "m0");
}

// Lines [q0, q1) of the own-row space: out = acc + ((P_a + P_b) + ...), the
// partials in ascending peer order.  64 lanes of 16 bytes cover one line
// (a 256-column row, or two 128-column rows).  Each wave stages the
// accumulator line and the R-1 partial lines of `rw` lines (1 KiB each) in
// its own 16 KiB of the idle GEMM stage
// area with global-to-LDS loads, all issued before the first add, then
// sums them: twice the rows in flight that registers allowed (measured:
// fused 169 -> 156-163 us, reduction-included GEMM-only 163-165 -> 151-152
// us at 8192x4096x1792 over 8 ranks).  Index arithmetic is 32-bit (a block
// has fewer than 2^31 elements).
template <int TILE>
__device__ void reduce_rows_lds(const RsArgs& a, int64_t q0, int64_t q1, uint16_t* lds) {
  constexpr int LPR = TILE / 4;      // lanes per row
  constexpr int RPL = 64 / LPR;      // rows per line
  constexpr int LPT = TILE / RPL;    // lines per tile
  uint8_t* l8 = reinterpret_cast<uint8_t*>(lds);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = a.ranks;
  const int rw = R <= 8 ? 2 : 1;
  const uint32_t wbase = lds_addr(l8) + (uint32_t)w * 16384u;
  const int tc = a.tc, n = (int)a.n, bm = (int)a.bm;
  for (int q = (int)q0 + w * rw; q < (int)q1; q += rs_waves<TILE>() * rw) {
    for (int u = 0; u < rw; ++u) {
      const int qq = q + u;
      const int t = qq / LPT;
      const int row = (t / tc) * TILE + (qq % LPT) * RPL + lane / LPR;
      const int col = (t % tc) * TILE + (lane % LPR) * 4;
      if (qq >= (int)q1) continue;               // wave-uniform
      if (row >= bm || col >= n) continue;       // lanes past M or N load nothing
      const int off = row * n + col;
      const uint32_t slot = wbase + (uint32_t)u * 8192u;
      gload16_to_lds(a.out + off, slot);
      int si = 1;
#pragma unroll
      for (int p = 0; p < kRsMaxRanks; ++p)
        if (p < R && p != a.rank) gload16_to_lds(a.peer_in[p] + off, slot + 1024u * (uint32_t)si++);
    }
    wave_drain();
    for (int u = 0; u < rw; ++u) {
      const int qq = q + u;
      const int t = qq / LPT;
      const int row = (t / tc) * TILE + (qq % LPT) * RPL + lane / LPR;
      const int col = (t % tc) * TILE + (lane % LPR) * 4;
      if (qq >= (int)q1 || row >= bm || col >= n) continue;
      const uint8_t* slot = l8 + (size_t)w * 16384 + (size_t)u * 8192 + (size_t)lane * 16;
      const f32x4 acc = *OVL_LDS(const f32x4, slot);
      f32x4 sum = *OVL_LDS(const f32x4, slot + 1024);
      for (int si = 2; si < R; ++si) sum += *OVL_LDS(const f32x4, slot + 1024 * si);
      *reinterpret_cast<f32x4*>(a.out + (int64_t)row * n + col) = acc + sum;
    }
  }
}

template <int TILE>
__device__ void reduce_job(const RsArgs& a, int64_t j, int64_t J, bool& timed_out, uint16_t* lds) {
  constexpr int LPT = TILE * TILE / 256;  // lines per tile
  const int tpb = a.tr * a.tc;
  const int64_t OL = (int64_t)tpb * LPT;
  const int64_t q0 = job_begin(j, J, OL), q1 = job_begin(j + 1, J, OL);
  if (q0 >= q1) return;
  // Wave 0 waits for the own tiles this job touches and, with flags on, for
  // every peer's partial of them; the barrier hands the acquire to the
  // other waves.
  // Every flag the job needs (own tiles, and with flags on every peer's
  // partial of them) is read in one round trip, lanes in parallel, until all
  // are set; then one acquire covers them.  Flag i of the job: tile
  // t0 + i / R, and within it the own-tile flag (peer slot `rank`) or peer
  // p's in flag.
  if (threadIdx.x < 64 && !timed_out) {
    const int64_t t0 = q0 / LPT, nt = (q1 - 1) / LPT - t0 + 1;
    const int64_t nflags = nt * (a.sync ? a.ranks : 1);
    // (32-bit index arithmetic: a job has few flags, and a poll should not
    // pay for 64-bit divisions.)
    auto flag_at = [&](int64_t i64, int64_t* idx, int32_t* site) -> const int64_t* {
      const int32_t i = (int32_t)i64;
      const int64_t t = t0 + (a.sync ? i / a.ranks : i);
      const int p = a.sync ? i % a.ranks : a.rank;
      if (p == a.rank) {
        *idx = t;
        *site = kSiteRsOwn;
        return a.own_flags + t;
      }
      *idx = (int64_t)p * tpb + t;
      *site = kSiteRsIn;
      return a.in_flags + *idx * a.flag_stride;
    };
    for (uint64_t polls = 0;; ++polls) {
      bool missing = false;
      for (int64_t i = lane_id(); i < nflags; i += 64) {
        int64_t idx;
        int32_t site;
        const int64_t v = __hip_atomic_load(flag_at(i, &idx, &site), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        missing |= v < a.epoch;
        check_epoch(a.err, site, idx, v, a.epoch);
      }
      if (!__ballot(missing)) break;
      if (polls >= a.spin_limit) {
        for (int64_t i = 0; i < nflags && !timed_out; ++i) {  // name the first missing flag
          int64_t idx;
          int32_t site;
          if (!wave_poll(flag_at(i, &idx, &site), a.epoch, 0, a.err, site, idx)) timed_out = true;
        }
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    wave_acquire();
  }
  __syncthreads();
  reduce_rows_lds<TILE>(a, q0, q1, lds);
}

template <int SYNC, int TILE>
__global__ __launch_bounds__(64 * rs_waves<TILE>(), 1) void gemm_rs_kernel(RsArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  constexpr int BM = TILE, BN = TILE, NW = rs_waves<TILE>();
  const int tpb = a.tr * a.tc;
  const int64_t total = (int64_t)a.ranks * tpb;
  const int64_t J = (int64_t)(a.ranks - 1) * tpb;  // reduce jobs = peer tiles
  const int Cn = a.workers;
  const int groups = (Cn % kRsXcds == 0) ? kRsXcds : 1;
  const int per = Cn / groups;
  const int cidx = blockIdx.x;
  const int x = cidx % groups, q = cidx / groups;
  bool timed_out = false;
  // Half of each die's workgroups run their first reduce job after their
  // next tile instead of right after the first: the workgroups would
  // otherwise all reduce at once (memory-bound, matrix units idle) and all
  // compute at once; staggered, one half's reduction overlaps the other
  // half's tile.  Any order gives the same bits (a job's sum order is fixed).
  const bool stagger = (q & 1) != 0;
  int64_t deferred = -1;  // a peer tile whose reduce job waits for the next tile

  for (int64_t w = 0;; ++w) {
    const int64_t j = deal_item(w, x, q, groups, per, total);
    if (j < 0) break;
    // Own tiles first, then peer tile pj of block rank+1+pj/tpb.
    const int64_t pj = j - tpb;
    const int blk = pj < 0 ? a.rank : (int)((a.rank + 1 + pj / tpb) % a.ranks);
    int t = (int)(pj < 0 ? j : pj % tpb);
    if (groups == kRsXcds && 2 * per == tpb && a.tc % 2 == 0 && (w + 1) * Cn <= total) {
      // A die's share of a round is half a block: take it as all row tiles
      // x half the column tiles (fewer A and B panels per die than whole
      // rows of tiles; measured fused 162-166 -> 156-157 us at 8192x4096x1792
      // over 8 ranks).  Only which workgroup computes a tile changes.
      const int hc = a.tc / 2, half = ((x * per) % tpb) / per;
      t = (q / hc) * a.tc + half * hc + q % hc;
    }
    const int trow = t / a.tc, tcol = t % a.tc;

    Operands op;
    op.a = a.a + (int64_t)blk * a.bm * a.k;
    op.lda = a.k;
    op.m_valid = a.bm;
    op.b = a.b;
    op.ldb = a.n;
    op.n0 = (int64_t)tcol * BN;
    op.n_valid = a.n;
    op.k = a.k;
    const int64_t m0 = (int64_t)trow * BM;

    Acc<BM, BN, NW> acc;
    gemm_tile<BM, BN, 64, 0, false, NW>(acc, op, m0, lds, [](int64_t, int64_t) {});

    // Partial and own tiles are stored with agent-scope stores (the sc1 bit:
    // complete at the device's point of coherence once drained), so their
    // flags need a drain, a barrier and a relaxed flag store, and no release
    // fence with its L2 writeback of the die (measured: fused 182 -> 165 us
    // at 8192x4096x1792 over 8 ranks, 512 such fences per launch).
    auto publish = [&](int64_t* f) {
      wave_drain();
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(f, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (blk != a.rank) {
      acc_store<BM, BN, kAuxAgent, NW>(acc, a.peer_out[blk], a.n, m0, op.n0, a.bm, a.n);
      if (SYNC) publish(a.out_flags + ((int64_t)blk * tpb + t) * a.flag_stride);
      if (stagger && w == 0 && deal_item(1, x, q, groups, per, total) >= 0) {
        deferred = pj;
      } else {
        reduce_job<TILE>(a, pj, J, timed_out, lds);
      }
    } else {
      acc_store<BM, BN, kAuxAgent, NW>(acc, a.out, a.n, m0, op.n0, a.bm, a.n);
      if (J > 0) publish(a.own_flags + t);
    }
    if (w == 1 && deferred >= 0) {
      reduce_job<TILE>(a, deferred, J, timed_out, lds);
      deferred = -1;
    }
  }
}

// LDS: the GEMM stages, which the reduction reuses as 16 KiB per wave.
template <int TILE>
constexpr int rs_lds_bytes() {
  return std::max(TileCfg<TILE, TILE, 64, 0, rs_waves<TILE>()>::LDS_BYTES, rs_waves<TILE>() * 16384);
}

bool rs_tile_ok(const gemm_rs_desc* d) { return d->tile_m == d->tile_n && (d->tile_m == 256 || d->tile_m == 128); }

template <int TILE>
ovl_status rs_launch(const gemm_rs_desc* d, RsArgs& r, void* workspace, int64_t* out_flags, int64_t epoch,
                     uint32_t mode, const DeviceInfo& di, hipStream_t stream) {
  constexpr int threads = 64 * rs_waves<TILE>();
  const int lds = rs_lds_bytes<TILE>();
  ovl_status st = allow_lds(reinterpret_cast<const void*>(&gemm_rs_kernel<0, TILE>), lds);
  if (st) return st;
  st = allow_lds(reinterpret_cast<const void*>(&gemm_rs_kernel<1, TILE>), lds);
  if (st) return st;
  int occ = 0;
  OVL_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_rs_kernel<1, TILE>, threads, lds));
  const int64_t total = (int64_t)d->ranks * r.tr * r.tc;
  int64_t workers = std::min<int64_t>(total, (int64_t)std::max(occ, 1) * di.cus);
  if (workers > kRsXcds) workers -= workers % kRsXcds;
  r.workers = (int32_t)workers;
  st = epoch_check(workspace, epoch);
  if (st) return st;
  if (d->ranks > 1 && mode == OVL_MODE_FUSED) {
    st = epoch_accept(out_flags, epoch);
    if (st) return st;
  }
  st = epoch_accept(workspace, epoch);
  if (st) return st;
  if (mode == OVL_MODE_FUSED)
    hipLaunchKernelGGL((gemm_rs_kernel<1, TILE>), dim3(workers), dim3(threads), lds, stream, r);
  else
    hipLaunchKernelGGL((gemm_rs_kernel<0, TILE>), dim3(workers), dim3(threads), lds, stream, r);
  OVL_HIP_TRY(hipGetLastError());
  return OVL_OK;
}

}  // namespace

}  // namespace ovl

using namespace ovl;

extern "C" size_t gemm_rs_flags_bytes(const gemm_rs_desc* d) {
  if (!d || d->ranks < 1 || d->m < 1 || d->n < 1 || d->flag_stride < 8 || d->m % d->ranks || !rs_tile_ok(d))
    return 0;
  const int64_t bm = d->m / d->ranks;
  const int64_t tpb = ceil_div(bm, d->tile_m) * ceil_div(d->n, d->tile_n);
  return (size_t)(d->ranks * tpb * d->flag_stride);
}

// Error record, then one int64 flag per own tile.
extern "C" size_t gemm_rs_workspace_bytes(const gemm_rs_desc* d) {
  if (!d || d->ranks < 1 || d->m < 1 || d->n < 1 || d->m % d->ranks || !rs_tile_ok(d)) return 0;
  const int64_t bm = d->m / d->ranks;
  const int64_t tpb = ceil_div(bm, d->tile_m) * ceil_div(d->n, d->tile_n);
  return OVL_ERROR_RECORD_BYTES + 8 * (size_t)tpb;
}

extern "C" ovl_status gemm_rs_run(const gemm_rs_desc* d, const void* a, const void* b, float* const* peer_out,
                                  const float* const* peer_in, float* out, int64_t* out_flags,
                                  const int64_t* in_flags, void* workspace, int64_t epoch, const ovl_opts* opts,
                                  hipStream_t stream) {
  if (!d || !a || !b || !out || !workspace) return OVL_EINVAL;
  if (d->ranks < 1 || d->rank < 0 || d->rank >= d->ranks) return OVL_EINVAL;
  if (d->ranks > kRsMaxRanks) return OVL_EUNSUPPORTED;
  if (!rs_tile_ok(d)) return OVL_EUNSUPPORTED;
  if (d->m < 1 || d->n < 8 || d->k < 8 || d->m % d->ranks) return OVL_ESHAPE;
  if (d->n % 8 || d->k % 8 || d->flag_stride < 8 || d->flag_stride % 8) return OVL_EALIGN;
  // Every operand below 1 GiB and rows below 2^20 elements: buffer offsets stay in 32 bits.
  if (d->m > (1 << 20) || d->n > (1 << 20) || d->k > (1 << 20) || d->m * d->k * 2 > (1ll << 30) ||
      d->k * d->n * 2 > (1ll << 30) || d->m * d->n * 4 > (1ll << 30))
    return OVL_EUNSUPPORTED;
  const uint32_t mode = opts ? opts->mode : OVL_MODE_FUSED;
  if (mode != OVL_MODE_FUSED && mode != OVL_MODE_GEMM_ONLY) return OVL_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out) || !aligned16(workspace)) return OVL_EALIGN;
  if (d->ranks > 1) {
    if (!peer_out || !peer_in || !out_flags || !in_flags) return OVL_EINVAL;
    if ((reinterpret_cast<uintptr_t>(out_flags) & 7u) || (reinterpret_cast<uintptr_t>(in_flags) & 7u))
      return OVL_EALIGN;
    for (int p = 0; p < d->ranks; ++p) {
      if (p == d->rank) continue;
      if (!peer_out[p] || !peer_in[p]) return OVL_EINVAL;
      if (!aligned16(peer_out[p]) || !aligned16(peer_in[p])) return OVL_EALIGN;
    }
  }
  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;

  RsArgs r = {};
  for (int p = 0; p < d->ranks; ++p) {
    if (p == d->rank) continue;
    r.peer_out[p] = peer_out[p];
    r.peer_in[p] = peer_in[p];
  }
  r.a = static_cast<const uint16_t*>(a);
  r.b = static_cast<const uint16_t*>(b);
  r.out = out;
  r.out_flags = out_flags;
  r.in_flags = in_flags;
  r.err = static_cast<ErrRec*>(workspace);
  r.own_flags = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + OVL_ERROR_RECORD_BYTES);
  r.m = d->m;
  r.n = d->n;
  r.k = d->k;
  r.bm = d->m / d->ranks;
  r.flag_stride = d->flag_stride / 8;
  r.epoch = epoch;
  r.spin_limit = spin_limit_of(opts);
  r.ranks = d->ranks;
  r.rank = d->rank;
  r.tr = (int32_t)ceil_div(r.bm, d->tile_m);
  r.tc = (int32_t)ceil_div(d->n, d->tile_n);
  r.sync = mode == OVL_MODE_FUSED;
  return d->tile_m == 256 ? rs_launch<256>(d, r, workspace, out_flags, epoch, mode, di, stream)
                          : rs_launch<128>(d, r, workspace, out_flags, epoch, mode, di, stream);
}
