// Ring all-reduce with per-tile signals ("Triton-distributed Semantics",
// Example: Ring AllReduce with Overlap), every rank of the ring emulated in
// one launch.  Each rank's vector is cut into R chunks and each chunk into
// tiles; a tile moves on around the ring as soon as it has arrived, with no
// step-wide barrier.
//
// Work items (step s, rank r, tile j), s = 0 .. 2R-3, chunk c = (r - s) mod R:
//   s = 0:              out[r+1][c, j] = in[r][c, j]                 (send)
//   1 <= s <= R-2:      out[r+1][c, j] = out[r][c, j] + in[r][c, j]  (add, send)
//   s = R-1:            v = out[r][c, j] + in[r][c, j]; out[r][c, j] = v and
//                       out[r+1][c, j] = v                          (complete, send)
//   R <= s <= 2R-3:     out[r+1][c, j] = out[r][c, j]                (forward)
// where out[r][c, j] for s >= 1 is what rank r-1 wrote there at step s-1,
// valid once flag (r, s, j) holds the epoch.  The partial sums travel in the
// receivers' output buffers (a chunk's partial at a rank is read before the
// completed chunk reaches it, by the chain of signals), so no other buffer
// is needed.  The sum of chunk c is ((x_c + x_{c+1}) + ...) + x_{c-1}.
//
// Items are handed out in step order from a ticket counter, so the item an
// item waits for was always handed out earlier, to a workgroup that is
// running: the launch needs no co-residency to finish.  Data that another
// rank reads is written with agent-scope stores and read with agent-scope
// loads, and a tile is published with a drain, a barrier and a relaxed flag
// store: an agent-scope release fence per tile (an L2 writeback of the die)
// would cost more than the tile's copy.
#include <algorithm>

#include "device.h"
#include "host.h"

namespace ovl {

namespace {

constexpr int kRingMaxRanks = 16;
constexpr int kRingBlocksPerCu = 2;

struct RingArgs {
  const float* in[kRingMaxRanks];
  float* out[kRingMaxRanks];
  int64_t* flags;
  ErrRec* err;
  int64_t* ticket;  // items handed out (workspace; returned to 0 by the launch's last workgroup)
  int64_t* done;    // workgroups finished (workspace; likewise)
  int64_t n, cs, tile;  // elements per rank, per chunk, per tile
  int64_t epoch, flag_stride;
  uint64_t spin_limit;
  int32_t ranks, tiles;  // tiles per chunk
  int32_t s0, s1;        // steps of this launch: [s0, s1)
  int32_t wait;
};

__device__ inline int64_t imin64(int64_t x, int64_t y) { return x < y ? x : y; }

__device__ inline uint64_t ld8_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float ld4f_agent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}

__device__ inline void st4f_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t add2(uint64_t a, uint64_t b) {
  const float lo = __builtin_bit_cast(float, (uint32_t)a) + __builtin_bit_cast(float, (uint32_t)b);
  const float hi = __builtin_bit_cast(float, (uint32_t)(a >> 32)) + __builtin_bit_cast(float, (uint32_t)(b >> 32));
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}

// Flag slot of (rank r, step s >= 1, tile j).
__device__ inline int64_t ring_flag(const RingArgs& a, int r, int s, int j) {
  return ((int64_t)r * (2 * a.ranks - 2) + (s - 1)) * a.tiles + j;
}

// One item over elements [lo, hi) of rank r's vectors (lo even).  KIND:
// 0 send, 1 add and send, 2 complete and send, 3 forward.
template <int KIND>
__device__ void ring_tile(const RingArgs& a, int r, int64_t lo, int64_t hi) {
  const int nx = r + 1 == a.ranks ? 0 : r + 1;
  const float* own_in = a.in[r];
  float* own_out = a.out[r];
  float* next_out = a.out[nx];
  const int64_t w0 = lo / 2, w1 = hi / 2;  // whole 8-byte words
  const uint64_t* pin = reinterpret_cast<const uint64_t*>(own_in);
  const uint64_t* pown = reinterpret_cast<const uint64_t*>(own_out);
  uint64_t* pmine = reinterpret_cast<uint64_t*>(own_out);
  uint64_t* pnext = reinterpret_cast<uint64_t*>(next_out);
  constexpr int U = 8;
  for (int64_t base = w0 + threadIdx.x; base < w1; base += (int64_t)kThreads * U) {
    uint64_t x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < w1) {
        if (KIND != 3) x[u] = __builtin_nontemporal_load(pin + i);
        if (KIND != 0) y[u] = ld8_agent(pown + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i >= w1) continue;
      const uint64_t v = KIND == 0 ? x[u] : KIND == 3 ? y[u] : add2(y[u], x[u]);
      if (KIND == 2) pmine[i] = v;
      st8_agent(pnext + i, v);
    }
  }
  if ((hi & 1) && hi > lo && threadIdx.x == 0) {  // the vector's odd last element
    const int64_t e = hi - 1;
    const float v = KIND == 0 ? own_in[e] : KIND == 3 ? ld4f_agent(own_out + e) : ld4f_agent(own_out + e) + own_in[e];
    if (KIND == 2) own_out[e] = v;
    st4f_agent(next_out + e, v);
  }
}

__device__ inline int ring_take(const RingArgs& a, int64_t total, int* sh) {
  if (threadIdx.x == 0) {
    const int64_t t = __hip_atomic_fetch_add(a.ticket, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sh = (int)(t < total ? t : total);
  }
  __syncthreads();
  const int v = uniform(*sh);
  __syncthreads();  // *sh is rewritten by the next call
  return v;
}

__global__ __launch_bounds__(kThreads) void ring_kernel(RingArgs a) {
  __shared__ int sh;
  const int R = a.ranks, per_step = R * a.tiles;
  const int64_t total = (int64_t)(a.s1 - a.s0) * per_step;
  for (int it; (it = ring_take(a, total, &sh)) < total;) {
    const int s = a.s0 + it / per_step, rem = it % per_step;
    const int j = rem / R, r = rem % R;  // consecutive tickets: one tile position, every rank
    const int c = ((r - s) % R + R) % R;
    const int64_t clo = imin64(a.n, (int64_t)c * a.cs), chi = imin64(a.n, clo + a.cs);
    const int64_t lo = imin64(chi, clo + (int64_t)j * a.tile), hi = imin64(chi, lo + a.tile);
    if (s >= 1 && a.wait) {
      if (threadIdx.x < 64) {
        const int64_t f = ring_flag(a, r, s, j);
        // Poll, then an agent-scope acquire before the workgroup reads the
        // predecessor's partial (the barrier below hands it to every wave).
        wave_wait(a.flags + f * a.flag_stride, a.epoch, a.spin_limit, a.err, kSiteRing, f);
      }
      __syncthreads();
    }
    if (s == 0)
      ring_tile<0>(a, r, lo, hi);
    else if (s < R - 1)
      ring_tile<1>(a, r, lo, hi);
    else if (s == R - 1)
      ring_tile<2>(a, r, lo, hi);
    else
      ring_tile<3>(a, r, lo, hi);
    // Publish: every wave's stores complete (agent scope), then the flag.
    wave_drain();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nx = r + 1 == R ? 0 : r + 1;
      __hip_atomic_store(a.flags + ring_flag(a, nx, s + 1, j) * a.flag_stride, a.epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // separates this thread-0 branch from the next ticket's
  }
  // The last workgroup out returns the ticket and the count to zero for the
  // next launch (every ticket of this one has been taken by then).
  if (threadIdx.x == 0) {
    const int64_t old = __hip_atomic_fetch_add(a.done, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (int64_t)gridDim.x) {
      __hip_atomic_store(a.ticket, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.done, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// R = 1: the all-reduce is a copy.
__global__ __launch_bounds__(kThreads) void ring_copy_kernel(const float* in, float* out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) out[i] = in[i];
}

struct RingGeom {
  int64_t cs, tiles;
};

RingGeom ring_geometry(const ring_desc* d) {
  RingGeom g;
  g.cs = (d->n + d->ranks - 1) / d->ranks;
  g.cs += g.cs & 1;
  g.tiles = g.cs ? (g.cs + d->tile - 1) / d->tile : 0;
  return g;
}

bool ring_desc_ok(const ring_desc* d) {
  return d && d->ranks >= 1 && d->n >= 0 && d->tile >= 2 && d->tile % 2 == 0 && d->flag_stride >= 8 &&
         d->flag_stride % 8 == 0;
}

}  // namespace

}  // namespace ovl

using namespace ovl;

extern "C" size_t ring_allreduce_flags_bytes(const ring_desc* d) {
  if (!ring_desc_ok(d)) return 0;
  const RingGeom g = ring_geometry(d);
  return (size_t)d->ranks * (size_t)(2 * d->ranks - 2) * (size_t)g.tiles * (size_t)d->flag_stride;
}

// Error record, ticket, finished-workgroup count.
extern "C" size_t ring_allreduce_workspace_bytes(const ring_desc* d) {
  if (!ring_desc_ok(d)) return 0;
  return 256;
}

extern "C" ovl_status ring_allreduce_run(const ring_desc* d, const float* const* in, float* const* out,
                                         int64_t* flags, void* workspace, int64_t epoch, const ovl_opts* opts,
                                         hipStream_t stream) {
  if (!d || !workspace) return OVL_EINVAL;
  if (d->ranks < 1 || d->n < 0) return OVL_EINVAL;
  if (d->ranks > kRingMaxRanks) return OVL_EUNSUPPORTED;
  if (d->tile < 2 || d->tile % 2) return OVL_ESHAPE;
  if (d->flag_stride < 8 || d->flag_stride % 8) return OVL_EALIGN;
  if (d->n > (1ll << 31)) return OVL_EUNSUPPORTED;
  const uint32_t mode = opts ? opts->mode : OVL_MODE_FUSED;
  if (mode != OVL_MODE_FUSED && mode != OVL_MODE_BARRIER) return OVL_EINVAL;
  const RingGeom g = ring_geometry(d);
  const int R = d->ranks;
  if ((int64_t)R * g.tiles > (1 << 24) || (int64_t)(2 * R - 2) * R * g.tiles > (1ll << 30)) return OVL_EUNSUPPORTED;
  if (!aligned16(workspace)) return OVL_EALIGN;
  if (d->n > 0) {
    if (!in || !out) return OVL_EINVAL;
    for (int r = 0; r < R; ++r) {
      if (!in[r] || !out[r]) return OVL_EINVAL;
      if (!aligned16(in[r]) || !aligned16(out[r])) return OVL_EALIGN;
    }
    // No output may overlap an input or another output: partial sums travel
    // through the outputs while the inputs are still read.
    const size_t bytes = (size_t)d->n * 4;
    for (int r = 0; r < R; ++r)
      for (int q = 0; q < R; ++q) {
        const uintptr_t o = reinterpret_cast<uintptr_t>(out[r]);
        const uintptr_t i = reinterpret_cast<uintptr_t>(in[q]);
        const uintptr_t o2 = reinterpret_cast<uintptr_t>(out[q]);
        if (o < i + bytes && i < o + bytes) return OVL_EINVAL;
        if (q != r && o < o2 + bytes && o2 < o + bytes) return OVL_EINVAL;
      }
  }
  const bool has_flags = R > 1 && g.tiles > 0;
  if (has_flags && !flags) return OVL_EINVAL;
  if (flags && (reinterpret_cast<uintptr_t>(flags) & 7u)) return OVL_EALIGN;
  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;
  if (has_flags) {
    st = epoch_accept(flags, epoch);
    if (st) return st;
  } else if (epoch < 1) {
    return OVL_EEPOCH;
  }
  if (d->n == 0) return OVL_OK;
  if (R == 1) {
    const int blocks = (int)std::min<int64_t>((int64_t)di.cus * 4, (d->n + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(ring_copy_kernel, dim3(blocks), dim3(kThreads), 0, stream, in[0], out[0], d->n);
    OVL_HIP_TRY(hipGetLastError());
    return OVL_OK;
  }

  RingArgs a = {};
  for (int r = 0; r < R; ++r) {
    a.in[r] = in[r];
    a.out[r] = out[r];
  }
  a.flags = flags;
  a.err = static_cast<ErrRec*>(workspace);
  a.ticket = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + OVL_ERROR_RECORD_BYTES);
  a.done = a.ticket + 1;
  a.n = d->n;
  a.cs = g.cs;
  a.tile = d->tile;
  a.epoch = epoch;
  a.flag_stride = d->flag_stride / 8;
  a.spin_limit = spin_limit_of(opts);
  a.ranks = R;
  a.tiles = (int32_t)g.tiles;
  const int64_t per_step = (int64_t)R * g.tiles;
  const int blocks = (int)std::min<int64_t>((int64_t)kRingBlocksPerCu * di.cus, std::max<int64_t>(per_step, 1));
  if (mode == OVL_MODE_FUSED) {
    a.s0 = 0;
    a.s1 = 2 * R - 2;
    a.wait = 1;
    hipLaunchKernelGGL(ring_kernel, dim3(blocks), dim3(kThreads), 0, stream, a);
    OVL_HIP_TRY(hipGetLastError());
  } else {
    // One launch per ring step: every tile of a step is in place before any
    // tile of the next moves (the launch boundary orders them), as a
    // collective without tile signals would run.
    a.wait = 0;
    for (int s = 0; s < 2 * R - 2; ++s) {
      a.s0 = s;
      a.s1 = s + 1;
      hipLaunchKernelGGL(ring_kernel, dim3(blocks), dim3(kThreads), 0, stream, a);
      OVL_HIP_TRY(hipGetLastError());
    }
  }
  return OVL_OK;
}
