// MoE combine: the reverse all-to-all of this rank's expert outputs, then
// the gate-weighted sum back in token order (the Aboleth README's compiled
// MoE dispatch *and combine*; the reverse all-to-all for expert-parallel MoE
// of the Triton distributed tutorials).  The same per-slice signal
// discipline as the dispatch, in reverse:
//  1. Layout, one workgroup per (rank q, local expert e) over this rank's
//     own routing: the row of every (token, choice) in q's slice of this
//     rank's tokens (ordered by (local expert, token), as q's dispatch
//     placed them).  It also zeroes this run's slice counters.
//  2. Fused, two workgroups per compute unit.  First the reverse puts, one
//     peer slice at a time (positions rank+1, rank+2, ...): y[s] (s != rank,
//     the rows this rank computed for source s, already in slice order) is
//     copied into ret_out[s], every workgroup taking a grid-strided share;
//     the last workgroup to finish slice s sets out_flags[s] (put + signal).
//     Then this rank's tokens, one per wave: once the flags of the peers'
//     returned rows are set, out[t] = sum over choices k (ascending) of
//     gates[t][k] * Y(t, k), Y from y[rank] for local experts or from the
//     returning peer's ret_in rows.
#include <algorithm>

#include "device.h"
#include "gemm_core.h"
#include "host.h"

namespace ovl {

namespace {

constexpr int kCbLoadAux = 2;  // the put reads each row once: nontemporal loads (the nt bit)

constexpr int kCbMaxRanks = 16;
constexpr int kCbBlocksPerCu = 2;

struct CombineArgs {
  float* ret_out[kCbMaxRanks];
  const float* ret_in[kCbMaxRanks];
  const float* y;
  const int32_t* recv_count;
  const int32_t* topk;
  const float* gates;
  float* out;
  int64_t* out_flags;
  const int64_t* in_flags;
  int32_t* pos;       // [tokens][topk] row of each choice in its owner's slice (workspace)
  int64_t* counters;  // [R] workgroups done with each slice's put (workspace)
  ErrRec* err;
  int64_t tokens, n, cap;
  int64_t flag_stride;  // int64 slots
  int64_t epoch;
  uint64_t spin_limit;
  int32_t ranks, rank, topk_n, experts;
  int32_t do_put, do_sum, wait_in;
};

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

// Workgroup (q, e): the choices of this rank's tokens that pick global
// expert q*E + e take rows base + 0, 1, ... of q's slice, base = the count
// of choices picking q's experts below e; order (token, choice).  Wave w
// takes a contiguous range of the choices and reads it 64 at a time, lane l
// the l-th (coalesced); the wave totals give each wave's first row, and a
// ballot each matching lane's place after the matches of the lanes below.
// Sixteen waves per (peer, expert) workgroup: at the MoE workload each wave
// reads its share of the choices in one round of loads per pass.
constexpr int kCbLayoutThreads = 1024;

__global__ __launch_bounds__(kCbLayoutThreads) void combine_layout_kernel(CombineArgs a) {
  constexpr int NWV = kCbLayoutThreads / 64;
  constexpr int B = 8;  // 64-choice groups loaded before they are looked at
  __shared__ int smem[2 * NWV];
  const int q = blockIdx.x / a.experts, e = blockIdx.x % a.experts;
  const int e_lo = q * a.experts;
  const int lane = lane_id(), wave = uniform(threadIdx.x >> 6);
  const int64_t NE = a.tokens * a.topk_n;
  const int64_t per_w = ((NE + NWV - 1) / NWV + 63) / 64 * 64;
  const int64_t w0 = min(NE, wave * per_w), w1 = min(NE, w0 + per_w);
  int lt = 0, eq = 0;
  for (int64_t i = w0; i < w1; i += 64 * B) {
    int32_t v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int64_t k = i + 64 * j + lane;
      v[j] = k < w1 ? a.topk[k] : -1;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int ex = v[j] - e_lo;
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
  int run = 0;  // first row of this wave's matches
#pragma unroll
  for (int w = 0; w < NWV; ++w) run += smem[NWV + w] + (w < wave ? smem[w] : 0);
  if (eq)
    for (int64_t i = w0; i < w1; i += 64 * B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int64_t k = i + 64 * j + lane;
        v[j] = k < w1 ? a.topk[k] : -1;
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const bool hit = v[j] - e_lo == e;
        const uint64_t m = __ballot(hit);
        if (hit)
          a.pos[i + 64 * j + lane] =
              run + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        run += __popcll(m);
      }
    }
  if (blockIdx.x == 0 && threadIdx.x < a.ranks) a.counters[threadIdx.x] = 0;
}

// Rows this rank sends back to each peer slice (rebuilt by every workgroup).
struct CbGeom {
  int32_t rows[kCbMaxRanks];
};

__device__ inline int cb_slice_at(const CombineArgs& a, int pos) { return (a.rank + 1 + pos) % a.ranks; }

__device__ void cb_geometry(const CombineArgs& a, CbGeom* g) {
  if (threadIdx.x < kCbMaxRanks) {
    const int s = threadIdx.x;
    int r = 0;
    if (s < a.ranks && s != a.rank && a.tokens > 0)
      for (int e = 0; e < a.experts; ++e) r += a.recv_count[s * a.experts + e];
    g->rows[s] = (int)min((int64_t)r, a.cap);  // a slice holds at most cap rows
  }
  __syncthreads();
}

// This workgroup's arrival for slice s, once every wave's stores of it are
// complete: the last workgroup to arrive sets out_flags[s].
__device__ void cb_arrive(const CombineArgs& a, int s) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t old = __hip_atomic_fetch_add(a.counters + s, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (int64_t)gridDim.x) {
      wave_acquire();
      __hip_atomic_store(a.out_flags + (int64_t)s * a.flag_stride, a.epoch, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // separates this thread-0 branch from the next one
}

// Reverse put of slice s: its rows of y[s] are contiguous, as are their
// places in ret_out[s].  Every workgroup copies a grid-strided share of the
// slice's 16-byte vectors, eight in flight per lane, as buffer loads and
// agent-scope buffer stores with no branch around them (a vector past the
// end gets an offset past its buffer: the load returns zeros, the store is
// dropped).  The arrival for the previous slice `prev` (or -1) waits behind
// this slice's first loads: the vector memory counter completes in order, so
// once no more than those eight remain, the previous slice's stores are
// complete, and the drain before an arrival no longer empties the pipeline.
__device__ void cb_put_slice(const CombineArgs& a, int s, int64_t rows, int prev) {
  constexpr int U = 8;  // 16 measured the same
  const uint32_t vecs = (uint32_t)(rows * a.n / 4);  // the host keeps y under 1 GiB
  const rsrc_t rs = make_rsrc(a.y + (int64_t)s * a.cap * a.n, (int64_t)vecs * 16);
  const rsrc_t rd = make_rsrc(a.ret_out[s], (int64_t)vecs * 16);
  const uint32_t stride = gridDim.x * kThreads;
  u32x4 v[U];
  uint32_t off[U];
  auto load = [&](uint32_t i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = i + u * stride;
      off[u] = k < vecs ? k * 16 : kOOB;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[u], 0, kCbLoadAux);
    }
  };
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  asm volatile("" ::: "memory");  // the previous slice's stores stay ahead of these loads
  load(i);
  static_assert(U == 8, "the wait below leaves the U loads in flight");
  if (uniform(prev) >= 0) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    cb_arrive(a, prev);
  }
  for (;;) {
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (int)off[u], 0, kAuxAgent);
    i += U * stride;
    if (i >= vecs) break;
    load(i);
  }
}

// Tokens t0 + j * stride (j < J), by one wave.  The lanes first load every
// (token, choice)'s expert id, row and gate at once (lane j * KMAX + k), the
// wave reads them back as scalars; then a lane sums 16-byte vectors lane,
// lane + 64, ... of each output row, V at a time, all J tokens' and all
// choices' loads issued before the first add.  KMAX bounds topk; J * KMAX * V
// = 16 keeps the loads in flight at 64 registers.
template <int KMAX, int J>
__device__ void cb_sum_tokens(const CombineArgs& a, int64_t t0, int64_t stride) {
  constexpr int V = 16 / (KMAX * J);
  static_assert(V >= 1 && J * KMAX <= 64, "loads in flight per lane");
  const int lane = lane_id();
  const int64_t vpr = a.n / 4;
  // Metadata, one (token, choice) per lane.
  int32_t my_e = -1;
  int32_t my_p = 0;
  float my_g = 0.f;
  {
    const int j = lane / KMAX, k = lane % KMAX;
    const int64_t t = t0 + j * stride;
    if (j < J && k < a.topk_n && t < a.tokens) {
      my_e = a.topk[t * a.topk_n + k];
      my_p = a.pos[t * a.topk_n + k];
      my_g = a.gates[t * a.topk_n + k];
    }
  }
  const f32x4* rowp[J][KMAX];
  float gk[J][KMAX];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int src = j * KMAX + k;
      const int32_t e = __builtin_amdgcn_readlane(my_e, src);
      const int64_t p = __builtin_amdgcn_readlane(my_p, src);
      gk[j][k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), src));
      rowp[j][k] = nullptr;
      if (e < 0 || e >= a.ranks * a.experts) continue;  // not an expert (or no token): contributes nothing
      const int q = e / a.experts;
      rowp[j][k] = reinterpret_cast<const f32x4*>(q == a.rank ? a.y + ((int64_t)a.rank * a.cap + p) * a.n
                                                               : a.ret_in[q] + p * a.n);
    }
  for (int64_t v0 = lane; v0 < vpr; v0 += 64 * V) {
    f32x4 x[J][KMAX][V];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
#pragma unroll
        for (int u = 0; u < V; ++u)
          if (rowp[j][k] && v0 + 64 * u < vpr) x[j][k][u] = __builtin_nontemporal_load(rowp[j][k] + v0 + 64 * u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t t = t0 + j * stride;
      if (t >= a.tokens) continue;
      f32x4* o = reinterpret_cast<f32x4*>(a.out + t * a.n);
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if (v0 + 64 * u >= vpr) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (rowp[j][k]) acc += gk[j][k] * x[j][k][u];
        o[v0 + 64 * u] = acc;
      }
    }
  }
}

// The peers' returned rows: every in flag, lanes in parallel; wave 0 of
// each workgroup polls, the workgroup continues after its acquire.
__device__ void cb_wait_in(const CombineArgs& a) {
  if (threadIdx.x < 64) {
    for (uint64_t polls = 0;; ++polls) {
      bool missing = false;
      for (int q = lane_id(); q < a.ranks; q += 64)
        if (q != a.rank) {
          const int64_t v =
              __hip_atomic_load(a.in_flags + (int64_t)q * a.flag_stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          missing |= v < a.epoch;
          check_epoch(a.err, kSiteCbIn, q, v, a.epoch);
        }
      if (!__ballot(missing)) break;
      if (polls >= a.spin_limit) {
        for (int q = 0; q < a.ranks; ++q)
          if (q != a.rank && !wave_poll(a.in_flags + (int64_t)q * a.flag_stride, a.epoch, 0, a.err, kSiteCbIn, q))
            break;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    wave_acquire();
  }
  __syncthreads();
}

template <int KMAX>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ CbGeom g;
  cb_geometry(a, &g);
  if (a.do_put) {
    // Peers this rank sends nothing back to are complete at once.
    if (blockIdx.x == 0 && threadIdx.x < a.ranks && threadIdx.x != a.rank && g.rows[threadIdx.x] == 0)
      __hip_atomic_store(a.out_flags + (int64_t)threadIdx.x * a.flag_stride, a.epoch, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    // Slices in position order rank+1, rank+2, ...: each is complete (and
    // signalled) before the next begins, so peers can start on it early.
    const int ranks = uniform(a.ranks);  // a loop around barriers: bounded by a scalar
    int prev = -1;  // the slice put last, not arrived for yet
    for (int pos = 0; pos + 1 < ranks; ++pos) {
      // scalars to the compiler: the slice picks the buffer resources
      const int s = uniform(cb_slice_at(a, pos));
      const int rows = uniform(g.rows[s]);
      if (!rows) continue;
      cb_put_slice(a, s, rows, prev);
      prev = s;
    }
    if (uniform(prev) >= 0) {
      wave_drain();
      cb_arrive(a, prev);
    }
  }
  if (!a.do_sum) return;
  if (a.wait_in) cb_wait_in(a);
  // J tokens per wave at a time, waves grid-strided over the tokens.
  constexpr int J = KMAX <= 2 ? 2 : 1;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); t < a.tokens; t += waves * J)
    cb_sum_tokens<KMAX, J>(a, t, waves);
}

}  // namespace

}  // namespace ovl

using namespace ovl;

extern "C" size_t a2a_combine_flags_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1 || d->flag_stride < 8) return 0;
  return (size_t)d->ranks * (size_t)d->flag_stride;
}

// Error record, then the R slice counters (256 bytes in all), then the
// choice rows int32 [tokens][topk].
extern "C" size_t a2a_combine_workspace_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1 || d->tokens < 0 || d->topk < 1) return 0;
  return 256 + aligned_up(4 * (size_t)d->tokens * (size_t)d->topk, 256);
}

extern "C" ovl_status a2a_combine_run(const a2a_desc* d, const float* y, const int32_t* recv_count,
                                      float* const* ret_out, const float* const* ret_in,
                                      const int32_t* topk_idx, const float* gates, float* out,
                                      int64_t* out_flags, const int64_t* in_flags, void* workspace,
                                      int64_t epoch, const ovl_opts* opts, hipStream_t stream) {
  if (!d || !workspace) return OVL_EINVAL;
  if (d->ranks < 1 || d->rank < 0 || d->rank >= d->ranks) return OVL_EINVAL;
  if (d->ranks > kCbMaxRanks || d->experts_per_rank > 64) return OVL_EUNSUPPORTED;
  if (d->experts_per_rank < 1 || d->topk < 1 || d->topk > 8 || d->tokens < 0 ||
      d->num_experts != d->ranks * d->experts_per_rank)
    return OVL_ESHAPE;
  if (d->n < 8 || d->n % 8 || d->flag_stride < 8 || d->flag_stride % 8) return OVL_EALIGN;
  const int64_t cap = d->tokens * std::min<int64_t>(d->topk, d->experts_per_rank);
  if (d->tokens > (1 << 20) || d->n > (1 << 20) || (int64_t)d->ranks * cap * d->n * 4 > (1ll << 30))
    return OVL_EUNSUPPORTED;
  const uint32_t mode = opts ? opts->mode : OVL_MODE_FUSED;
  if (mode != OVL_MODE_FUSED && mode != OVL_MODE_COPY_ONLY && mode != OVL_MODE_GEMM_ONLY) return OVL_EINVAL;
  const bool put = mode != OVL_MODE_GEMM_ONLY, sum = mode != OVL_MODE_COPY_ONLY;
  const bool empty = d->tokens == 0;
  const bool peers = d->ranks > 1;
  if (!recv_count) return OVL_EINVAL;
  if (put && peers && !out_flags) return OVL_EINVAL;
  if (sum && mode == OVL_MODE_FUSED && peers && !in_flags) return OVL_EINVAL;
  if (!empty) {
    if (!y) return OVL_EINVAL;
    if (sum && (!topk_idx || !gates || !out)) return OVL_EINVAL;
    if (!aligned16(y) || (sum && !aligned16(out)) || (sum && (reinterpret_cast<uintptr_t>(topk_idx) & 3u)) ||
        (sum && (reinterpret_cast<uintptr_t>(gates) & 3u)))
      return OVL_EALIGN;
    for (int q = 0; q < d->ranks; ++q) {
      if (q == d->rank) continue;
      if ((put && (!ret_out || !ret_out[q])) || (sum && (!ret_in || !ret_in[q]))) return OVL_EINVAL;
      if ((put && !aligned16(ret_out[q])) || (sum && !aligned16(ret_in[q]))) return OVL_EALIGN;
    }
  }
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(recv_count) & 3u) ||
      (out_flags && (reinterpret_cast<uintptr_t>(out_flags) & 7u)) ||
      (in_flags && (reinterpret_cast<uintptr_t>(in_flags) & 7u)))
    return OVL_EALIGN;
  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;

  CombineArgs a = {};
  for (int q = 0; q < d->ranks; ++q) {
    if (q == d->rank || empty) continue;
    if (put) a.ret_out[q] = ret_out[q];
    if (sum) a.ret_in[q] = ret_in[q];
  }
  a.y = y;
  a.recv_count = recv_count;
  a.topk = topk_idx;
  a.gates = gates;
  a.out = out;
  a.out_flags = out_flags;
  a.in_flags = in_flags;
  a.err = static_cast<ErrRec*>(workspace);
  a.counters = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + OVL_ERROR_RECORD_BYTES);
  a.pos = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + 256);
  a.tokens = d->tokens;
  a.n = d->n;
  a.cap = cap;
  a.flag_stride = d->flag_stride / 8;
  a.epoch = epoch;
  a.spin_limit = spin_limit_of(opts);
  a.ranks = d->ranks;
  a.rank = d->rank;
  a.topk_n = d->topk;
  a.experts = d->experts_per_rank;
  a.do_put = put && peers;  // with no tokens no slice has rows, and every out flag is set at once
  a.do_sum = sum && !empty;
  a.wait_in = mode == OVL_MODE_FUSED && peers;

  if (put && peers) {
    st = epoch_accept(out_flags, epoch);
    if (st) return st;
  }
  hipLaunchKernelGGL(combine_layout_kernel, dim3(d->ranks * d->experts_per_rank), dim3(kCbLayoutThreads), 0, stream, a);
  OVL_HIP_TRY(hipGetLastError());
  // Two workgroups per compute unit (the put's grid stride and the final
  // arrival count both use this number).
  const int blocks = kCbBlocksPerCu * di.cus;
  if (d->topk <= 2)
    hipLaunchKernelGGL(combine_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<8>, dim3(blocks), dim3(kThreads), 0, stream, a);
  OVL_HIP_TRY(hipGetLastError());
  return OVL_OK;
}
