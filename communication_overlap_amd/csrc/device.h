// Device-side building blocks shared by the overlap kernels: vector types,
// the error record, the flag wait (acquire) and the flag publish (release).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ovl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes per workgroup

// Device error record at the start of every workspace (OVL_ERROR_RECORD_BYTES).
struct ErrRec {
  int32_t status;    // 0 or an ovl_status
  int32_t site;      // which wait gave up
  int64_t index;     // flag slot index
  int64_t observed;  // last value read
  int64_t expected;  // value awaited
  int64_t pad[4];
};
static_assert(sizeof(ErrRec) == 64, "error record size");

enum : int32_t {
  kSiteAgUnit = 1, kSiteAgBarrier = 2, kSiteRsIn = 3, kSiteA2aSlice = 4, kSiteRsOwn = 5, kSiteAgSplit = 6,
  kSiteCbIn = 7, kSiteRing = 8, kSiteA2aCap = 9
};

__device__ inline void report_error(ErrRec* e, int32_t code, int32_t site, int64_t index,
                                    int64_t observed, int64_t expected) {
  if (atomicCAS(&e->status, 0, code) == 0) {
    e->site = site;
    e->index = index;
    e->observed = observed;
    e->expected = expected;
  }
}

__device__ inline int lane_id() { return threadIdx.x & 63; }

// The constant-rate (100 MHz) real-time counter, common to all compute units.
__device__ inline int64_t now_ticks() { return (int64_t)__builtin_amdgcn_s_memrealtime(); }
// The shader-clock cycle counter (its rate is the actual clock).
__device__ inline int64_t now_cycles() { return (int64_t)__builtin_amdgcn_s_memtime(); }

// A flag above the awaited epoch breaks the epoch rule (epochs increase from
// run to run, and a producer stores exactly the run's epoch): the slot holds
// a signal of a later run, or the caller awaits a stale epoch.  The wait
// still counts the flag as set (the predicate is flag >= epoch, the pages'
// ge wait), so nothing blocks, but the run reports OVL_EEPOCH with the slot
// and the value seen: a consumer may have read data its producer had not
// written yet.  Any lane may call this with its own value.
__device__ inline void check_epoch(ErrRec* e, int32_t site, int64_t index, int64_t v, int64_t epoch) {
  if (v > epoch) report_error(e, -4 /* OVL_EEPOCH */, site, index, v, epoch);
}

// A value every lane of the workgroup holds alike (read from LDS after a
// barrier, or from a broadcast), made a scalar.  Loop bounds and branches
// that enclose workgroup barriers must be uniform to the compiler, not only
// in fact: a loop whose exit it takes for divergent may be restructured so
// that lanes leave it separately, splitting one barrier into several.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// The same for a 64-bit value.
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Work item of consumer (x, q) (die x, index q on its die) in round w of a
// persistent deal over `groups` dies of `per` consumers: a whole round gives
// die x the `per` consecutive items from x * per (consecutive items share A
// rows or B columns, and a die shares one L2); the last, partial round gives
// every die an even share of consecutive items.  Dealt in whole die shares,
// a partial round loaded some dies fully and left others idle: the
// 8192 x 3584 x 4096 GEMM alone ran 234 us against 213 us with its second
// round spread over all dies.  Returns -1 past the consumer's last item.
__device__ inline int64_t deal_item(int64_t w, int x, int q, int groups, int per, int64_t items) {
  const int64_t cn = (int64_t)groups * per, base = w * cn;
  if (base >= items) return -1;
  const int64_t rem = items - base;
  if (rem >= cn) return base + (int64_t)x * per + q;
  const int64_t share = (rem + groups - 1) / groups;
  const int64_t j = base + (int64_t)x * share + q;
  return (q < share && j < items) ? j : -1;
}

// Wave-level poll: every lane of the calling wavefront polls `flag` (one
// load per poll, uniform address) with relaxed agent-scope loads until it
// holds a value >= epoch.  Returns false (after recording OVL_ETIMEOUT) if
// spin_limit polls pass.  The caller follows one or more polls with
// wave_acquire() before it reads what the flags guard.
__device__ inline bool wave_poll(const int64_t* flag, int64_t epoch, uint64_t spin_limit,
                                 ErrRec* err, int32_t site, int64_t index) {
  int64_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t polls = 0;
  while (__builtin_amdgcn_readfirstlane((int)(v < epoch))) {
    if (++polls > spin_limit) {
      if (lane_id() == 0) report_error(err, -6 /* OVL_ETIMEOUT */, site, index, v, epoch);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
    v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane_id() == 0) check_epoch(err, site, index, v, epoch);
  return true;
}

// Agent-scope acquire fence: every load the wave issues afterwards sees what
// the producers released before the flag values its polls observed.
__device__ inline void wave_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Wave-level acquire wait on one flag: wave_poll, then wave_acquire.
__device__ inline bool wave_wait(const int64_t* flag, int64_t epoch, uint64_t spin_limit,
                                 ErrRec* err, int32_t site, int64_t index) {
  const bool ok = wave_poll(flag, epoch, spin_limit, err, site, index);
  wave_acquire();
  return ok;
}

// Waits until this wave's outstanding memory operations have completed
// (stores included: they have reached the L2 of this die).
__device__ inline void wave_drain() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // The same wait as a builtin, which the compiler's own wait insertion
  // reads (it does not read inline asm): it then knows no load is pending
  // here, and adds no wait for one later, e.g. at the top of every K-step of
  // a GEMM that follows a copy.  vmcnt(0), expcnt(7), lgkmcnt(15).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup-level publish: every thread calls this after its own stores of
// the unit.  Each wave drains its stores, the workgroup barrier orders all of
// them before thread 0, and thread 0 issues one agent-scope release fence
// (which writes this die's L2 back, so that the other dies see the data)
// followed by the flag store.  One writeback per unit rather than one per
// wave keeps the release cheap; the barrier carries the other waves' stores
// into thread 0's release (scope inclusion: workgroup scope, then agent).
__device__ inline void wg_publish(int64_t* flag, int64_t epoch) {
  wave_drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroup-level arrival on a counter, with the same release as
// wg_publish; thread 0 adds n and returns the value it observed before the
// add (only thread 0's value is meaningful).
__device__ inline int64_t wg_arrive(int64_t* counter, int64_t n = 1) {
  wave_drain();
  __syncthreads();
  int64_t old = 0;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    old = __hip_atomic_fetch_add(counter, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return old;
}

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Nontemporal 16-byte load, for data read once: a lone workgroup copies
// from HBM faster with it (measured 24 against 20 GB/s cold), though slower
// when the source sits in the last-level cache.
__device__ inline u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Stores for data that workgroups on other dies read after a flag.  An
// agent-scope store (a relaxed atomic store at agent scope: the sc1 bit) is
// complete at the device's point of coherence once it drains, so a workgroup
// that wrote a unit only with these publishes it with a drain and a barrier
// (wg_arrive_agent) and skips the agent-scope release fence, whose L2
// writeback of the die was measured at about 0.5 us, serialised per die.
// Lanes take consecutive 8-byte words, so one store covers 512 contiguous
// bytes per wave.
__device__ inline void st8_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wg_arrive for a unit written only with st8_agent: every wave drains its
// stores, the barrier orders them before thread 0's add, and no L2
// writeback is needed.  Returns the value before the add (thread 0 only).
__device__ inline int64_t wg_arrive_agent(int64_t* counter) {
  wave_drain();
  __syncthreads();
  int64_t old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(counter, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

}  // namespace ovl
