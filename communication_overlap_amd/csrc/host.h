// Host-side helpers shared by the entry points (not part of the C-ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ovl.h"

namespace ovl {

#define OVL_HIP_TRY(expr)                         \
  do {                                            \
    if ((expr) != hipSuccess) return OVL_EHIP;    \
  } while (0)

constexpr uint64_t kDefaultSpinLimit = 1ull << 22;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t aligned_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct DeviceInfo {
  int device;
  int cus;
};

// Current device and its compute-unit count (cached per device).
ovl_status current_device_info(DeviceInfo* out);

// Epoch bookkeeping per flag buffer: OVL_EEPOCH unless epoch >= 1 and
// greater than the last epoch accepted for `flags` since its reset; on
// success records `epoch` as the last one.
ovl_status epoch_accept(const void* flags, int64_t epoch);
ovl_status epoch_check(const void* flags, int64_t epoch);
void epoch_forget(const void* flags);

// Zeroes `bytes` bytes at p (16-byte aligned) on `stream` with a fill kernel
// (not a memset node, so that the work may be captured in a graph).
ovl_status zero_async(void* p, size_t bytes, hipStream_t stream);

// Device address of the current device's scratch array, which the
// allocation-free entry point uses as its workspace (looked up once per
// device, with that device current).
ovl_status noalloc_scratch(void** out);

// Raises the dynamic-LDS limit of `kernel` to `bytes` once per process.
ovl_status allow_lds(const void* kernel, int bytes);

inline uint64_t spin_limit_of(const ovl_opts* o) {
  return (o && o->spin_limit) ? o->spin_limit : kDefaultSpinLimit;
}

}  // namespace ovl
