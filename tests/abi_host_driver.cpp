// Exercises the host side of every C-ABI entry point without a GPU: plans
// and their tables, size queries, the host mirror of the consumer order,
// argument validation of every *_run call (which refuses before touching a
// device), strerror.  Built with AddressSanitizer and UndefinedBehavior-
// Sanitizer against a library whose host code carries the same sanitizers
// (tests/test_host_sanitizers.py); any report or a wrong answer fails.
//
// Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <random>
#include <vector>

#include "ovl.h"

namespace {

int g_failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                    \
    }                                                                  \
  } while (0)

void* fake(uintptr_t v) { return reinterpret_cast<void*>(v); }  // never dereferenced: refusals come first

void plans(std::mt19937_64& rng) {
  // Random descriptors, valid and not: every accepted plan answers its
  // queries consistently, and its consumer order is a permutation with the
  // own row tiles first.
  for (int it = 0; it < 3000; ++it) {
    ag_gemm_desc d{};
    d.ranks = (int)(rng() % 18);
    d.rank = (int)(rng() % 18) - 1;
    d.shard_m = (int64_t)(rng() % 3000) - 5;
    d.k = 8 * (int64_t)(rng() % 600) + (rng() % 8 == 0 ? 3 : 0);
    d.n = 8 * (int64_t)(rng() % 600);
    d.tile_m = (int)(rng() % 300) - 2;
    d.tile_n = 8 * (int)(rng() % 40);
    d.tiles_per_flag = (int)(rng() % 6) - 1;
    d.flag_stride = 8 * (int)(rng() % 20);
    d.unit_producers = (int)(rng() % 19) - 1;
    ag_gemm_plan_t p = nullptr;
    const ovl_status st = ag_gemm_plan(&d, &p);
    if (st != OVL_OK) {
      EXPECT(p == nullptr);
      EXPECT(st == OVL_EINVAL || st == OVL_ESHAPE || st == OVL_EALIGN || st == OVL_EUNSUPPORTED);
      continue;
    }
    const int64_t units = ag_gemm_num_units(p);
    EXPECT(units >= d.ranks);
    EXPECT(ag_gemm_flags_bytes(p) == (size_t)units * (size_t)d.flag_stride);
    EXPECT(ag_gemm_workspace_bytes(p) >= OVL_ERROR_RECORD_BYTES + (d.unit_producers > 1 ? 8 * (size_t)units : 0));
    EXPECT(ag_gemm_splits(p) >= 1);
    EXPECT(ag_gemm_trace_bytes(p) >= 8 * (size_t)units);
    const int T = ag_gemm_row_tiles(p), bm = ag_gemm_tile_rows(p);
    EXPECT(bm == 128 || bm == 256);
    EXPECT((int64_t)T * bm >= (int64_t)d.ranks * d.shard_m);
    if (units <= (1 << 16)) {
      std::vector<int32_t> order(units), out(T, -1);
      for (int64_t i = 0; i < units; ++i) order[i] = (int32_t)i;
      std::shuffle(order.begin(), order.end(), rng);
      EXPECT(ag_gemm_consumer_order(p, order.data(), out.data()) == OVL_OK);
      std::vector<int> seen(T, 0);
      for (int v : out) {
        EXPECT(v >= 0 && v < T);
        if (v >= 0 && v < T) ++seen[v];
      }
      for (int s : seen) EXPECT(s == 1);
      EXPECT(ag_gemm_consumer_order(p, nullptr, out.data()) == OVL_OK);
      order[units - 1] = (int32_t)units;  // not a unit
      EXPECT(ag_gemm_consumer_order(p, order.data(), out.data()) == OVL_EINVAL);
      // run refusals: null shard table, null workspace, bad mode
      EXPECT(ag_gemm_run(p, nullptr, fake(16), fake(16), (float*)fake(16), (int64_t*)fake(16), fake(16), 1, nullptr,
                         nullptr, nullptr) == OVL_EINVAL);
      ovl_opts o{};
      o.mode = 9;
      std::vector<const void*> sh(d.ranks, fake(16));
      EXPECT(ag_gemm_run(p, sh.data(), fake(16), fake(16), (float*)fake(16), (int64_t*)fake(16), fake(16), 1, nullptr,
                         &o, nullptr) == OVL_EINVAL);
      EXPECT(ag_gemm_run(p, sh.data(), fake(16), fake(20), (float*)fake(16), (int64_t*)fake(16), fake(16), 1, nullptr,
                         nullptr, nullptr) == OVL_EALIGN);
    }
    EXPECT(ag_gemm_plan_destroy(p) == OVL_OK);
  }
  EXPECT(ag_gemm_plan(nullptr, nullptr) == OVL_EINVAL);
  EXPECT(ag_gemm_num_units(nullptr) == 0 && ag_gemm_flags_bytes(nullptr) == 0);
}

void gemm_rs() {
  for (int tm : {128, 256, 64}) {
    gemm_rs_desc d{8, 0, 8192, 4096, 1792, tm, 256, 8};
    std::vector<float*> po(8, (float*)fake(16));
    std::vector<const float*> pi(8, (const float*)fake(16));
    const ovl_status st = gemm_rs_run(&d, fake(16), fake(16), po.data(), pi.data(), (float*)fake(16),
                                      (int64_t*)fake(16), (const int64_t*)fake(16), fake(16), 1, nullptr, nullptr);
    EXPECT(st == (tm == 256 ? OVL_EHIP : OVL_EUNSUPPORTED) || (tm == 256 && st == OVL_OK));
  }
  gemm_rs_desc d{8, 0, 8192, 4096, 1792, 256, 256, 8};
  EXPECT(gemm_rs_flags_bytes(&d) == 8 * 64 * 8);
  EXPECT(gemm_rs_workspace_bytes(&d) == OVL_ERROR_RECORD_BYTES + 8 * 64);
  gemm_rs_desc bad{3, 0, 1000, 256, 256, 256, 256, 8};
  EXPECT(gemm_rs_flags_bytes(&bad) == 0);
  EXPECT(gemm_rs_run(&bad, fake(16), fake(16), nullptr, nullptr, (float*)fake(16), nullptr, nullptr, fake(16), 1,
                     nullptr, nullptr) == OVL_ESHAPE);
}

void dispatch() {
  a2a_desc d{8, 0, 4096, 4096, 1408, 2, 64, 8, 8, 0, 0};
  EXPECT(a2a_flags_bytes(&d) == 64);
  EXPECT(a2a_workspace_bytes(&d) >= OVL_ERROR_RECORD_BYTES);
  EXPECT(a2a_combine_flags_bytes(&d) == 64);
  EXPECT(a2a_combine_workspace_bytes(&d) >= 256);
  a2a_desc t = d;
  t.tile_m = 128;
  t.tile_n = 128;
  EXPECT(a2a_dispatch_grouped_gemm_run(&t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, 1, nullptr, nullptr) == OVL_EUNSUPPORTED);
  EXPECT(a2a_dispatch_grouped_gemm_run(&d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, 1, nullptr, nullptr) == OVL_EINVAL);
  a2a_desc many = d;
  many.ranks = 17;
  many.num_experts = 17 * 8;
  std::vector<const void*> x(17, fake(16));
  std::vector<const int32_t*> tk(17, (const int32_t*)fake(16));
  EXPECT(a2a_dispatch_grouped_gemm_run(&many, x.data(), tk.data(), fake(16), fake(16), (int32_t*)fake(16),
                                       (int32_t*)fake(16), (float*)fake(16), (int64_t*)fake(16), fake(16), 1, nullptr,
                                       nullptr) == OVL_EUNSUPPORTED);
}

void ring_and_misc() {
  ring_desc r{8, 8 << 20, 16 << 10, 8};
  EXPECT(ring_allreduce_flags_bytes(&r) > 0);
  EXPECT(ring_allreduce_workspace_bytes(&r) == 256);
  ring_desc odd{8, 1000, 3, 8};
  EXPECT(ring_allreduce_workspace_bytes(&odd) == 0);
  for (int s = 1; s >= -8; --s) EXPECT(ovl_strerror(s) != nullptr);
  EXPECT(ovl_flags_reset(nullptr, 8, nullptr, 0, nullptr) == OVL_EINVAL);
  EXPECT(ovl_flags_reset((int64_t*)fake(24), 8, nullptr, 0, nullptr) == OVL_EALIGN);
  EXPECT(ovl_copy(fake(16), fake(16), 17, 0, nullptr) == OVL_EALIGN);
  EXPECT(fp8_quantize_rows(nullptr, nullptr, nullptr, 4, 16, nullptr) == OVL_EINVAL);
}

}  // namespace

int main() {
  std::mt19937_64 rng(12345);
  plans(rng);
  gemm_rs();
  dispatch();
  ring_and_misc();
  if (g_failures) {
    std::fprintf(stderr, "%d failed expectations\n", g_failures);
    return 1;
  }
  std::printf("host driver ok\n");
  return 0;
}
