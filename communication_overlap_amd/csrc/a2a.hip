// All-to-all dispatch of routed tokens followed by a grouped expert GEMM.
#include "device.h"
#include "host.h"

using namespace ovl;

extern "C" size_t a2a_flags_bytes(const a2a_desc* d) {
  if (!d || d->ranks < 1 || d->flag_stride < 8) return 0;
  return (size_t)d->ranks * (size_t)d->flag_stride;
}

extern "C" size_t a2a_workspace_bytes(const a2a_desc* d) { return d ? 256 : 0; }

extern "C" ovl_status a2a_dispatch_grouped_gemm_run(const a2a_desc* d, const void* const* x,
                                                    const int32_t* const* topk_idx, const void* w, void* recv_x,
                                                    int32_t* recv_src, int32_t* recv_count, float* y,
                                                    int64_t* flags, void* workspace, int64_t epoch,
                                                    const ovl_opts* opts, hipStream_t stream) {
  (void)d; (void)x; (void)topk_idx; (void)w; (void)recv_x; (void)recv_src; (void)recv_count; (void)y;
  (void)flags; (void)workspace; (void)epoch; (void)opts; (void)stream;
  return OVL_EUNSUPPORTED;
}
