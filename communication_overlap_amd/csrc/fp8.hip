// Per-row FP8 (OCP E4M3) quantization of bf16 rows: the source side of the
// FP8 dispatch (tokens) and the offline form of the FP8 expert weights (rows
// of the transposed weight).  A row x with amax = max |x| gets the float32
// scale amax / 448 and the codes of x * (448 / amax), clamped to +-448 and
// rounded to the nearest code, ties to even (gfx950's conversion
// instruction); a row of zeros gets scale 1 and zero codes.  The Aboleth
// README's MoE measurement runs "one FP8 layer" and fixes nothing more.
#include "device.h"
#include "host.h"

namespace ovl {

namespace {

__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Four float32 values (already within +-448) to four E4M3 codes, byte i
// holding value i.
__device__ inline uint32_t cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// One wave per row, rows strided over the grid's waves; each lane takes 8
// elements (16 bytes) at a time.  Pass 1 finds the row's amax, pass 2 reads
// the row again (from cache) and converts.
__global__ __launch_bounds__(kThreads) void fp8_quantize_kernel(const uint16_t* in, uint8_t* q, float* scale,
                                                                int64_t rows, int64_t cols) {
  const int lane = lane_id();
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t vpr = cols / 8;
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows; r += waves) {
    const u32x4* src = reinterpret_cast<const u32x4*>(in + r * cols);
    float amax = 0.f;
    for (int64_t v = lane; v < vpr; v += 64) {
      const u32x4 x = src[v];
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(x[i])), fabsf(bf16_hi(x[i]))));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    const bool pos = amax > 0.f;
    const float inv = pos ? 448.f / amax : 0.f;
    if (lane == 0) scale[r] = pos ? amax / 448.f : 1.f;
    u32x2* dst = reinterpret_cast<u32x2*>(q + r * cols);
    for (int64_t v = lane; v < vpr; v += 64) {
      const u32x4 x = src[v];
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = fminf(fmaxf(bf16_lo(x[i]) * inv, -448.f), 448.f);
        f[2 * i + 1] = fminf(fmaxf(bf16_hi(x[i]) * inv, -448.f), 448.f);
      }
      u32x2 o;
      o[0] = cvt4(f[0], f[1], f[2], f[3]);
      o[1] = cvt4(f[4], f[5], f[6], f[7]);
      dst[v] = o;
    }
  }
}

}  // namespace

}  // namespace ovl

using namespace ovl;

extern "C" ovl_status fp8_quantize_rows(const void* in, void* q, float* scale, int64_t rows, int64_t cols,
                                        hipStream_t stream) {
  if (rows < 0 || cols < 0) return OVL_EINVAL;
  if (rows == 0) return OVL_OK;
  if (!in || !q || !scale) return OVL_EINVAL;
  if (cols % 16 || !aligned16(in) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scale) & 3u)) return OVL_EALIGN;
  if (cols > (1 << 24) || rows > (1ll << 31)) return OVL_EUNSUPPORTED;
  DeviceInfo di;
  ovl_status st = current_device_info(&di);
  if (st) return st;
  const int64_t wpb = kThreads / 64;
  const int blocks = (int)std::min<int64_t>((int64_t)di.cus * 8, (rows + wpb - 1) / wpb);
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(in), static_cast<uint8_t*>(q), scale, rows, cols);
  OVL_HIP_TRY(hipGetLastError());
  return OVL_OK;
}
