// bf16 x bf16 -> fp32 tile GEMM on gfx950 matrix cores.
//
// One workgroup of 4 wavefronts computes a BM x BN output tile; the waves
// form a 2 x 2 grid, each owning a (BM/2) x (BN/2) sub-tile made of 32 x 32
// blocks computed with v_mfma_f32_32x32x16_bf16.  K advances in steps of 64
// through a two-stage LDS ring:
//   - A (row-major, K contiguous) is copied to LDS as is, 16 bytes a lane;
//   - B (row-major, N contiguous) is transposed on its way to LDS: each lane
//     loads an 8 (k) x BV (n) block, transposes it in registers and writes
//     BV vectors of 8 consecutive k values, so that both MFMA operands read
//     K-contiguous 16-byte fragments from LDS.
// LDS rows are padded by 16 bytes (pitch 144 B), which spreads the 16-byte
// fragment reads and the staging writes over all banks.
//
// Accumulation order of every output element is fixed: K ascending in steps
// of 16 (one MFMA each), whatever the order tiles or flags arrive in.
#pragma once

#include "device.h"

namespace ovl {

constexpr int kBK = 64;        // K per pipeline stage
constexpr int kKP = kBK + 8;   // LDS row pitch in bf16 elements

template <int BM, int BN>
struct TileCfg {
  static_assert(BM % 64 == 0 && BN % 64 == 0 && BN <= 256 && BM <= 256, "tile shape");
  static constexpr int FM = BM / 64;        // 32-row blocks per wave
  static constexpr int FN = BN / 64;        // 32-col blocks per wave
  static constexpr int AV = BM / 32;        // 16-byte A vectors per thread per stage
  static constexpr int BV = BN / 32;        // B columns per thread per stage (8 k-rows each)
  static constexpr int A_ELEMS = BM * kKP;
  static constexpr int B_ELEMS = BN * kKP;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2;
};

template <int BM, int BN>
struct Acc {
  f32x16 v[TileCfg<BM, BN>::FM][TileCfg<BM, BN>::FN];
};

template <int BV>
struct BRow;
template <>
struct BRow<8> { u32x4 d; };
template <>
struct BRow<4> { u32x2 d; };
template <>
struct BRow<2> { uint32_t d; };

template <int BM, int BN>
struct Stage {
  u32x4 a[TileCfg<BM, BN>::AV];
  BRow<TileCfg<BM, BN>::BV> b[8];
};

// Operand view for one tile: A rows [0, m_valid) at a (row pitch lda),
// B rows [0, k) at b (row pitch ldb), columns [n0, n_valid) of B.
struct Operands {
  const uint16_t* a;
  int64_t lda;
  int64_t m_valid;  // rows of A that exist, counted from a's row 0
  const uint16_t* b;
  int64_t ldb;
  int64_t n0;       // first column of the tile
  int64_t n_valid;  // columns of B that exist
  int64_t k;
};

template <int BV>
__device__ inline BRow<BV> load_brow(const uint16_t* p);
template <>
__device__ inline BRow<8> load_brow<8>(const uint16_t* p) { return {*reinterpret_cast<const u32x4*>(p)}; }
template <>
__device__ inline BRow<4> load_brow<4>(const uint16_t* p) { return {*reinterpret_cast<const u32x2*>(p)}; }
template <>
__device__ inline BRow<2> load_brow<2>(const uint16_t* p) { return {*reinterpret_cast<const uint32_t*>(p)}; }

template <int BV>
__device__ inline uint32_t brow_word(const BRow<BV>& r, int w);
template <>
__device__ inline uint32_t brow_word<8>(const BRow<8>& r, int w) { return r.d[w]; }
template <>
__device__ inline uint32_t brow_word<4>(const BRow<4>& r, int w) { return r.d[w]; }
template <>
__device__ inline uint32_t brow_word<2>(const BRow<2>& r, int w) { return r.d; }

// Global -> registers for the K-step starting at k0 (tile rows start at m0 of A).
template <int BM, int BN>
__device__ inline void stage_load(Stage<BM, BN>& st, const Operands& op, int64_t m0, int64_t k0) {
  using C = TileCfg<BM, BN>;
  const int t = threadIdx.x;
  const int chunk = t & 7;
  const int64_t kc = k0 + chunk * 8;
#pragma unroll
  for (int v = 0; v < C::AV; ++v) {
    const int64_t r = m0 + v * 32 + (t >> 3);
    if (r < op.m_valid && kc < op.k)
      st.a[v] = ld16(op.a + r * op.lda + kc);
    else
      st.a[v] = u32x4{0, 0, 0, 0};
  }
  const int kb = (t & 7) * 8;
  const int64_t n = op.n0 + (t >> 3) * C::BV;
  const bool nvalid = n < op.n_valid;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = k0 + kb + i;
    if (nvalid && k < op.k)
      st.b[i] = load_brow<C::BV>(op.b + k * op.ldb + n);
    else
      st.b[i] = BRow<C::BV>{};
  }
}

// Registers -> LDS stage buffer (B transposed to [n][k]).
template <int BM, int BN>
__device__ inline void stage_store(const Stage<BM, BN>& st, uint16_t* lds_stage) {
  using C = TileCfg<BM, BN>;
  const int t = threadIdx.x;
  uint16_t* la = lds_stage;
  uint16_t* lb = lds_stage + C::A_ELEMS;
  const int chunk = t & 7;
#pragma unroll
  for (int v = 0; v < C::AV; ++v) {
    const int r = v * 32 + (t >> 3);
    st16(la + r * kKP + chunk * 8, st.a[v]);
  }
  const int kb = (t & 7) * 8;
  const int nb = (t >> 3) * C::BV;
#pragma unroll
  for (int j = 0; j < C::BV; ++j) {
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = brow_word<C::BV>(st.b[2 * q], j >> 1);
      const uint32_t hi = brow_word<C::BV>(st.b[2 * q + 1], j >> 1);
      out[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    st16(lb + (nb + j) * kKP + kb, out);
  }
}

// MFMA over one LDS stage (4 sub-steps of K=16).
template <int BM, int BN>
__device__ inline void stage_compute(Acc<BM, BN>& acc, const uint16_t* lds_stage) {
  using C = TileCfg<BM, BN>;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
  const uint16_t* la = lds_stage + (wm + (lane & 31)) * kKP + (lane >> 5) * 8;
  const uint16_t* lb = lds_stage + C::A_ELEMS + (wn + (lane & 31)) * kKP + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      af[fm] = *reinterpret_cast<const bf16x8*>(la + fm * 32 * kKP + kk * 16);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      bfr[fn] = *reinterpret_cast<const bf16x8*>(lb + fn * 32 * kKP + kk * 16);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc.v[fm][fn], 0, 0, 0);
  }
}

template <int BM, int BN>
__device__ inline void acc_zero(Acc<BM, BN>& acc) {
  using C = TileCfg<BM, BN>;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[fm][fn][r] = 0.f;
}

// The K loop of one tile.  before_step(k0) runs before the global loads of
// the K-step at k0 are issued (the consumer's flag wait goes there), in
// every wave.  Ends with a workgroup barrier, so LDS may be reused at once.
template <int BM, int BN, class BeforeStep>
__device__ inline void gemm_tile(Acc<BM, BN>& acc, const Operands& op, int64_t m0, uint16_t* lds,
                                 BeforeStep before_step) {
  using C = TileCfg<BM, BN>;
  acc_zero(acc);
  const int64_t steps = (op.k + kBK - 1) / kBK;
  Stage<BM, BN> st;
  before_step(0);
  stage_load(st, op, m0, 0);
  stage_store(st, lds);
  __syncthreads();
  for (int64_t s = 0; s < steps; ++s) {
    const bool more = s + 1 < steps;
    if (more) {
      before_step((s + 1) * kBK);
      stage_load(st, op, m0, (s + 1) * kBK);
    }
    stage_compute(acc, lds + (s & 1) * C::STAGE_ELEMS);
    if (more) stage_store(st, lds + ((s + 1) & 1) * C::STAGE_ELEMS);
    __syncthreads();
  }
}

// Calls f(row, col, value) for every accumulator element of this lane, with
// row/col relative to the tile origin (32x32 MFMA output layout: lane l holds
// column l%32; register r holds row (r%4) + 8*(r/4) + 4*(l/32)).
template <int BM, int BN, class F>
__device__ inline void acc_foreach(const Acc<BM, BN>& acc, F f) {
  using C = TileCfg<BM, BN>;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm + fm * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
        const int col = wn + fn * 32 + (lane & 31);
        f(row, col, acc.v[fm][fn][r]);
      }
}

// Stores the tile to fp32 C (row pitch ldc) at (m0, n0), clipped to m_valid x n_valid.
template <int BM, int BN>
__device__ inline void acc_store(const Acc<BM, BN>& acc, float* c, int64_t ldc, int64_t m0, int64_t n0,
                                 int64_t m_valid, int64_t n_valid) {
  acc_foreach(acc, [&](int row, int col, float v) {
    const int64_t m = m0 + row, n = n0 + col;
    if (m < m_valid && n < n_valid) c[m * ldc + n] = v;
  });
}

}  // namespace ovl
