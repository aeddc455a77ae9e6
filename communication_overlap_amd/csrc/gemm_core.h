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
// Global traffic goes through buffer resources whose size ends exactly at
// the tile's last valid row: loads past it return zero and stores past it
// are dropped by the hardware, so ragged M and K tails cost no branches;
// columns past N get an out-of-range offset once per tile.
//
// Accumulation order of every output element is fixed: K ascending in steps
// of 16 (one MFMA each), whatever the order tiles or flags arrive in.
#pragma once

#include "device.h"

namespace ovl {

constexpr int kBK = 64;        // K per pipeline stage
constexpr int kKP = kBK + 8;   // LDS row pitch in bf16 elements
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer (operands are < 2 GiB)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes); bytes is clamped to [0, 2^31 - 1].
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ inline u32x4 bload128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ inline u32x2 bload64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ inline uint32_t bload32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ inline float bloadf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ inline void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}

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

template <int BV>
__device__ inline BRow<BV> load_brow(rsrc_t r, uint32_t off);
template <>
__device__ inline BRow<8> load_brow<8>(rsrc_t r, uint32_t off) { return {bload128(r, off)}; }
template <>
__device__ inline BRow<4> load_brow<4>(rsrc_t r, uint32_t off) { return {bload64(r, off)}; }
template <>
__device__ inline BRow<2> load_brow<2>(rsrc_t r, uint32_t off) { return {bload32(r, off)}; }

template <int BV>
__device__ inline uint32_t brow_word(const BRow<BV>& r, int w);
template <>
__device__ inline uint32_t brow_word<8>(const BRow<8>& r, int w) { return r.d[w]; }
template <>
__device__ inline uint32_t brow_word<4>(const BRow<4>& r, int w) { return r.d[w]; }
template <>
__device__ inline uint32_t brow_word<2>(const BRow<2>& r, int) { return r.d; }

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

// Per-tile, per-lane addressing of the global loads.
template <int BM, int BN>
struct TileAddr {
  rsrc_t ra, rb;
  uint32_t a_off;   // this lane's A offset at k0 = 0 for vector v = 0 (bytes)
  uint32_t a_vstep; // bytes between the rows of consecutive A vectors (32 rows)
  uint32_t b_off;   // this lane's B offset at k0 = 0, or kOOB for columns past N
  uint32_t ldb_b;   // B row pitch in bytes
  int32_t k;
  int32_t kchunk;   // this lane's K offset within a stage (elements)
};

template <int BM, int BN>
__device__ inline TileAddr<BM, BN> tile_addr(const Operands& op, int64_t m0) {
  using C = TileCfg<BM, BN>;
  TileAddr<BM, BN> t;
  const int tid = threadIdx.x;
  t.ra = make_rsrc(op.a + m0 * op.lda, (op.m_valid - m0) * op.lda * 2);
  t.rb = make_rsrc(op.b + op.n0, op.k * op.ldb * 2 - op.n0 * 2);
  t.kchunk = (tid & 7) * 8;
  t.a_off = (uint32_t)(((tid >> 3) * op.lda + t.kchunk) * 2);
  t.a_vstep = (uint32_t)(32 * op.lda * 2);
  const int kb = (tid & 7) * 8;
  const int nb = (tid >> 3) * C::BV;
  t.ldb_b = (uint32_t)(op.ldb * 2);
  t.b_off = (op.n0 + nb < op.n_valid) ? (uint32_t)(kb * op.ldb * 2 + nb * 2) : kOOB;
  t.k = (int32_t)op.k;
  return t;
}

// Global -> registers for the K-step starting at k0.
template <int BM, int BN>
__device__ inline void stage_load(Stage<BM, BN>& st, const TileAddr<BM, BN>& t, int32_t k0) {
  using C = TileCfg<BM, BN>;
  const uint32_t abase = (k0 + t.kchunk < t.k) ? t.a_off + (uint32_t)k0 * 2 : kOOB;
#pragma unroll
  for (int v = 0; v < C::AV; ++v) st.a[v] = bload128(t.ra, abase + v * t.a_vstep);
  const uint32_t bbase = t.b_off + (uint32_t)k0 * t.ldb_b;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.b[i] = load_brow<C::BV>(t.rb, bbase + i * t.ldb_b);
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

template <int BM, int BN>
struct Frags {
  bf16x8 a[TileCfg<BM, BN>::FM];
  bf16x8 b[TileCfg<BM, BN>::FN];
};

template <int BM, int BN>
__device__ inline void load_frags(Frags<BM, BN>& f, const uint16_t* la, const uint16_t* lb, int kk) {
  using C = TileCfg<BM, BN>;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    f.a[fm] = *reinterpret_cast<const bf16x8*>(la + fm * 32 * kKP + kk * 16);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
    f.b[fn] = *reinterpret_cast<const bf16x8*>(lb + fn * 32 * kKP + kk * 16);
}

template <int BM, int BN>
__device__ inline void mfma_frags(Acc<BM, BN>& acc, const Frags<BM, BN>& f) {
  using C = TileCfg<BM, BN>;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fm], f.b[fn], acc.v[fm][fn], 0, 0, 0);
}

// Keeps the compiler from treating x as loop-invariant (the value is
// unchanged), so that address arithmetic built on it is not hoisted out of
// the persistent tile loop and kept live in hundreds of registers.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

#define OVL_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// MFMA over one LDS stage (4 sub-steps of K=16), fragments double-buffered
// so that the LDS reads of sub-step kk+1 are in flight during the MFMAs of
// kk.  The scheduling fences keep that pipeline shape.  When `next` is not
// null, the next stage's registers are written to it during the last
// sub-step, under the MFMAs.
template <int BM, int BN>
__device__ inline void stage_compute(Acc<BM, BN>& acc, const uint16_t* lds_stage, const Stage<BM, BN>* st,
                                     uint16_t* next) {
  using C = TileCfg<BM, BN>;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (BM / 2);
  const int wn = (wave & 1) * (BN / 2);
  const uint16_t* la = lds_stage + (wm + (lane & 31)) * kKP + (lane >> 5) * 8;
  const uint16_t* lb = lds_stage + C::A_ELEMS + (wn + (lane & 31)) * kKP + (lane >> 5) * 8;
  Frags<BM, BN> f0, f1;
  load_frags(f0, la, lb, 0);
  OVL_SCHED_FENCE();
  load_frags(f1, la, lb, 1);
  mfma_frags(acc, f0);
  OVL_SCHED_FENCE();
  load_frags(f0, la, lb, 2);
  mfma_frags(acc, f1);
  OVL_SCHED_FENCE();
  load_frags(f1, la, lb, 3);
  mfma_frags(acc, f0);
  if (next) stage_store(*st, next);
  OVL_SCHED_FENCE();
  mfma_frags(acc, f1);
  OVL_SCHED_FENCE();
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
  const TileAddr<BM, BN> ta = tile_addr<BM, BN>(op, m0);
  const int32_t steps = (int32_t)((op.k + kBK - 1) / kBK);
  Stage<BM, BN> st;
  before_step(0);
  stage_load(st, ta, 0);
  stage_store(st, lds);
  __syncthreads();
  for (int32_t s = 0; s < steps; ++s) {
    const bool more = s + 1 < steps;
    if (more) {
      before_step((int64_t)(s + 1) * kBK);
      stage_load(st, ta, (s + 1) * kBK);
    }
    stage_compute(acc, lds + (s & 1) * C::STAGE_ELEMS, &st, more ? lds + ((s + 1) & 1) * C::STAGE_ELEMS : nullptr);
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

// fp32 output view of one tile of a row-major matrix with pitch ldc: the
// resource spans rows [0, m_valid) of the whole matrix, so rows past the
// last are dropped by the hardware; the tile origin is folded into the
// per-lane offset, and columns past n_valid get kOOB.
struct OutTile {
  rsrc_t r;
  uint32_t ldc_b;   // row pitch in bytes (opaque to loop-invariant motion)
  uint32_t base;    // byte offset of the tile origin
  int64_t n_left;   // columns that exist from the tile origin on
};

__device__ inline OutTile out_tile(float* c, int64_t ldc, int64_t m0, int64_t n0, int64_t m_valid,
                                   int64_t n_valid) {
  OutTile o;
  o.r = make_rsrc(c, m_valid * ldc * 4);
  o.ldc_b = opaque((uint32_t)(ldc * 4));
  o.base = (uint32_t)(m0 * ldc * 4 + n0 * 4);
  o.n_left = n_valid - n0;
  return o;
}

// Byte offset of (row, col) of the tile, or kOOB for a column past N.
__device__ inline uint32_t out_off(const OutTile& o, int row, int col) {
  return col < o.n_left ? o.base + (uint32_t)row * o.ldc_b + (uint32_t)col * 4 : kOOB;
}

// Stores the tile to fp32 C (row pitch ldc) at (m0, n0), clipped to m_valid x n_valid.
template <int BM, int BN>
__device__ inline void acc_store(const Acc<BM, BN>& acc, float* c, int64_t ldc, int64_t m0, int64_t n0,
                                 int64_t m_valid, int64_t n_valid) {
  const OutTile o = out_tile(c, ldc, m0, n0, m_valid, n_valid);
  acc_foreach(acc, [&](int row, int col, float v) { bstoref(o.r, out_off(o, row, col), v); });
}

}  // namespace ovl
