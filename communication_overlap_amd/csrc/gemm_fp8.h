// FP8 (OCP E4M3) x FP8 -> fp32 tile GEMM on gfx950 matrix cores.
//
// One workgroup of NW = 4 or 8 wavefronts computes a BM x BN output tile, the
// waves in a 2 x (NW/2) grid of sub-tiles made of 32 x 32 blocks, each
// block a v_mfma_scale_f32_32x32x64_f8f6f4 (both operands E4M3, unit block
// scales) per 64 codes of K.  Both operands are K-major: A as [row][k] codes
// (optionally gathered through a row table), B transposed as [n][k] codes,
// so both travel global -> LDS the same way as the bf16 core's A operand:
// buffer loads that write LDS directly, 128-byte rows of 8 XOR-permuted
// 16-byte chunks (the permutation of the bf16 core's 64-element K step, which
// has the same byte geometry), K steps of 128 codes through 2 LDS stages.
//
// The MFMA sums a lane's 32 codes against the other operand's 32 codes of
// the same lane group, so any map of K onto (lane group, byte) works if both
// operands share it (checked on the device); here lane group g = l / 32 of a
// 64-code sub-step takes codes 32g .. 32g + 31, i.e. logical chunks 2g and
// 2g + 1 of the sub-step's half of the stage row.
//
// Accumulation order of every output element is fixed (K ascending in steps
// of 64, one MFMA each), whatever the order the tiles run in.
#pragma once

#include "gemm_core.h"

namespace ovl {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8BK = 128;  // codes (bytes) of K per LDS stage

// A rows [0, m_valid) at a (row pitch lda bytes), or rows[i] of a row table
// (IND); B^T rows (output columns) [n0, n_valid) at bt (pitch ldb bytes);
// k codes.  k must be a multiple of 16.
struct Operands8 {
  const uint8_t* a;
  int64_t lda;
  int64_t m_valid;
  const int32_t* rows = nullptr;
  const uint8_t* bt;
  int64_t ldb;
  int64_t n0;
  int64_t n_valid;
  int64_t k;
};

template <int BM, int BN, int NW = 4>
struct F8Cfg {
  static_assert(NW == 4 || NW == 8, "waves per workgroup: a 2 x 2 or 2 x 4 grid");
  static constexpr int WN = NW / 2;  // waves along N
  static_assert(BM % 64 == 0 && BN % (32 * WN) == 0, "tile shape");
  static constexpr int FM = BM / 64;
  static constexpr int FN = BN / (32 * WN);
  static constexpr int A_BYTES = BM * kF8BK;
  static constexpr int B_BYTES = BN * kF8BK;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int RPI = 1024 / kF8BK;  // rows per load instruction
  static constexpr int QA = BM / RPI / NW;  // A load instructions per wave per stage
  static constexpr int QB = BN / RPI / NW;
  static_assert(QA % 2 == 0 && QB % 2 == 0, "swizzle parity per instruction");
};

// Chunk permutation of a 128-byte row r (that of the bf16 core's BK = 64).
__device__ inline uint32_t swz8(uint32_t r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BM, int BN, bool IND, int NW>
struct F8Addr {
  u32x4 ra, rb;
  uint32_t a_off[IND ? F8Cfg<BM, BN, NW>::QA : 2];  // IND: per instruction (kOOB: no row); else by parity
  uint32_t a_qstep;
  uint32_t lc[2];     // lane's logical chunk for instructions of parity 0 / 1
  uint32_t b_off[2];  // by parity
  uint32_t b_qstep;
  int32_t k;
};

template <int BM, int BN, bool IND, int NW>
__device__ inline F8Addr<BM, BN, IND, NW> f8_addr(const Operands8& op) {
  using C = F8Cfg<BM, BN, NW>;
  F8Addr<BM, BN, IND, NW> t;
  const uint32_t l = lane_id();
  const uint32_t w = threadIdx.x >> 6;
  t.ra = make_srd(op.a, op.m_valid * op.lda);
  t.rb = make_srd(op.bt + op.n0 * op.ldb, (op.n_valid - op.n0) * op.ldb);
  t.k = (int32_t)op.k;
  const uint32_t lda = (uint32_t)op.lda, ldb = (uint32_t)op.ldb;
  // Instruction iq = w*Q + q fills rows iq*8 .. +7: lane l row iq*8 + l/8,
  // physical chunk l%8 = logical chunk (l%8) ^ swz8(row); swz8 depends on the
  // row through l/8 and the parity of iq (Q even), hence two variants.
  for (uint32_t par = 0; par < 2; ++par) t.lc[par] = (l & 7) ^ ((l >> 3) ^ par);
  if constexpr (IND) {
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
      const uint32_t row = (w * C::QA + q) * C::RPI + (l >> 3);
      const int32_t r = op.rows[row];
      t.a_off[q] = r >= 0 ? (uint32_t)r * lda + t.lc[q & 1] * 16 : kOOB;
    }
  } else {
    for (uint32_t par = 0; par < 2; ++par) t.a_off[par] = ((w * C::QA + par) * C::RPI + (l >> 3)) * lda + t.lc[par] * 16;
  }
  t.a_qstep = C::RPI * lda;
  for (uint32_t par = 0; par < 2; ++par) t.b_off[par] = ((w * C::QB + par) * C::RPI + (l >> 3)) * ldb + t.lc[par] * 16;
  t.b_qstep = C::RPI * ldb;
  return t;
}

template <int BM, int BN, bool IND, int NW>
__device__ inline void f8_issue(const F8Addr<BM, BN, IND, NW>& t, uint32_t stage, int32_t k0) {
  using C = F8Cfg<BM, BN, NW>;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < C::QA; ++q) {
    const int par = q & 1;
    uint32_t off;
    if (k0 + (int32_t)t.lc[par] * 16 >= t.k)
      off = kOOB;
    else if constexpr (IND)
      off = t.a_off[q] + (uint32_t)k0;  // kOOB + k0 is still past every buffer
    else
      off = t.a_off[par] + (q & ~1) * t.a_qstep + (uint32_t)k0;
    load_to_lds(t.ra, stage + (w * C::QA + q) * 1024, off);
  }
#pragma unroll
  for (int q = 0; q < C::QB; ++q) {
    const int par = q & 1;
    const uint32_t off = k0 + (int32_t)t.lc[par] * 16 >= t.k ? kOOB : t.b_off[par] + (q & ~1) * t.b_qstep + (uint32_t)k0;
    load_to_lds(t.rb, stage + C::A_BYTES + (w * C::QB + q) * 1024, off);
  }
}

// 32 codes (two 16-byte chunks) of LDS row `row` for sub-step kk and lane group g.
__device__ inline i32x8 f8_frag(const uint8_t* region, uint32_t row, int kk, uint32_t g) {
  const uint32_t c0 = (4 * kk + 2 * g) ^ swz8(row), c1 = (4 * kk + 2 * g + 1) ^ swz8(row);
  const i32x4 lo = *OVL_LDS(const i32x4, region + row * kF8BK + c0 * 16);
  const i32x4 hi = *OVL_LDS(const i32x4, region + row * kF8BK + c1 * 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int BM, int BN, int NW>
__device__ inline void f8_stage_compute(Acc<BM, BN, NW>& acc, const uint8_t* stage) {
  using C = F8Cfg<BM, BN, NW>;
  const uint32_t l = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t wm = (wave / C::WN) * (BM / 2), wn = (wave % C::WN) * (BN / C::WN);
  const uint32_t g = l >> 5, lr = l & 31;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    i32x8 fa[C::FM], fb[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) fb[fn] = f8_frag(stage + C::A_BYTES, wn + fn * 32 + lr, kk, g);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) fa[fm] = f8_frag(stage, wm + fm * 32 + lr, kk, g);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc.v[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[fm], fb[fn], acc.v[fm][fn], 0, 0, 0, 127,
                                                                        0, 127);
    // One sub-step's fragments live at a time (64 registers): the next
    // sub-step's reads are not hoisted above these MFMAs.
    OVL_SCHED_FENCE();
  }
}

// The K loop of one tile: the next stage's loads are issued at the start of
// a step, before the MFMAs over the current one.  Ends with a workgroup
// barrier, so LDS may be reused at once.
template <int BM, int BN, bool IND = false, int NW = 4>
__device__ inline void gemm_tile_fp8(Acc<BM, BN, NW>& acc, const Operands8& op, uint8_t* lds) {
  using C = F8Cfg<BM, BN, NW>;
  acc_zero(acc);
  const F8Addr<BM, BN, IND, NW> t = f8_addr<BM, BN, IND, NW>(op);
  const int32_t steps = (int32_t)((op.k + kF8BK - 1) / kF8BK);
  const uint32_t lbase = lds_addr(lds);
  __syncthreads();
  if (steps > 0) f8_issue(t, lbase, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int32_t s = 0; s < steps; ++s) {
    if (s + 1 < steps) f8_issue(t, lbase + (uint32_t)((s + 1) & 1) * C::STAGE_BYTES, (s + 1) * kF8BK);
    f8_stage_compute<BM, BN, NW>(acc, lds + (s & 1) * C::STAGE_BYTES);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// Stores the tile through a row table with both scales: tile row i goes to
// row rows[i] of fp32 C (pitch ldc, c_rows rows; nothing where rows[i] < 0)
// as acc * tile_scale[i] * col_scale[n0 + col], columns clipped to n_valid.
// rows and tile_scale are LDS tables of BM entries.
template <int BM, int BN, int NW = 4>
__device__ inline void acc_store_rows_scaled(const Acc<BM, BN, NW>& acc, float* c, int64_t ldc, int64_t c_rows,
                                             const int32_t* rows, const float* tile_scale, const float* col_scale,
                                             int64_t n0, int64_t n_valid) {
  using C = F8Cfg<BM, BN, NW>;
  const rsrc_t r = make_rsrc(c, c_rows * ldc * 4);
  const uint32_t ldc_b = opaque((uint32_t)(ldc * 4));
  const int64_t n_left = n_valid - n0;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = (wave / C::WN) * (BM / 2);
  const int wn = (wave % C::WN) * (BN / C::WN);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      // one 32 x 32 block at a time out of the accumulation registers
      const int col = wn + fn * 32 + (lane & 31);
      // (an unconditional load: a branch here splits the epilogue into blocks
      // and the compiler then copies every accumulator out at its start)
      const float cs = col_scale[n0 + (col < n_left ? col : 0)];
      const f32x16 blk = acc.v[fm][fn];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = wm + fm * 32 + (i & 3) + 8 * (i >> 2) + 4 * (lane >> 5);
        const int32_t cr = rows[row];
        const uint32_t off = (cr >= 0 && col < n_left) ? (uint32_t)cr * ldc_b + (uint32_t)(n0 + col) * 4 : kOOB;
        bstoref(r, off, blk[i] * tile_scale[row] * cs);
      }
      OVL_SCHED_FENCE();
    }
}

}  // namespace ovl
