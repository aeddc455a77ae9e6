// bf16 x bf16 -> fp32 tile GEMM on gfx950 matrix cores.
//
// One workgroup of NW = 4 or 8 wavefronts computes a BM x BN output tile; the
// waves form a 2 x (NW/2) grid, each owning a (BM/2) x (2*BN/NW) sub-tile made
// of 32 x 32 blocks computed with v_mfma_f32_32x32x16_bf16 (8 waves: half the
// accumulators per wave, two waves per SIMD to hide each other's LDS reads).  K advances in steps of BK
// through a ring of NS LDS stages (BK = 32: 4 stages, the loads of a step
// issued three steps ahead; BK = 64: 2 stages, one step ahead).
//
// Both operands travel global -> LDS with buffer loads that write LDS
// directly (16 bytes a lane; lane i of an instruction lands at byte 16*i of
// a 1 KiB LDS block), so staging costs neither registers nor LDS-write
// instructions:
//   - A (row-major, K contiguous) is kept as [row][k] (2*BK bytes per row);
//   - B (row-major, N contiguous) is kept as [k][n] and its MFMA fragments
//     are read with ds_read_b64_tr_b16, which transposes 4 x 4 blocks of
//     16-bit elements across each group of 16 lanes: source lane s of a
//     group points at row s/4, columns 4*(s%4)..+3 of a 4 x 16 block, and
//     lane i receives column i of the block's 4 rows, i.e. 4 consecutive k
//     of one n; two such reads give the 8 consecutive k of one MFMA operand.
// Each LDS row's 16-byte chunks are stored XOR-permuted (the permutation is
// applied when each lane picks the global address it fetches), so that the
// fragment reads hit every bank once.
//
// Global traffic goes through buffer resources whose size ends at the last
// valid row: loads past it return zero, so ragged M and K tails cost no
// branches; chunks past K (for A) or past N (for B) get an out-of-range
// offset.
//
// Accumulation order of every output element is fixed (K ascending in steps
// of 16, one MFMA each), whatever the order tiles or flags arrive in.
#pragma once

#include "device.h"

namespace ovl {

constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer (operands are < 1 GiB)

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define OVL_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Raw buffer resource over [base, base + bytes); bytes is clamped to [0, 2^31 - 1].
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ inline float bloadf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
// Cache-policy operand of a buffer store that makes it an agent-scope store
// (the sc1 bit on gfx950): complete at the device's point of coherence once
// it drains, so data written only with such stores is published by a drain,
// a barrier and a relaxed flag store, with no release fence.
constexpr int kAuxAgent = 16;

template <int AUX = 0>
__device__ inline void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, AUX);
}

// Buffer descriptor as four scalar words, for the inline-asm loads below
// (base address, stride 0, size in bytes, raw-buffer format word).
__device__ inline u32x4 make_srd(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  d.z = __builtin_amdgcn_readfirstlane(n);
  d.w = 0x00020000u;
  return d;
}

// LDS byte address of a pointer into the workgroup's LDS.
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)OVL_LDS(const void, p); }

// 16 bytes per lane from global (buffer offset) straight into LDS at
// lds_block + 16 * lane.  Issued through inline assembly on purpose: the
// compiler cannot tell that these writes go to the other half of the LDS
// ring from the one being read, and would otherwise wait for them before
// the very next LDS read, serialising the prefetch with the MFMAs.  The
// caller waits for them (vmcnt(0)) before the barrier that publishes the
// stage.
__device__ inline void load_to_lds(const u32x4& srd, uint32_t lds_block, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_block), "v"(off), "s"(srd)
               : "memory", "m0");
}

// Chunk permutations.  An A row r of BK bf16 (BK/8 chunks of 16 B):
// physical chunk p holds logical chunk p ^ swz_a<BK>(r).  A B row k (BN/8
// chunks): p holds p ^ swz_b(k).  Each is chosen so that the fragment reads
// (16 consecutive rows at one logical chunk for A; 4 rows x 2 chunks per
// 16-lane group for B) hit distinct banks under 32- and 64-bank LDS layouts.
template <int BK>
__device__ inline uint32_t swz_a(uint32_t r);
template <>
__device__ inline uint32_t swz_a<64>(uint32_t r) { return (r & 7) ^ ((r >> 3) & 1); }
template <>
__device__ inline uint32_t swz_a<32>(uint32_t r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ inline uint32_t swz_b(uint32_t k) { return (0xCA60u >> ((k & 3) * 4)) & 15; }  // 0, 6, 10, 12

// NSTAGES: LDS ring depth (0: 4 for BK 32, 2 for BK 64).  Deeper rings keep
// more loads in flight for bandwidth-bound (skinny) tiles.
template <int BM, int BN, int BK = 64, int NSTAGES = 0, int NW = 4>
struct TileCfg {
  static_assert(BM % 64 == 0 && BN % 128 == 0 && BN <= 256 && BM <= 256, "tile shape");
  static_assert(BK == 32 || BK == 64, "K step");
  static constexpr int NS = NSTAGES ? NSTAGES : (BK == 32 ? 4 : 2);  // LDS stages
  static_assert(NW == 4 || NW == 8, "waves per workgroup: a 2 x 2 or 2 x 4 grid");
  static constexpr int WN = NW / 2;              // waves along N
  static constexpr int FM = BM / 64;             // 32-row blocks per wave
  static constexpr int FN = BN / (32 * WN);      // 32-col blocks per wave
  static constexpr int KK = BK / 16;             // MFMA sub-steps per stage
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static constexpr int A_RPI = 1024 / (BK * 2);  // A rows per load instruction
  static constexpr int QA = BM / A_RPI / NW;     // A load instructions per wave per stage
  static constexpr int B_LPR = BN / 8;           // lanes per B row in one instruction
  static constexpr int B_RPI = 64 / B_LPR;       // B rows per instruction
  static constexpr int QB = BK / B_RPI / NW;     // B load instructions per wave per stage
  static constexpr int LPS = QA + QB;            // load instructions per wave per stage
};

template <int BM, int BN, int NW = 4>
struct Acc {
  f32x16 v[TileCfg<BM, BN, 64, 0, NW>::FM][TileCfg<BM, BN, 64, 0, NW>::FN];
};

// Operand view for one tile: A rows [0, m_valid) at a (row pitch lda),
// B rows [0, k) at b (row pitch ldb), columns [n0, n_valid) of B.  For a
// gathered-rows tile (gemm_tile's IND), `rows` is an LDS table of BM
// entries: tile row i is A row rows[i], or no row (zeros) where rows[i] < 0.
struct Operands {
  const uint16_t* a;
  int64_t lda;
  int64_t m_valid;  // rows of A that exist, counted from a's row 0
  const int32_t* rows = nullptr;
  const uint16_t* b;
  int64_t ldb;
  int64_t n0;       // first column of the tile
  int64_t n_valid;  // columns of B that exist
  int64_t k;
};

// Per-tile, per-lane addressing of the global -> LDS loads.  IND: A rows
// come from a row table, so every A instruction keeps its own offset.
template <int BM, int BN, int BK, bool IND = false, int NW = 4>
struct TileAddr {
  u32x4 ra, rb;
  // Direct: lane offset of A instructions with index parity 0 / 1 at k0 = 0
  // (bytes).  IND: lane offset of each A instruction, or kOOB for no row.
  uint32_t a_off[IND ? TileCfg<BM, BN, BK, 0, NW>::QA : 2];
  uint32_t a_kc[2];    // lane's K column (elements) for A instructions of index parity 0 / 1
  uint32_t a_qstep;    // direct: bytes between consecutive A instructions
  uint32_t b_off[2];   // lane offset of B instructions with index parity 0 / 1 at k0 = 0, or kOOB past N
  uint32_t b_qstep;    // bytes between consecutive B instructions
  uint32_t ldb_b;
  int32_t k;
  uint32_t wl;         // this wave's index among the NW waves that issue the loads
};

// NW here counts the waves that issue the stage loads, and wl is this
// wave's index among them.
template <int BM, int BN, int BK, bool IND = false, int NW = 4>
__device__ inline TileAddr<BM, BN, BK, IND, NW> tile_addr(const Operands& op, int64_t m0,
                                                          uint32_t wl = threadIdx.x >> 6) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  TileAddr<BM, BN, BK, IND, NW> t;
  const uint32_t l = lane_id();
  const uint32_t w = wl;
  t.wl = wl;
  t.ra = make_srd(op.a + m0 * op.lda, (op.m_valid - m0) * op.lda * 2);
  t.rb = make_srd(op.b + op.n0, op.k * op.ldb * 2 - op.n0 * 2);
  t.k = (int32_t)op.k;
  // A: instruction iq = w*QA + q covers tile rows iq*A_RPI .. +A_RPI-1; lane
  // l fills row iq*A_RPI + l/CPR, physical chunk l%CPR (CPR = BK/8 chunks).
  constexpr uint32_t CPR = BK / 8;
  const uint32_t lda_b = (uint32_t)(op.lda * 2);
  for (uint32_t par = 0; par < 2; ++par) {
    const uint32_t row = (w * C::QA + par) * C::A_RPI + l / CPR;
    const uint32_t lc = (l % CPR) ^ swz_a<BK>(row);
    t.a_kc[par] = lc * 8;
    if constexpr (!IND) t.a_off[par] = row * lda_b + lc * 16;
  }
  t.a_qstep = C::A_RPI * lda_b;
  if constexpr (IND) {
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
      const uint32_t row = (w * C::QA + q) * C::A_RPI + l / CPR;
      const int32_t r = op.rows[row];
      t.a_off[q] = r >= 0 ? (uint32_t)r * lda_b + (t.a_kc[q & 1] / 8) * 16 : kOOB;
    }
  }
  // B: instruction iq = w*QB + q covers k rows iq*B_RPI .. +B_RPI-1; lane l
  // fills row iq*B_RPI + l/LPR, physical chunk l%LPR.
  t.ldb_b = (uint32_t)(op.ldb * 2);
  for (uint32_t par = 0; par < 2; ++par) {
    const uint32_t row = (w * C::QB + par) * C::B_RPI + l / C::B_LPR;
    const uint32_t lc = (l % C::B_LPR) ^ swz_b(row);
    const bool nvalid = op.n0 + (int64_t)lc * 8 < op.n_valid;
    t.b_off[par] = nvalid ? row * t.ldb_b + lc * 16 : kOOB;
  }
  t.b_qstep = (uint32_t)(C::B_RPI * t.ldb_b);
  return t;
}

// Buffer offset of A instruction q of the K-step at k0 (kOOB past K, or for
// a row the table leaves out: kOOB + 2 * k0 is still past every buffer).
template <int BM, int BN, int BK, bool IND, int NW>
__device__ inline uint32_t a_offset(const TileAddr<BM, BN, BK, IND, NW>& t, int q, int32_t k0) {
  const int par = q & 1;
  if (k0 + (int32_t)t.a_kc[par] >= t.k) return kOOB;
  if constexpr (IND)
    return t.a_off[q] + (uint32_t)k0 * 2;
  else
    return t.a_off[par] + (q & ~1) * t.a_qstep + (uint32_t)k0 * 2;
}

// Issues this wave's share of the global -> LDS loads of the K-step at k0:
// the A part and the B part separately, so that each can sit under MFMAs.
// The swizzle of an instruction's rows depends on the instruction index only
// through its parity (even QA / QB and row counts), hence the two variants.
template <int BM, int BN, int BK, bool IND, int NW>
__device__ inline void stage_issue_a(const TileAddr<BM, BN, BK, IND, NW>& t, uint32_t stage, int32_t k0) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  const uint32_t w = __builtin_amdgcn_readfirstlane(t.wl);
#pragma unroll
  for (int q = 0; q < C::QA; ++q) load_to_lds(t.ra, stage + (w * C::QA + q) * 1024, a_offset(t, q, k0));
}

template <int BM, int BN, int BK, bool IND, int NW>
__device__ inline void stage_issue_b(const TileAddr<BM, BN, BK, IND, NW>& t, uint32_t stage, int32_t k0) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  const uint32_t w = __builtin_amdgcn_readfirstlane(t.wl);
  const uint32_t sb = stage + C::A_BYTES;
  const uint32_t kb = (uint32_t)k0 * t.ldb_b;
#pragma unroll
  for (int q = 0; q < C::QB; ++q) {
    const int par = q & 1;
    load_to_lds(t.rb, sb + (w * C::QB + q) * 1024, t.b_off[par] + (q & ~1) * t.b_qstep + kb);
  }
}

// One load instruction of a stage: q < QA is A instruction q, otherwise B
// instruction q - QA.
template <int BM, int BN, int BK, bool IND, int NW, int Q>
__device__ inline void stage_issue_one(const TileAddr<BM, BN, BK, IND, NW>& t, uint32_t stage, int32_t k0) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  const uint32_t w = __builtin_amdgcn_readfirstlane(t.wl);
  if constexpr (Q < C::QA) {
    load_to_lds(t.ra, stage + (w * C::QA + Q) * 1024, a_offset(t, Q, k0));
  } else {
    constexpr int q = Q - C::QA, par = q & 1;
    load_to_lds(t.rb, stage + C::A_BYTES + (w * C::QB + q) * 1024,
                t.b_off[par] + (q & ~1) * t.b_qstep + (uint32_t)k0 * t.ldb_b);
  }
}

// The loads of one stage, to be spread over the MFMA groups of the step
// before (on == false: nothing to load).
template <int BM, int BN, int BK, bool IND, int NW>
struct Prefetch {
  static constexpr int QA = TileCfg<BM, BN, BK, 0, NW>::QA;    // A loads per loading wave
  static constexpr int LPS = TileCfg<BM, BN, BK, 0, NW>::LPS;  // loads per loading wave
  const TileAddr<BM, BN, BK, IND, NW>* t;
  uint32_t slot;
  int32_t k0;
  bool on;
  template <int Q>
  __device__ inline void issue() const {
    if (on) stage_issue_one<BM, BN, BK, IND, NW, Q>(*t, slot, k0);
  }
};

// Per-lane LDS read offsets (bytes, within a stage) of the MFMA fragments.
template <int BM, int BN, int BK, int NW>
struct FragAddr {
  uint32_t a[BK / 16];               // A fragment of sub-step kk (add fm * 32 rows)
  uint32_t b[TileCfg<BM, BN, BK, 0, NW>::FN];  // B: row (h*8 + s/4), chunk for block fn (add kk*16 rows)
};

template <int BM, int BN, int BK, int NW>
__device__ inline FragAddr<BM, BN, BK, NW> frag_addr() {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  FragAddr<BM, BN, BK, NW> f;
  const uint32_t l = lane_id();
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t wm = (wave / C::WN) * (BM / 2);
  const uint32_t wn = (wave % C::WN) * (BN / C::WN);
  // A: row wm + fm*32 + l%32, logical chunk 2*kk + l/32 (the swizzle of a
  // row depends on it modulo 16 only, so fm*32 does not change it).
  const uint32_t row = wm + (l & 31);
  for (int kk = 0; kk < C::KK; ++kk) f.a[kk] = row * (BK * 2) + (((2 * kk) | (l >> 5)) ^ swz_a<BK>(row)) * 16;
  // B: group g = l/16 (h = g/2), source lane s = l%16 points at row
  // kk*16 + h*8 + s/4 (+4 for the second read), columns
  // wn + fn*32 + (g%2)*16 + 4*(s%4) .. +3.
  const uint32_t g = l >> 4, s = l & 15;
  const uint32_t brow = (g >> 1) * 8 + (s >> 2);
  for (int fn = 0; fn < C::FN; ++fn) {
    const uint32_t col = wn + fn * 32 + (g & 1) * 16 + 4 * (s & 3);
    const uint32_t chunk = (col >> 3) ^ swz_b(brow);
    f.b[fn] = C::A_BYTES + brow * (BN * 2) + chunk * 16 + (col & 4) * 2;
  }
  return f;
}

// MFMA operands of one sub-step: A fragments, and B fragments as the two
// 4-element halves that two transposing LDS reads produce.
template <int BM, int BN, int NW>
struct Frags {
  bf16x8 a[TileCfg<BM, BN, 64, 0, NW>::FM];
  s16x4 blo[TileCfg<BM, BN, 64, 0, NW>::FN];
  s16x4 bhi[TileCfg<BM, BN, 64, 0, NW>::FN];
};

template <int BM, int BN, int NW>
__device__ inline bf16x8 bfrag(const Frags<BM, BN, NW>& f, int fn) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(f.blo[fn], f.bhi[fn], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Read R of the fragments of sub-step kk, in the order the next sub-step
// needs them: the low and high halves of each B fragment first (the first
// MFMA group uses them all), then A fragment R - 2*FN.
template <int BM, int BN, int BK, int NW, int R>
__device__ inline void load_piece(Frags<BM, BN, NW>& f, const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa,
                                  int kk) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  if constexpr (R >= 2 * C::FN) {
    constexpr int fm = R - 2 * C::FN;
    f.a[fm] = *OVL_LDS(const bf16x8, stage + fa.a[kk] + fm * 32 * (BK * 2));
  } else {
    constexpr int fn = R / 2;
    constexpr int hi = R & 1;
    const uint8_t* p = stage + fa.b[fn] + kk * 16 * (BN * 2) + hi * 4 * (BN * 2);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(OVL_LDS(s16x4, p));
    if (hi)
      f.bhi[fn] = v;
    else
      f.blo[fn] = v;
  }
}

template <int BM, int BN, int BK, int NW, int R0, int R1>
__device__ inline void load_pieces(Frags<BM, BN, NW>& f, const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa,
                                   int kk) {
  if constexpr (R0 < R1) {
    load_piece<BM, BN, BK, NW, R0>(f, stage, fa, kk);
    load_pieces<BM, BN, BK, NW, R0 + 1, R1>(f, stage, fa, kk);
  }
}

template <int BM, int BN, int BK, int NW>
__device__ inline void load_frags(Frags<BM, BN, NW>& f, const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa,
                                  int kk) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  load_pieces<BM, BN, BK, NW, 0, C::FM + 2 * C::FN>(f, stage, fa, kk);
}

template <int BM, int BN, int NW>
__device__ inline void mfma_frags(Acc<BM, BN, NW>& acc, const Frags<BM, BN, NW>& f) {
  using C = TileCfg<BM, BN, 64, 0, NW>;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fm], bfrag(f, fn), acc.v[fm][fn], 0, 0, 0);
}

// Keeps the compiler from treating x as loop-invariant (the value is
// unchanged), so that address arithmetic built on it is not hoisted out of
// the persistent tile loop and kept live in hundreds of registers.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

#define OVL_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Inside one scheduling region: alternate one MFMA with one LDS read, n
// times, then let the remaining MFMAs follow.
template <int N>
__device__ inline void interleave_mfma_ds_read() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
}

// Issues loads [Q0, Q1) of the prefetch, in order.
template <int Q0, int Q1, class P>
__device__ inline void issue_range(const P& p) {
  if constexpr (Q0 < Q1) {
    p.template issue<Q0>();
    issue_range<Q0 + 1, Q1>(p);
  }
}

// One MFMA group (the FN blocks of A-fragment row fm = G % FM) of sub-step
// KKI, on fragments `cur`, with this group's share of the next sub-step's
// fragment reads into `nxt` interleaved (one read after each MFMA), followed
// by a burst of a later stage's global loads where it is due.
template <int BM, int BN, int BK, int NW, int KKI, int G, class P>
__device__ inline void mfma_group(Acc<BM, BN, NW>& acc, const Frags<BM, BN, NW>& cur, Frags<BM, BN, NW>& nxt,
                                  const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa, const P& pf) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  constexpr int fm = G % C::FM;
  constexpr int reads = C::FM + 2 * C::FN;  // fragment reads per sub-step
  constexpr int per = (reads + C::FM - 1) / C::FM;
  constexpr int r0 = fm * per < reads ? fm * per : reads;
  constexpr int r1 = (fm + 1) * per < reads ? (fm + 1) * per : reads;
  constexpr int rd = KKI + 1 < C::KK ? r1 - r0 : 0;
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
    acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[fm], bfrag(cur, fn), acc.v[fm][fn], 0, 0, 0);
  if constexpr (KKI + 1 < C::KK) load_pieces<BM, BN, BK, NW, r0, r1>(nxt, stage, fa, KKI + 1);
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (i < rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  OVL_SCHED_FENCE();
  // The next stage's loads go in two bursts: B after the first MFMA group
  // of the step, A after the first group of the second sub-step.  (Measured
  // on the 8-wave 256 x 256 tile: 4% faster than bursts in mid-step, which
  // left the B loads half a step to land; a 4-stage ring of 32-wide K steps,
  // with three steps of lookahead, was no faster.)
  if constexpr (G == 0) issue_range<P::QA, P::LPS>(pf);
  if constexpr (G == C::FM) issue_range<0, P::QA>(pf);
  OVL_SCHED_FENCE();
}

template <int BM, int BN, int BK, int NW, int KKI, int G0, int N, class P>
__device__ inline void mfma_groups(Acc<BM, BN, NW>& acc, const Frags<BM, BN, NW>& cur, Frags<BM, BN, NW>& nxt,
                                   const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa, const P& pf) {
  if constexpr (N > 0) {
    mfma_group<BM, BN, BK, NW, KKI, G0>(acc, cur, nxt, stage, fa, pf);
    mfma_groups<BM, BN, BK, NW, KKI, G0 + 1, N - 1>(acc, cur, nxt, stage, fa, pf);
  }
}

// MFMA over one LDS stage (BK/16 sub-steps of K = 16), fragments
// double-buffered so that the LDS reads of sub-step kk+1 are in flight
// during the MFMAs of kk (one read after each MFMA), with the global -> LDS
// loads of a later stage in two bursts in mid-step.
template <int BM, int BN, int BK, int NW, class P>
__device__ inline void stage_compute(Acc<BM, BN, NW>& acc, const uint8_t* stage, const FragAddr<BM, BN, BK, NW>& fa,
                                     const P& pf) {
  using C = TileCfg<BM, BN, BK, 0, NW>;
  Frags<BM, BN, NW> f0, f1;
  load_frags(f0, stage, fa, 0);
  OVL_SCHED_FENCE();
  mfma_groups<BM, BN, BK, NW, 0, 0, C::FM>(acc, f0, f1, stage, fa, pf);
  if constexpr (C::KK == 4) {
    mfma_groups<BM, BN, BK, NW, 1, C::FM, C::FM>(acc, f1, f0, stage, fa, pf);
    mfma_groups<BM, BN, BK, NW, 2, 2 * C::FM, C::FM>(acc, f0, f1, stage, fa, pf);
    mfma_groups<BM, BN, BK, NW, 3, 3 * C::FM, C::FM>(acc, f1, f0, stage, fa, pf);
  } else {
    mfma_groups<BM, BN, BK, NW, 1, C::FM, C::FM>(acc, f1, f0, stage, fa, pf);
  }
}

// Waits until at most `pending_stages` stages' worth of this wave's
// asm-issued stage loads are in flight (LPS loads per stage; at most
// MAXP stages, and MAXP * LPS fits the 6-bit load counter).
template <int LPS, int P>
__device__ inline void wait_pending(int pending_stages) {
  if constexpr (P == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (pending_stages >= P)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(P * LPS) : "memory");
    else
      wait_pending<LPS, P - 1>(pending_stages);
  }
}

template <int LPS, int MAXP = 2>
__device__ inline void wait_stage_loads(int pending_stages) {
  static_assert(MAXP * LPS <= 63, "the load counter holds 63 loads");
  wait_pending<LPS, MAXP>(pending_stages);
}

template <int BM, int BN, int NW>
__device__ inline void acc_zero(Acc<BM, BN, NW>& acc) {
  using C = TileCfg<BM, BN, 64, 0, NW>;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[fm][fn][r] = 0.f;
}

// The K loop of one tile.  before_step(k0, k1) is where a consumer waits
// for the data of the K-step that reads columns [k0, k1) of A: every wave
// calls it, before a workgroup barrier that precedes the first load of that
// step (so a wave that acquires there orders the whole workgroup's loads).
// Ends with a workgroup barrier, so LDS may be reused at once.
// NL: how many of the NW waves issue the stage loads (the last NL).  With
// NL = NW / 2 every SIMD holds one loading and one computing wave: when the
// memory pipeline backs up, a loading wave stalls at its load instructions
// while the other wave still has MFMAs to issue.
template <int BM, int BN, int BK = 64, int NSTAGES = 0, bool IND = false, int NW = 4, int NL = NW,
          class BeforeStep>
__device__ inline void gemm_tile(Acc<BM, BN, NW>& acc, const Operands& op, int64_t m0, uint16_t* lds,
                                 BeforeStep before_step) {
  static_assert(NL == NW || 2 * NL == NW, "all waves load, or the second half");
  using C = TileCfg<BM, BN, BK, NSTAGES, NL>;  // stage geometry and the loads of one loading wave
  constexpr int NS = C::NS;
  constexpr int MAXP = NS - 2 > 0 ? NS - 2 : 0;  // stages that may stay in flight at a step's end
  uint8_t* l8 = reinterpret_cast<uint8_t*>(lds);
  acc_zero(acc);
  const int wl_raw = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - (NW - NL);
  const bool loader = wl_raw >= 0;
  const TileAddr<BM, BN, BK, IND, NL> ta = tile_addr<BM, BN, BK, IND, NL>(op, m0, (uint32_t)(loader ? wl_raw : 0));
  const FragAddr<BM, BN, BK, NW> fa = frag_addr<BM, BN, BK, NW>();
  const int32_t steps = (int32_t)((op.k + BK - 1) / BK);
  const uint32_t lbase = lds_addr(l8);
  // Prologue: the first NS-1 stages.
  auto step_cols = [&](int32_t i) { before_step((int64_t)i * BK, min((int64_t)(i + 1) * BK, op.k)); };
  for (int32_t i = 0; i < NS - 1 && i < steps; ++i) step_cols(i);
  __syncthreads();
  if (loader)
    for (int32_t i = 0; i < NS - 1 && i < steps; ++i) {
      stage_issue_a(ta, lbase + i * C::STAGE_BYTES, i * BK);
      stage_issue_b(ta, lbase + i * C::STAGE_BYTES, i * BK);
    }
  if (NS - 1 < steps) step_cols(NS - 1);
  wait_stage_loads<C::LPS, MAXP>(min(NS - 2, steps - 1));  // stage 0 has landed
  __syncthreads();
  for (int32_t s = 0; s < steps; ++s) {
    const int32_t nxt = s + NS - 1;  // stage issued during this step
    const Prefetch<BM, BN, BK, IND, NL> pf{&ta, lbase + (uint32_t)(nxt % NS) * C::STAGE_BYTES, nxt * BK,
                                           loader && nxt < steps};
    stage_compute<BM, BN, BK, NW>(acc, l8 + (s % NS) * C::STAGE_BYTES, fa, pf);
    if (s + NS < steps) step_cols(s + NS);
    // Stage s+1 must have landed; the stages issued after it may stay in flight.
    wait_stage_loads<C::LPS, MAXP>(max(0, min(s + NS - 1, steps - 1) - (s + 1)));
    __syncthreads();
  }
}

// Calls f(row, col, value) for every accumulator element of this lane, with
// row/col relative to the tile origin (32x32 MFMA output layout: lane l holds
// column l%32; register r holds row (r%4) + 8*(r/4) + 4*(l/32)).
template <int BM, int BN, int NW, class F>
__device__ inline void acc_foreach(const Acc<BM, BN, NW>& acc, F f) {
  using C = TileCfg<BM, BN, 64, 0, NW>;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = (wave / C::WN) * (BM / 2);
  const int wn = (wave % C::WN) * (BN / C::WN);
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
// AUX is the buffer store's cache-policy operand (0: default).  Each store
// instruction writes 128 contiguous bytes of two rows (measured faster than
// computing the blocks transposed for 16-byte stores: 32-byte row pieces).
template <int BM, int BN, int AUX = 0, int NW = 4>
__device__ inline void acc_store(const Acc<BM, BN, NW>& acc, float* c, int64_t ldc, int64_t m0, int64_t n0,
                                 int64_t m_valid, int64_t n_valid) {
  const OutTile o = out_tile(c, ldc, m0, n0, m_valid, n_valid);
  acc_foreach(acc, [&](int row, int col, float v) { bstoref<AUX>(o.r, out_off(o, row, col), v); });
}

// Stores the tile through a row table: tile row i goes to row rows[i] of
// fp32 C (row pitch ldc, c_rows rows; nothing where rows[i] < 0), columns
// n0 + col clipped to n_valid.
template <int BM, int BN, int NW = 4>
__device__ inline void acc_store_rows(const Acc<BM, BN, NW>& acc, float* c, int64_t ldc, int64_t c_rows,
                                      const int32_t* rows, int64_t n0, int64_t n_valid) {
  using C = TileCfg<BM, BN, 64, 0, NW>;
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
    for (int i = 0; i < 16; ++i) {
      const int row = wm + fm * 32 + (i & 3) + 8 * (i >> 2) + 4 * (lane >> 5);
      const int32_t cr = rows[row];
      const uint32_t rb = cr >= 0 ? (uint32_t)cr * ldc_b + (uint32_t)n0 * 4 : kOOB;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int col = wn + fn * 32 + (lane & 31);
        bstoref(r, (rb != kOOB && col < n_left) ? rb + (uint32_t)col * 4 : kOOB, acc.v[fm][fn][i]);
      }
    }
}

}  // namespace ovl
