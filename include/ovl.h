/*
 * ovl.h: tile-centric overlap of communication with computation on one
 * MI355X (gfx950).
 *
 * Five operations, each one persistent HIP launch in which producer
 * workgroups move tiles and publish one int64 flag per tile batch, and
 * consumer workgroups wait on each flag and compute on that tile at once
 * ("Triton-distributed Semantics": Producer-Consumer Model, Signal-Based
 * Synchronization, Kernel Design Patterns).  The other ranks of a group are
 * emulated: their buffers are ordinary device buffers in the same HBM, and
 * a "peer" is a pointer in a host-side table (the role the symmetric heap's
 * per-rank base table plays in "Distributed Architecture Design", 5.3).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked HOST.  All buffers belong to
 *    the caller; the library never allocates device memory and keeps no
 *    pointer after a call returns.
 *  - bf16 is stored as uint16 bit patterns.  Matrices are row-major.
 *  - Device buffers must be 16-byte aligned, and row lengths (K, N, hidden)
 *    multiples of 8 elements, so that every row moves in 16-byte vectors.
 *  - *_run calls are asynchronous on `stream`: they validate, enqueue one or
 *    two kernels and return.  Argument errors are returned before anything
 *    is enqueued and nothing is written.  Errors found on the device (a
 *    wait that timed out) are recorded in the workspace and returned by
 *    ovl_check().
 *  - Flags: a flag slot is an int64 holding the epoch of the last signal
 *    (0 = never signalled).  A consumer waits until the slot is >= the
 *    epoch; the wait never modifies the slot, so any number of waiters may
 *    share it, and clearing is the reset's job (the pages' wait is
 *    non-consuming: "Triton-distributed Semantics", Wait Polling Mechanism).
 *    Epochs used on one flag buffer must increase from call to call; zero
 *    the buffer with ovl_flags_reset() before its first use, after which
 *    epochs start again at 1.
 *  - Ordering: a producer's data stores are complete at agent scope before
 *    its flag store (released by an agent-scope fence, or written as
 *    agent-scope stores and drained); a consumer acquires at agent scope
 *    after its flag load, or reads the data with agent-scope loads, and
 *    issues its tile loads only afterwards (the role consume_token plays in
 *    "Triton-distributed Semantics", Token-Based Data Dependency).  No
 *    system-scope ordering is used: every peer lives in the same HBM.
 *  - Two calls must not run concurrently on the same flags or workspace.
 *  - Results do not depend on the producer order, the mode or the number of
 *    producer workgroups: every output element is accumulated in one fixed
 *    order.
 */
#ifndef OVL_H_
#define OVL_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ovl_status;

enum {
  OVL_OK = 0,
  OVL_EINVAL = -1,       /* null pointer, bad rank, bad mode, bad option */
  OVL_ESHAPE = -2,       /* sizes that do not fit the tiling rules */
  OVL_EALIGN = -3,       /* pointer not 16-byte aligned, or a row length not a multiple of 8 */
  OVL_EEPOCH = -4,       /* epoch < 1, or not above the last epoch used on these flags */
  OVL_EHIP = -5,         /* a HIP runtime call failed */
  OVL_ETIMEOUT = -6,     /* device: a wait exceeded its spin limit */
  OVL_EUNSUPPORTED = -7  /* a limit of this implementation (listed at each call) */
};

/* Run modes.  FUSED is the method; the others exist to measure it and to
 * test it.  BARRIER lets every consumer start only after every unit has
 * been moved (the pages' debugging advice: rule out fine-grained
 * synchronisation bugs by synchronising everything first); COPY_ONLY runs
 * the producers alone; GEMM_ONLY runs the consumers alone, without any
 * wait, on operands the caller has already gathered or flagged. */
enum {
  OVL_MODE_FUSED = 0,
  OVL_MODE_COPY_ONLY = 1,
  OVL_MODE_GEMM_ONLY = 2,
  OVL_MODE_BARRIER = 3
};

typedef struct ovl_opts {
  uint32_t mode;        /* OVL_MODE_* */
  uint32_t producers;   /* producer workgroups; 0 = library default */
  uint64_t spin_limit;  /* polls before a wait gives up (OVL_ETIMEOUT); 0 = default (~2^22) */
  int64_t* trace;       /* AG-GEMM and dispatch: zero-filled device buffer of ag_gemm_trace_bytes()
                           or a2a_trace_bytes() bytes that the run fills with timestamps (see
                           there), or NULL for none */
  uint32_t jitter;      /* AG-GEMM only, a test aid: before moving each unit a producer
                           workgroup sleeps h(unit, epoch) mod (jitter + 1) intervals of about
                           64 shader clocks (h a fixed integer hash), so that units arrive in
                           shuffled, uneven order; 0 = off.  Results do not depend on it. */
  uint32_t reserved;    /* 0 */
} ovl_opts;

/* Size in bytes of the device-side error record at the start of every
 * workspace; the workspaces below are at least this large. */
#define OVL_ERROR_RECORD_BYTES 64

/* ------------------------------------------------------------------------
 * AllGather -> GEMM ("Triton-distributed Semantics", Kernel Design Patterns,
 * "AllGather and GEMM Overlapping").
 *
 * R ranks each hold an A shard of shard_m x k bf16; B is k x n bf16.  The
 * producer copies every shard s into rows [s*shard_m, (s+1)*shard_m) of
 * `gathered` (the own shard too, so that gathered is the concatenation of
 * all shards) and signals each flag unit; the consumer computes
 * C = gathered @ B in fp32 as the units arrive.
 *
 * Flag units: a unit is a row panel of min(tile_m, shard_m) rows of one
 * shard and a K-range of tiles_per_flag * tile_n columns (tiles_per_flag =
 * 0: all of k); the last panel of a shard and the last K-range may be
 * shorter.  Unit u = (shard * panels_per_shard + panel) * batches + batch;
 * its slot is at byte u * flag_stride of `flags`.  Tiles of one panel that
 * are always read together share one flag ("Triton-distributed Semantics",
 * Best Practices: batch signals when possible).
 *
 * Consumer order: tiles whose rows are all the own rank's are computed
 * first, straight from the own shard (they wait on nothing: Threadblock
 * Swizzling, start on local data); the others follow in the order their
 * first K-batch arrives under `producer_order`.
 * ---------------------------------------------------------------------- */
/* Tiles: the caller's tile_m x tile_n is the tile of the communication side
 * (the flag unit's rows, and the K-tile width that tiles_per_flag counts).
 * The consumer's output tile is chosen by the library from the problem
 * size: 256 x 256 when M and N are both at least 256 and there are at least
 * 128 such tiles, else 128 x 128 (then split along K when the tiles would
 * fill less than half the compute units; see ag_gemm_splits).  Any
 * consumer tile maps onto whole flag units: a tile waits on every unit its
 * rows and K-step touch, so the two tilings need not agree.
 * ag_gemm_tile_rows() reports the choice. */
typedef struct ag_gemm_desc {
  int32_t ranks;           /* R, 1..16 */
  int32_t rank;            /* this rank, 0 <= rank < R */
  int64_t shard_m;         /* rows per shard, >= 1 */
  int64_t k;               /* >= 8, multiple of 8 */
  int64_t n;               /* >= 8, multiple of 8 */
  int32_t tile_m;          /* flag-unit rows (capped at shard_m), >= 1; any value */
  int32_t tile_n;          /* K-tile width for tiles_per_flag, multiple of 8; any such value */
  int32_t tiles_per_flag;  /* K-tiles per flag unit, >= 0 (0 = all of k) */
  int32_t flag_stride;     /* bytes between flag slots, multiple of 8, >= 8 */
  int32_t unit_producers;  /* W, 0..16 (0 and 1: one producer workgroup moves and publishes
                              each unit).  W > 1: the unit's rows are split evenly over W
                              producer workgroups, each of which adds one arrival to the unit's
                              counter in the workspace after its rows (signal ADD); the arrival
                              that brings the counter to a multiple of W publishes the flag
                              (signal SET).  The counter only grows (by W per run), so it needs
                              no reset between runs; after a run that ended in an error, or a
                              change of plan on the same workspace, reset the workspace. */
} ag_gemm_desc;

typedef struct ag_gemm_plan_s* ag_gemm_plan_t;

/* Validates `desc` and builds an immutable, host-only plan (thread-safe to
 * share; touches no device).  Errors: EINVAL, ESHAPE, EALIGN; EUNSUPPORTED if
 * R > 16, if R*shard_m, k or n exceeds 2^20, or if an operand (gathered, B
 * or C) exceeds 1 GiB. */
ovl_status ag_gemm_plan(const ag_gemm_desc* desc, ag_gemm_plan_t* out);
ovl_status ag_gemm_plan_destroy(ag_gemm_plan_t plan);

int64_t ag_gemm_num_units(ag_gemm_plan_t plan);       /* R * panels_per_shard * batches */
size_t ag_gemm_flags_bytes(ag_gemm_plan_t plan);      /* num_units * flag_stride */
size_t ag_gemm_workspace_bytes(ag_gemm_plan_t plan);  /* >= OVL_ERROR_RECORD_BYTES */

/* Consumer tiling of the plan: the kernel's output tile has
 * ag_gemm_tile_rows(plan) rows, and there are ag_gemm_row_tiles(plan) rows
 * of tiles. */
int32_t ag_gemm_row_tiles(ag_gemm_plan_t plan);
int32_t ag_gemm_tile_rows(ag_gemm_plan_t plan);

/* K split of the plan (1 = none).  When few output tiles would leave most
 * compute units idle (skinny, bandwidth-bound shapes), each tile is computed
 * as `splits` ranges of K by different workgroups; every range stores its
 * fp32 product in the workspace and the last range to finish sums them in
 * range order, C = ((P_0 + P_1) + ...), so the result does not depend on
 * timing or producer order.  When every range runs in the launch's first
 * round the ranges of a tile wait for each other and each sums a stripe of
 * the tile's rows; otherwise the last range to finish sums the whole tile.
 * The workspace then holds two arrival counters per tile (returned to zero
 * by the tile's last range) and the partial products; after a run that
 * ended in an error, reset the workspace (ovl_flags_reset) before the
 * next. */
int32_t ag_gemm_splits(ag_gemm_plan_t plan);

/* The order in which consumers take rows of output tiles for a given
 * producer order (HOST int32 [num_units] permutation, or NULL = ascending):
 * writes ag_gemm_row_tiles(plan) row-tile indices to `out` (HOST).  Rows of
 * tiles whose rows are all the own rank's come first (the pages' Threadblock
 * Swizzling: each rank starts on its local data), then the others by the
 * latest position, in the producer order, of a first-K-batch unit covering
 * them; ties keep ascending index.  The device follows the same rule; this
 * host copy exists to inspect and test the schedule.  Errors: EINVAL for a
 * unit index out of range. */
ovl_status ag_gemm_consumer_order(ag_gemm_plan_t plan, const int32_t* producer_order, int32_t* out);

/* Device trace of a run (the pages ask to profile overlap efficiency and
 * synchronisation bottlenecks: "Triton-distributed Semantics", Best
 * Practices).  int64 records, times from the constant 100 MHz real-time
 * counter (s_memrealtime, 10 ns ticks), common to all compute units:
 *   [u], u < num_units:    the time unit u's flag was published (0: not moved);
 *   [num_units + 6 j + 0]: work item j's start (j = tile * splits + range, in
 *                          the launch's item order), [+1] its end (after its
 *                          stores), [+2] ticks its workgroup spent waiting for
 *                          flags, [+3] the consumer index that ran it, [+4] and
 *                          [+5] the shader-clock cycle counter (s_memtime) at
 *                          its start and end (their rate over the ticks is the
 *                          clock the item ran at).
 * Items of BARRIER and GEMM_ONLY runs record no waits. */
size_t ag_gemm_trace_bytes(ag_gemm_plan_t plan);

/* shards:   HOST array of R device pointers, bf16 [shard_m][k] each (read only).
 * b:        bf16 [k][n] (read only).
 * gathered: bf16 [R*shard_m][k], written by the producer (bit-exact copy).
 * c:        fp32 [R*shard_m][n], written by the consumer.
 * flags:    ag_gemm_flags_bytes(plan) bytes; unit slots are set to `epoch`.
 * workspace: ag_gemm_workspace_bytes(plan) bytes, zeroed by ovl_flags_reset.
 * producer_order: device int32 [num_units], a permutation of the unit
 *           indices giving the order in which producers move units; NULL =
 *           ascending.  Entries outside [0, num_units) are skipped; a unit
 *           that never appears is never moved, and waits on it end in
 *           OVL_ETIMEOUT.
 * opts:     NULL = FUSED with defaults; opts->trace: see ag_gemm_trace_bytes
 *           (8-byte aligned).
 * In GEMM_ONLY mode `gathered` must already hold the gathered operand and
 * neither flags nor shards other than the own one are read. */
ovl_status ag_gemm_run(ag_gemm_plan_t plan, const void* const* shards, const void* b,
                       void* gathered, float* c, int64_t* flags, void* workspace,
                       int64_t epoch, const int32_t* producer_order,
                       const ovl_opts* opts, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): ag_gemm_run
 * without the workspace argument.  Its workspace is a 16 MiB array inside the
 * library, one per GPU, held from the library's first use on that GPU until
 * the process ends.  A plan whose ag_gemm_workspace_bytes exceeds it is
 * refused with OVL_EUNSUPPORTED; every plan with one producer per unit fits
 * (at most 14 MiB), and unit_producers > 1 adds 8 bytes per flag unit.
 * Before the launch the call clears the array's run state (error record,
 * split counters, unit arrival counters) with a fill kernel on `stream`; it
 * calls no allocator.  Device errors are read with ovl_check(NULL, ...).  Every call on
 * one GPU shares its array: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and must not be issued.
 * Arguments, modes, results and errors as ag_gemm_run; the same kernels run,
 * so the outputs are bit-identical to ag_gemm_run's. */
ovl_status ag_gemm_run_noalloc(ag_gemm_plan_t plan, const void* const* shards, const void* b,
                               void* gathered, float* c, int64_t* flags, int64_t epoch,
                               const int32_t* producer_order, const ovl_opts* opts,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * GEMM -> ReduceScatter ("Triton-distributed Semantics", Kernel Design
 * Patterns, "GEMM and ReduceScatter Overlapping").
 *
 * This rank computes its local product L = A @ B (A: m x k bf16, B: k x n
 * bf16, fp32 result) whose m rows split into R blocks of m/R rows.  Block
 * p != rank is a partial destined for rank p: each tile of it is stored to
 * peer_out[p] and signalled in out_flags (put + signal).  For its own block
 * the rank waits for every peer's partial tile (in_flags) and writes
 *   out = L[rank block] + (sum over p != rank, ascending, of peer_in[p])
 * in fp32.  The own block's tiles are computed first, then the peer
 * blocks, starting at block rank+1.
 *
 * Flag layout (both buffers): R rows of tiles_per_block slots, tile t of
 * block p at byte (p * tiles_per_block + t) * flag_stride, with
 * tiles_per_block = ceil((m/R) / tile_m) * ceil(n / tile_n) and tiles
 * numbered row-major.  The own rank's row is never written.
 * ---------------------------------------------------------------------- */
typedef struct gemm_rs_desc {
  int32_t ranks;        /* R, 1..16; m must be a multiple of R */
  int32_t rank;
  int64_t m, n, k;      /* n, k multiples of 8 */
  int32_t tile_m;       /* output and flag tile: 256 x 256 (eight-wave workgroups) or */
  int32_t tile_n;       /* 128 x 128 (four-wave); tile_m == tile_n */
  int32_t flag_stride;  /* bytes, multiple of 8, >= 8 */
} gemm_rs_desc;

size_t gemm_rs_flags_bytes(const gemm_rs_desc* desc);      /* per flag buffer */
size_t gemm_rs_workspace_bytes(const gemm_rs_desc* desc);

/* a: bf16 [m][k]; b: bf16 [k][n].
 * peer_out: HOST array[R] of fp32 [m/R][n] device buffers (entry `rank` ignored).
 * peer_in:  HOST array[R] of fp32 [m/R][n] device buffers holding the peers'
 *           partials for this rank's block (entry `rank` ignored), valid once
 *           their in_flags slot reaches `epoch`.
 * out:      fp32 [m/R][n].
 * out_flags: written (epoch) per sent tile.  in_flags: read only.
 * workspace: gemm_rs_workspace_bytes(desc) bytes: besides the error record
 *           it holds one flag per own tile, so successive runs on one
 *           workspace need increasing epochs too (ovl_flags_reset restarts).
 * The own block's tiles store their accumulators to `out` first; the
 * reduction of the peers' partials is spread over the workgroups that
 * computed peer tiles: each takes a contiguous share of the own block's
 * rows, sums the partials in ascending peer order and adds the stored
 * accumulator, so out = acc + ((P_a + P_b) + ...).
 * Modes: FUSED, or GEMM_ONLY (same work and result, without in/out flag
 * traffic).
 * Errors as for ag_gemm_run; EUNSUPPORTED if tile_m x tile_n is not 256 x 256
 * or 128 x 128 (the size queries then return 0), if m, n or k exceeds 2^20,
 * or if A, B or the local product exceeds 1 GiB.  At 8192 x 4096 x 1792 over
 * 8 ranks the 256-tile runs in about 150 us and the 128-tile in about 205. */
ovl_status gemm_rs_run(const gemm_rs_desc* desc, const void* a, const void* b,
                       float* const* peer_out, const float* const* peer_in, float* out,
                       int64_t* out_flags, const int64_t* in_flags, void* workspace,
                       int64_t epoch, const ovl_opts* opts, hipStream_t stream);

/* ------------------------------------------------------------------------
 * All-to-all dispatch of routed tokens, then a grouped expert GEMM (the
 * Aboleth README's all-to-all with one program per peer, which puts a slice
 * at an offset indexed by the sender's rank and sets that sender's flag on
 * the receiver; and its compiled MoE dispatch).
 *
 * This rank owns experts [rank*E, (rank+1)*E), E = experts_per_rank.
 * Source s (every rank, this one included) sends, for each (token t,
 * choice j) with topk_idx[s][t][j] in that range, a copy of token row t.
 * Slice s of the receive buffers holds these rows ordered by (local expert,
 * token id); it has room for cap = tokens * min(topk, E) rows.  When slice s
 * is complete its flag is set to the epoch; the grouped GEMM waits on it and
 * computes y[s][row] = recv_x[s][row] @ w[local expert of row] in fp32.
 * Rows past a slice's count are never written (the caller zero-fills the
 * receive buffers once).
 * ---------------------------------------------------------------------- */
typedef struct a2a_desc {
  int32_t ranks;             /* R, 1..16 */
  int32_t rank;
  int64_t tokens;            /* tokens per source, 0..2^20 */
  int64_t hidden;            /* multiple of 8 */
  int64_t n;                 /* expert output width, multiple of 8 */
  int32_t topk;              /* 1..8, distinct experts per token */
  int32_t num_experts;       /* global experts = ranks * experts_per_rank */
  int32_t experts_per_rank;  /* 1..64 */
  int32_t flag_stride;       /* bytes, multiple of 8, >= 8 */
  int32_t tile_m, tile_n;    /* grouped-GEMM tile: tile_m rows of one expert's received rows
                                (taken across slices) x tile_n output columns.  0, 0 = the
                                default; the implemented tile is 256 x 256 for bf16 and for FP8
                                rows (a last column block at most half a tile wide runs as
                                256 x 128).  Any other pair: OVL_EUNSUPPORTED.
                                The combine does not read them. */
} a2a_desc;

size_t a2a_flags_bytes(const a2a_desc* desc);      /* ranks * flag_stride */
size_t a2a_workspace_bytes(const a2a_desc* desc);

/* Device trace of a fused dispatch -> grouped GEMM run (bf16 or FP8; the
 * pages ask to profile overlap efficiency: "Triton-distributed Semantics",
 * Best Practices), int64 records in 10 ns ticks of the 100 MHz real-time
 * counter (as for ag_gemm_trace_bytes):
 *   [s], s < R:        the time slice s's flag was published by a copy (0: not
 *                      by a copy: an empty slice);
 *   [R + p], p < 64:   the time producer workgroup p finished copying;
 *   [R + 64 + 8 j + 0] work item j's start, [+1] its end (after its stores),
 *                      [+2] ticks it spent waiting for slices (copying chunks
 *                      meanwhile), [+3] chunks it copied while waiting, [+4] the
 *                      consumer that ran it (-1: a producer, after the copy),
 *                      [+5] expert, [+6] m-tile, [+7] n-tile
 *                      (items in the launch's item order; unused records stay 0).
 * A bound for any routing: 8 * (R + 64 + 8 * (R * cap / 256 + E) * ceil(n / 128))
 * bytes, cap = tokens * min(topk, E); 0 for an invalid desc.  Only fused
 * (and GEMM_ONLY: no waits) runs record items. */
size_t a2a_trace_bytes(const a2a_desc* desc);

/* x:        HOST array[R] of bf16 [tokens][hidden] device buffers.
 * topk_idx: HOST array[R] of int32 [tokens][topk] device buffers (global expert ids;
 *           ids outside [0, num_experts) are ignored).
 * w:        bf16 [experts_per_rank][hidden][n].
 * recv_x:   bf16 [R][cap][hidden];  recv_src: int32 [R][cap] source token ids;
 * recv_count: int32 [R][experts_per_rank];  y: fp32 [R][cap][n].
 * flags:    a2a_flags_bytes(desc) bytes, slot s = slice from source s.
 * With tokens = 0 the row buffers (x, topk_idx, w, recv_x, recv_src, y) may
 * be NULL; counts are zeroed and every slice flag is still set. */
ovl_status a2a_dispatch_grouped_gemm_run(const a2a_desc* desc, const void* const* x,
                                         const int32_t* const* topk_idx, const void* w,
                                         void* recv_x, int32_t* recv_src, int32_t* recv_count,
                                         float* y, int64_t* flags, void* workspace,
                                         int64_t epoch, const ovl_opts* opts,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 dispatch -> FP8 grouped expert GEMM.  The Aboleth README measures its
 * compiled MoE dispatch and combine on "one FP8 layer" and fixes no format;
 * the reading: OCP FP8 E4M3 codes (bias 7, subnormals, no infinities,
 * largest finite 448) with one float32 scale per row.
 *
 * fp8_quantize_rows: bf16 [rows][cols] (uint16 bits) -> codes uint8
 * [rows][cols] and scales float32 [rows]: for a row with amax = max |x|,
 * scale = amax / 448 and code = E4M3(clamp(x * (448 / amax), +-448)), nearest
 * with ties to even, both quotients in float32; a row of zeros gets scale 1
 * and zero codes.  Used for the tokens (each source, before its dispatch)
 * and for the expert weights, quantized as rows of W_e transposed ([n][hidden]:
 * one scale per output column).  cols must be a multiple of 16.
 * ---------------------------------------------------------------------- */
ovl_status fp8_quantize_rows(const void* in_bf16, void* codes, float* scale, int64_t rows, int64_t cols,
                             hipStream_t stream);

/* As a2a_dispatch_grouped_gemm_run, with FP8 rows: x8 (HOST array[R] of
 * uint8 [tokens][hidden] codes) and x_scale (HOST array[R] of float32
 * [tokens]) per source; w8 uint8 [experts_per_rank][n][hidden] (W_e
 * transposed, K contiguous) with w_scale float32 [experts_per_rank][n].
 * The dispatch moves each row's codes to recv_x8 uint8 [R][cap][hidden] and
 * its scale to recv_scale float32 [R][cap] (same layout, recv_src and
 * recv_count as the bf16 call); then
 *   y[s][j][c] = (sum_k recv_x8[s][j][k] * w8[e][c][k]) * recv_scale[s][j] * w_scale[e][c]
 * in fp32 (MFMA sums of exact code products, K ascending in steps of 64).
 * hidden must be a multiple of 16.  Same modes, flags, workspace
 * (a2a_workspace_bytes) and errors as the bf16 call. */
ovl_status a2a_dispatch_grouped_gemm_fp8_run(const a2a_desc* desc, const void* const* x8,
                                             const float* const* x_scale, const int32_t* const* topk_idx,
                                             const void* w8, const float* w_scale, void* recv_x8,
                                             float* recv_scale, int32_t* recv_src, int32_t* recv_count,
                                             float* y, int64_t* flags, void* workspace, int64_t epoch,
                                             const ovl_opts* opts, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MoE combine: the reverse all-to-all of the expert outputs, then the
 * gate-weighted sum back in token order (the Aboleth README's compiled MoE
 * dispatch *and combine*; the reverse all-to-all for expert-parallel MoE in
 * the Triton distributed tutorial list).  Same slice signal discipline as
 * the dispatch, in reverse.  The pages give no formula; the reading:
 *
 *  - reverse put: this rank computed y[s][0:count_s] for source s (the rows
 *    of a2a_dispatch_grouped_gemm_run, slice order); for every peer s it
 *    copies them to ret_out[s] (row j to row j) and sets out_flags[s] to the
 *    epoch once all are there (a peer it sends nothing to is flagged at once);
 *  - sum: for this rank's own tokens (routing topk_idx [tokens][topk],
 *    gates [tokens][topk] fp32), every peer q returns, in ret_in[q], the rows
 *    its experts computed for them, in q's slice order for this rank (local
 *    expert, then token), valid once in_flags[q] >= epoch.  Then
 *      out[t] = sum over choices k, ascending, of gates[t][k] * Y(t, k)
 *    in fp32, Y(t, k) being the row of (t, k) in y[rank] when its expert is
 *    local, else in ret_in[owner]; choices with ids outside
 *    [0, num_experts) contribute nothing.
 *
 * desc: as for the dispatch (tokens = this rank's tokens = the per-source
 * token count, so cap = tokens * min(topk, experts_per_rank) rows per
 * slice; hidden is not used).
 * ---------------------------------------------------------------------- */
size_t a2a_combine_flags_bytes(const a2a_desc* desc);      /* ranks * flag_stride (each of out/in) */
size_t a2a_combine_workspace_bytes(const a2a_desc* desc);  /* 256 + choice rows */

/* y:          fp32 [R][cap][n]; recv_count: int32 [R][experts_per_rank] (both as the
 *             dispatch left them).
 * ret_out:    HOST array[R] of fp32 [cap][n] device buffers (entry rank ignored).
 * ret_in:     HOST array[R] of fp32 [cap][n] device buffers (entry rank ignored).
 * topk_idx:   int32 [tokens][topk]; gates: fp32 [tokens][topk]; out: fp32 [tokens][n].
 * out_flags:  written (slot s), in_flags: read (slot q); a2a_combine_flags_bytes each.
 * Modes: FUSED; COPY_ONLY (reverse put and its flags only); GEMM_ONLY (the sum
 * only, without waiting on in_flags: ret_in must be there).  With tokens = 0
 * the row buffers may be NULL and the out flags are still set. */
ovl_status a2a_combine_run(const a2a_desc* desc, const float* y, const int32_t* recv_count,
                           float* const* ret_out, const float* const* ret_in,
                           const int32_t* topk_idx, const float* gates, float* out,
                           int64_t* out_flags, const int64_t* in_flags, void* workspace,
                           int64_t epoch, const ovl_opts* opts, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Ring all-reduce with per-tile signals ("Triton-distributed Semantics",
 * Example: Ring AllReduce with Overlap).  Every one of the R ranks of the
 * ring is emulated in the one launch: in[r] and out[r] are rank r's vectors
 * (fp32, n elements each) and out[r] ends as the element-wise sum of all
 * in[q], with the same bits on every rank.
 *
 * The vector is cut into R chunks of cs = ceil(n / R) elements, rounded up to
 * an even count (the last ones may be short or empty), and each chunk into
 * tiles of `tile` elements.  Reduce-scatter step s (0 <= s < R - 1): rank r
 * sends chunk (r - s) mod R to rank r + 1 (the example's send schedule),
 * which adds its own copy of that chunk; after R - 1 steps rank r holds the
 * complete chunk (r + 1) mod R, and R - 1 all-gather steps pass the complete
 * chunks on around the ring.  (The printed example reduces into the tile it
 * has just sent and its phases disagree by one chunk; this is the reading
 * its send schedule supports.)  So chunk c is summed in float32 as
 * ((x_c + x_{c+1}) + x_{c+2}) + ... + x_{c-1}, ranks mod R.  Each tile of
 * each step is signalled on its own: flag slot ((r * (2R - 2)) + s - 1) *
 * tiles_per_chunk + j holds the epoch once tile j of rank r's step-s input
 * (s >= 1) is in out[r]; every slot is set by the end of a run.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t ranks;        /* R, 1 .. 16 */
  int64_t n;            /* fp32 elements per rank, 0 .. 2^31 */
  int64_t tile;         /* elements per signalled tile: even, >= 2 */
  int32_t flag_stride;  /* bytes between flag slots: a multiple of 8 */
} ring_desc;

size_t ring_allreduce_flags_bytes(const ring_desc* desc);      /* R * (2R - 2) * tiles_per_chunk * flag_stride */
size_t ring_allreduce_workspace_bytes(const ring_desc* desc);  /* 256 (0 if desc is invalid) */

/* in, out: HOST arrays[R] of device fp32 [n] buffers.  Partial sums travel
 * through the outputs while the inputs are read, so no output may overlap
 * an input or another output (OVL_EINVAL).  Modes: FUSED (one launch, tiles
 * pipelined through their flags); BARRIER (one launch per ring step, so every
 * tile of a step is in place before any tile of the next moves: the same
 * steps without tile-level overlap).  Both give the same bits and flags.
 * Device errors (site 8, index = flag slot) come only from a wait that
 * exceeded opts->spin_limit. */
ovl_status ring_allreduce_run(const ring_desc* desc, const float* const* in, float* const* out,
                              int64_t* flags, void* workspace, int64_t epoch, const ovl_opts* opts,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Flags, errors, measurement.
 * ---------------------------------------------------------------------- */

/* Zeroes flag_bytes of `flags` and ws_bytes of `workspace` on `stream`
 * (either pointer may be NULL with size 0) and restarts the epoch sequence
 * of `flags` at 1.  Uses a fill kernel, not a memset node, so it may be
 * captured in a graph. */
ovl_status ovl_flags_reset(int64_t* flags, size_t flag_bytes, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/* Waits for `stream`, then returns the status recorded on the device in
 * `workspace` (the first error recorded wins):
 *  - OVL_ETIMEOUT: a wait exceeded its spin limit;
 *  - OVL_EEPOCH: a wait found a flag ABOVE the awaited epoch (a signal of a
 *    later run, or a stale epoch: the pages' wait accepts flag >= epoch, and
 *    producers store exactly the epoch, so a larger value means the epoch
 *    rule was broken and a consumer may have run ahead of its producer);
 *  - OVL_ESHAPE (site 9): a dispatch slice would exceed its capacity (routing
 *    rows that repeat a local expert); the rows past the capacity were dropped.
 * detail (HOST, may be NULL) receives {site, index, observed value, awaited
 * value}; sites: 1 AG-GEMM unit flag, 2 AG-GEMM barrier mode, 3 GEMM-RS in
 * flag, 4 dispatch slice flag, 5 GEMM-RS own-tile flag, 6 AG-GEMM split-K
 * range counter (index = tile), 7 combine in flag (index = peer), 8 ring
 * all-reduce tile flag, 9 dispatch slice capacity (index = source; observed =
 * rows asked for, awaited = capacity).
 * workspace = NULL reads the record of the allocation-free calls on the
 * current device (ag_gemm_run_noalloc). */
ovl_status ovl_check(const void* workspace, int64_t* detail, hipStream_t stream);

const char* ovl_strerror(ovl_status status);

/* Plain 16-byte-vector copy of `bytes` bytes (a multiple of 16) from src to
 * dst, with `blocks` workgroups of 256 threads (0 = one per compute unit,
 * the fastest count measured).  A reference point for the
 * HBM roofline and for scaling hardware byte counters. */
ovl_status ovl_copy(void* dst, const void* src, size_t bytes, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* OVL_H_ */
