"""AllGather followed by GEMM, and the flags it leaves behind.

Follows "Triton-distributed Semantics", Kernel Design Patterns, "AllGather
and GEMM Overlapping": the producer moves every rank's tiles into a shared
buffer and signals each one; the consumer runs the GEMM on the gathered
operand.  The overlapped kernel reaches exactly the plain result below.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f64


def all_gather(shards) -> np.ndarray:
    """Gathered operand: rank s's shard occupies rows [s*Ms, (s+1)*Ms), in
    rank order whatever order the tiles moved in (the gather of the
    "AllGather and GEMM Overlapping" pattern).  Bits are moved, not
    converted."""
    shards = [np.asarray(s) for s in shards]
    rows = [s.shape[0] for s in shards]
    out = np.empty((sum(rows),) + shards[0].shape[1:], dtype=shards[0].dtype)
    r0 = 0
    for s in shards:
        out[r0:r0 + s.shape[0]] = s
        r0 += s.shape[0]
    return out


def gemm(a_u16: np.ndarray, b_u16: np.ndarray) -> np.ndarray:
    """C[m][n] = sum_k A[m][k] * B[k][n] in float64 (bf16 inputs decoded
    exactly; each product of two bf16 values is exact in float64)."""
    return bf16_to_f64(a_u16) @ bf16_to_f64(b_u16)


def gemm_entries(a_u16: np.ndarray, b_u16: np.ndarray, rows, cols) -> np.ndarray:
    """Selected entries C[rows[i]][cols[i]] of the same product, one dot
    product each (for outputs too large to form whole)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(len(rows), dtype=np.float64)
    for i, (r, c) in enumerate(zip(rows, cols)):
        out[i] = np.dot(bf16_to_f64(a_u16[r]), bf16_to_f64(b_u16[:, c]))
    return out


def ag_gemm(shards, b_u16):
    """(gathered bf16 bits, C float64) for C = gather(shards) @ B."""
    g = all_gather(shards)
    return g, gemm(g, b_u16)


def ag_flag_units(ranks: int, shard_m: int, k: int, tile_m: int, tile_n: int, tiles_per_flag: int):
    """Flag units of the gathered operand: (units, panels_per_shard, batches).

    One flag per batch of tiles that are always read together ("Triton-
    distributed Semantics", Best Practices, batching signals): a unit is a
    row panel of min(tile_m, shard_m) rows of one shard and a K-range of
    tiles_per_flag * tile_n columns (tiles_per_flag = 0: all of K).  The
    pages leave ragged sizes open; here a shard's last panel and the last
    K-range are simply shorter, so every row and column belongs to exactly
    one unit.  The unit index is (shard * panels_per_shard + panel) *
    batches + batch.
    """
    unit_rows = min(tile_m, shard_m)
    panels = -(-shard_m // unit_rows)
    width = k if tiles_per_flag <= 0 else tiles_per_flag * tile_n
    batches = -(-k // width)
    return ranks * panels * batches, panels, batches


def expected_flags(num_units: int, flag_stride: int, epoch: int) -> np.ndarray:
    """The flag buffer's bytes after a completed run: every unit's int64 slot
    holds the epoch it was signalled with (the Aboleth README's put_signal /
    wait_signal pair carries the epoch as the flag value), every other byte
    is 0.  Slot u starts at byte u * flag_stride."""
    if flag_stride % 8:
        raise ValueError("flag stride must be a multiple of 8 bytes")
    buf = np.zeros(num_units * flag_stride, dtype=np.uint8)
    slots = buf.view(np.int64)
    slots[:: flag_stride // 8] = epoch
    return buf
