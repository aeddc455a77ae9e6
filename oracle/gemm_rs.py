"""GEMM followed by ReduceScatter.

Follows "Triton-distributed Semantics", Kernel Design Patterns, "GEMM and
ReduceScatter Overlapping": the GEMM produces output tiles and signals them;
the reduce-scatter side waits for tiles and reduces them.  With R ranks the
M rows split into R blocks of M/R rows; block p is sent to rank p, and the
own rank's output is its own block plus every peer's partial for it.
"""

from __future__ import annotations

import numpy as np

from .ag_gemm import gemm


def gemm_rs(a_u16, b_u16, partials, rank: int, ranks: int):
    """(local product, outbound blocks, own reduced block), all float64.

    local = A @ B (M x N); outbound[p] = rows of block p for p != rank (None
    at the own rank); own = local's block `rank` + sum over p != rank of
    partials[p], added in ascending p.
    """
    loc = gemm(a_u16, b_u16)
    m = loc.shape[0]
    if m % ranks:
        raise ValueError("M must split into equal row blocks")
    bm = m // ranks
    outbound = [None if p == rank else loc[p * bm:(p + 1) * bm] for p in range(ranks)]
    own = loc[rank * bm:(rank + 1) * bm].copy()
    for p in range(ranks):
        if p != rank:
            own += np.asarray(partials[p], dtype=np.float64)
    return loc, outbound, own


def rs_expected_flags(ranks: int, rank: int, tiles_per_block: int, flag_stride: int, epoch: int) -> np.ndarray:
    """Bytes of the outbound flag buffer after a completed run: R rows of
    `tiles_per_block` int64 slots (slot (p, t) at byte (p * tiles + t) *
    stride); every tile sent to a peer p != rank holds the epoch, the own
    row and all padding stay 0."""
    buf = np.zeros(ranks * tiles_per_block * flag_stride, dtype=np.uint8)
    slots = buf.view(np.int64).reshape(ranks, tiles_per_block, flag_stride // 8)
    for p in range(ranks):
        if p != rank:
            slots[p, :, 0] = epoch
    return buf
