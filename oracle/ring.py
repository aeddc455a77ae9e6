"""Ring all-reduce with per-tile signals (TEST INFRASTRUCTURE ONLY).

"Triton-distributed Semantics", section "Example: Ring AllReduce with
Overlap": W ranks each hold a vector; the vector is cut into W chunks; a
reduce-scatter phase of W - 1 steps, in which every rank sends one chunk to
the next rank and adds what it receives from the previous rank to its own
copy, is followed by an all-gather phase of W - 1 steps that passes the
reduced chunks on around the same ring.  Each tile of a chunk is signalled
on its own, so a tile can move on as soon as it has arrived.

The printed example is garbled (its reduce step adds into the tile it has
just sent, and its two phases disagree by one chunk on where the reduced
chunks sit).  The reading taken here keeps its send schedule: at
reduce-scatter step s rank r sends chunk (r - s) mod W to rank r + 1.  The
receiver therefore gets chunk (r - 1 - s) mod W, adds its own copy of that
chunk, and forwards the sum at the next step; after W - 1 steps rank r holds
the complete sum of chunk (r + 1) mod W.  All-gather step s' (0-based) then
has rank r forward chunk (r + 1 - s') mod W, the one it completed or last
received.  So the sum of chunk c is built in ring order from its first owner:
((x_c + x_{c+1}) + x_{c+2}) + ... + x_{c-1} (ranks mod W), each step adding
the rank's own element to the incoming partial, in the data type (float32);
every rank ends with the same bits.

Chunk c covers elements [c * cs, min(n, (c + 1) * cs)), cs = ceil(n / W)
rounded up to an even number of elements (chunks start on 8-byte words);
trailing chunks may be short or empty.

`ring_allreduce` simulates exactly those steps, message by message, in
float32.  `allreduce_sum` is the plain definition of the result (the float64
sum over ranks) that the pins hold the simulation to.
"""

from __future__ import annotations

import numpy as np


def ring_chunk_bounds(n: int, ranks: int):
    """[(lo, hi)] for chunks 0..ranks-1 of an n-element vector."""
    cs = -(-n // ranks) if ranks else 0
    cs += cs & 1
    return [(min(n, c * cs), min(n, (c + 1) * cs)) for c in range(ranks)]


def allreduce_sum(inputs) -> np.ndarray:
    """The plain definition: the element-wise sum over ranks, in float64."""
    return np.sum(np.stack([np.asarray(x, dtype=np.float64) for x in inputs]), axis=0)


def ring_allreduce(inputs) -> list:
    """Every rank's output (float32 [n]) after the reduce-scatter and
    all-gather phases of the ring, simulated step by step: all messages of a
    step are formed from the state before the step, then delivered."""
    W = len(inputs)
    x = [np.asarray(v, dtype=np.float32) for v in inputs]
    n = x[0].shape[0]
    bounds = ring_chunk_bounds(n, W)
    part = lambda c: slice(*bounds[c])  # noqa: E731
    # what each rank currently holds for each chunk (a partial, then the sum)
    held = [dict() for _ in range(W)]
    out = [np.zeros(n, dtype=np.float32) for _ in range(W)]
    # reduce-scatter
    for s in range(W - 1):
        msgs = []
        for r in range(W):
            c = (r - s) % W
            data = x[r][part(c)].copy() if s == 0 else held[r][c]
            msgs.append(((r + 1) % W, c, data))
        for dst, c, data in msgs:
            held[dst][c] = (data + x[dst][part(c)]).astype(np.float32)
    for r in range(W):
        c = (r + 1) % W
        out[r][part(c)] = held[r][c] if W > 1 else x[r][part(c)]
    # all-gather
    for s in range(W - 1):
        msgs = []
        for r in range(W):
            c = (r + 1 - s) % W
            msgs.append(((r + 1) % W, c, out[r][part(c)].copy()))
        for dst, c, data in msgs:
            out[dst][part(c)] = data
    return out
