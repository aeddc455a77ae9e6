"""MoE combine: the reverse all-to-all of the expert outputs, then the
gate-weighted sum back in token order (TEST INFRASTRUCTURE ONLY).

The pages name the compiled MoE "dispatch and combine" programs (the Aboleth
README) and a reverse all-to-all for expert-parallel MoE (the Triton
distributed tutorial list); they give no formula, so this is the plain
reading the dispatch fixes.  Rank `rank` computed, for every source s, the
expert outputs y[s][j] of the rows it received from s (slice order: local
expert, then token).  The combine

  1. sends those rows back: source s receives this rank's rows y[s][0:count_s]
     (in the same order) -- the reverse put, one slice per peer;
  2. for this rank's own tokens, receives from every peer q the rows q
     computed for them (ret_in[q], in q's slice order for this rank), and
     writes out[t] = sum over choices k (ascending) of gates[t][k] * Y(t, k),
     Y(t, k) being the expert output of token t under its k-th expert: the
     row of (t, k) in the slice of the rank that owns that expert; a choice
     whose id is not an expert contributes nothing (the dispatch skips it).
"""

from __future__ import annotations

import numpy as np

from .dispatch import dispatch_layout


def combine_positions(topk_idx, ranks: int, experts_per_rank: int):
    """pos [T][topk] int64 and owner [T][topk]: for each (token t, choice k),
    the rank q owning expert topk_idx[t][k] and the row of (t, k) in q's slice
    of this source's rows -- the layout the dispatch on q gives them
    (ordered by (local expert, token), a token's repeated expert by choice)."""
    topk_idx = np.asarray(topk_idx)
    T, K = topk_idx.shape
    owner = topk_idx // experts_per_rank
    pos = np.full((T, K), -1, dtype=np.int64)
    for q in range(ranks):
        e_loc, tok = dispatch_layout(topk_idx, q, experts_per_rank)
        seen = {}
        for j, (e, t) in enumerate(zip(e_loc.tolist(), tok.tolist())):
            # the j-th row of q's slice is the next not yet placed choice of t
            # that picks expert q*E + e
            ks = [k for k in range(K) if topk_idx[t, k] == q * experts_per_rank + e]
            n = seen.get((t, e), 0)
            pos[t, ks[n]] = j
            seen[(t, e)] = n + 1
    return pos, owner


def combine(y, recv_count, ret_in, topk_idx, gates, rank: int, experts_per_rank: int):
    """(ret_out, out): ret_out[s] float64 [count_s][N] for s != rank (None at
    rank) -- the rows this rank sends back to source s; out float64 [T][N]."""
    y = np.asarray(y, dtype=np.float64)
    R = y.shape[0]
    ret_out = [None if s == rank else y[s, :int(np.sum(recv_count[s]))].copy() for s in range(R)]
    pos, owner = combine_positions(topk_idx, R, experts_per_rank)
    T, K = np.asarray(topk_idx).shape
    out = np.zeros((T, y.shape[2]), dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    idx = np.asarray(topk_idx)
    for t in range(T):
        for k in range(K):
            if not 0 <= idx[t, k] < R * experts_per_rank:
                continue  # not an expert: contributes nothing
            q = int(owner[t, k])
            row = y[rank, pos[t, k]] if q == rank else np.asarray(ret_in[q][pos[t, k]], dtype=np.float64)
            out[t] += g[t, k] * row
    return ret_out, out
