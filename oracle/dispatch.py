"""All-to-all dispatch of routed tokens, then a grouped expert GEMM.

The all-to-all follows the Aboleth README's example: one program per peer
puts its slice into the receiver's buffer at an offset indexed by the source
rank and sets the receiver's flag for that source to the epoch.  Here the
receiving rank `rank` owns experts [rank*E, (rank+1)*E); source s's slice
holds, for every (token t, choice k) routed to a local expert, a copy of
token row t.  Rows in a slice are ordered by (local expert, token id); a
slice has room for `cap` rows.  The grouped GEMM multiplies each expert's
rows by that expert's weight.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f64


def dispatch_layout(topk_idx, rank: int, experts_per_rank: int):
    """For one source: (local expert ids, token ids) of its routed pairs that
    land on `rank`, sorted by (local expert, token id)."""
    topk_idx = np.asarray(topk_idx)
    e_lo = rank * experts_per_rank
    tok, _choice = np.nonzero((topk_idx >= e_lo) & (topk_idx < e_lo + experts_per_rank))
    e_loc = topk_idx[tok, _choice] - e_lo
    order = np.lexsort((tok, e_loc))  # primary key e_loc, then token id
    return e_loc[order].astype(np.int32), tok[order].astype(np.int32)


def dispatch(x, topk_idx, rank: int, experts_per_rank: int, cap: int):
    """(recv_x [R][cap][H] bf16 bits, recv_src [R][cap] int32,
    recv_count [R][E] int32).  Rows past a slice's count stay 0."""
    R = len(x)
    T, H = np.asarray(x[0]).shape
    recv_x = np.zeros((R, cap, H), dtype=np.uint16)
    recv_src = np.zeros((R, cap), dtype=np.int32)
    recv_count = np.zeros((R, experts_per_rank), dtype=np.int32)
    for s in range(R):
        e_loc, tok = dispatch_layout(topk_idx[s], rank, experts_per_rank)
        if len(tok) > cap:
            raise ValueError("slice capacity exceeded")
        recv_x[s, :len(tok)] = np.asarray(x[s])[tok]
        recv_src[s, :len(tok)] = tok
        recv_count[s] = np.bincount(e_loc, minlength=experts_per_rank)
    return recv_x, recv_src, recv_count


def _segments(count_row):
    start = 0
    for e, c in enumerate(count_row):
        yield e, start, start + int(c)
        start += int(c)


def grouped_gemm(recv_x, recv_count, w):
    """y [R][cap][N] float64: row j of slice s, which belongs to local expert
    e, is recv_x[s][j] @ w[e]; rows past the slice's count stay 0."""
    R, cap, H = recv_x.shape
    N = w.shape[2]
    y = np.zeros((R, cap, N), dtype=np.float64)
    wf = [bf16_to_f64(w[e]) for e in range(w.shape[0])]
    for s in range(R):
        for e, r0, r1 in _segments(recv_count[s]):
            if r1 > r0:
                y[s, r0:r1] = bf16_to_f64(recv_x[s, r0:r1]) @ wf[e]
    return y


def grouped_gemm_rows(recv_x, recv_count, w, s: int, rows) -> np.ndarray:
    """Rows `rows` of slice s of the same y (each row must be below the
    slice's count), for outputs too large to form whole."""
    bounds = np.cumsum(np.asarray(recv_count[s], dtype=np.int64))
    out = np.empty((len(rows), w.shape[2]), dtype=np.float64)
    for i, j in enumerate(rows):
        e = int(np.searchsorted(bounds, j, side="right"))
        out[i] = bf16_to_f64(recv_x[s, j]) @ bf16_to_f64(w[e])
    return out
