"""Pins for the GEMM -> ReduceScatter and dispatch -> grouped GEMM oracles (CPU only)."""

import math

import numpy as np
import pytest

import oracle
import synth
from tests import pins

C3 = synth.CONFIGS["rs_r8_8192x4096x1792"]
C5 = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]


def _rs_small(kind="normal", R=4, rank=1):
    cfg = synth.GemmRsCfg("rs_small", R, 8 * R, 24, 16, 8, 8, 1.0, 0.25, 1.0, 77, rank)
    return cfg, synth.rs_inputs(cfg, kind)


# ------------------------------------------------------------------ GEMM-RS

def test_rs_own_minus_local_is_sum_of_partials():
    cfg, (a, b, parts) = _rs_small()
    loc, out, own = oracle.gemm_rs(a, b, parts, cfg.rank, cfg.ranks)
    bm = cfg.block_m
    blk = loc[cfg.rank * bm:(cfg.rank + 1) * bm]
    for i in range(bm):
        for j in range(cfg.n):
            want = math.fsum([blk[i, j]] + [float(parts[p][i, j]) for p in range(cfg.ranks) if p != cfg.rank])
            assert abs(own[i, j] - want) <= 8 * 2.0 ** -52 * (abs(blk[i, j]) + sum(
                abs(float(parts[p][i, j])) for p in range(cfg.ranks) if p != cfg.rank))


def test_rs_outbound_blocks_are_product_rows():
    cfg, (a, b, parts) = _rs_small()
    loc, out, own = oracle.gemm_rs(a, b, parts, cfg.rank, cfg.ranks)
    assert out[cfg.rank] is None
    ref = np.array(pins.brute_gemm(a, b))
    bm = cfg.block_m
    for p in range(cfg.ranks):
        if p != cfg.rank:
            assert np.allclose(out[p], ref[p * bm:(p + 1) * bm], rtol=0, atol=1e-13)


def test_rs_zero_partials_reduce_to_plain_block():
    cfg, (a, b, parts) = _rs_small()
    zeros = [None if p is None else np.zeros_like(p) for p in parts]
    loc, _, own = oracle.gemm_rs(a, b, zeros, cfg.rank, cfg.ranks)
    ref = np.array(pins.brute_gemm(a, b))
    bm = cfg.block_m
    assert np.allclose(own, ref[cfg.rank * bm:(cfg.rank + 1) * bm], rtol=0, atol=1e-13)


def test_rs_small_integers_exact():
    cfg, (a, b, parts) = _rs_small("smallint", R=8, rank=0)
    loc, out, own = oracle.gemm_rs(a, b, parts, cfg.rank, cfg.ranks)
    prod = pins.bf16_ints(a) @ pins.bf16_ints(b)
    bm = cfg.block_m
    want = prod[:bm].copy()
    for p in range(1, 8):
        want += parts[p].astype(np.int64)
    assert np.array_equal(own, want.astype(np.float64))


def test_rs_sampled_entries_fsum_full_shape():
    # Sampled entries of the 8192x4096x1792 product, against exact sums.
    a = synth.normal_bf16(C3.seed, 1, 0, (C3.m, C3.k))[:64]
    b = synth.normal_bf16(C3.seed, 2, 0, (C3.k, C3.n), C3.b_sigma)
    rows = np.arange(0, 64, 9)
    cols = (rows * 131) % C3.n
    vals = oracle.gemm_entries(a, b, rows, cols)
    ok, msg = pins.check_entries_fsum(vals, a, b, rows, cols)
    assert ok, msg


def test_rs_expected_flags():
    buf = oracle.rs_expected_flags(4, 2, 3, 8, 5).view(np.int64).reshape(4, 3)
    assert buf.tolist() == [[5, 5, 5], [5, 5, 5], [0, 0, 0], [5, 5, 5]]


# ------------------------------------------------------------------ dispatch

def _scan_layout(topk, rank, E):
    """Second construction: per local expert, scan tokens in order."""
    e_lo = rank * E
    e_list, t_list = [], []
    for e in range(E):
        for t in range(topk.shape[0]):
            for c in range(topk.shape[1]):
                if topk[t, c] == e_lo + e:
                    e_list.append(e)
                    t_list.append(t)
    return e_list, t_list


def _tiny_dispatch(R=2, T=8, H=4, E=2, num_experts=4, seed=5):
    cfg = synth.DispatchCfg("tiny", R, T, H, 3, 2, num_experts, E, 1.1, 1.0, 1.0, seed)
    return cfg, synth.dispatch_inputs(cfg)


@pytest.mark.parametrize("seed", range(4))
def test_dispatch_two_constructions_agree(seed):
    cfg, (x, topk, w) = _tiny_dispatch(R=3, T=16, seed=seed)
    for rank in range(cfg.ranks):
        for s in range(cfg.ranks):
            e1, t1 = oracle.dispatch_layout(topk[s], rank, cfg.experts_per_rank)
            e2, t2 = _scan_layout(topk[s], rank, cfg.experts_per_rank)
            assert e1.tolist() == e2 and t1.tolist() == t2


def test_dispatch_bruteforce_tiny():
    cfg, (x, topk, w) = _tiny_dispatch()
    rx, rs, rc = oracle.dispatch(x, topk, 0, cfg.experts_per_rank, cfg.cap)
    for s in range(cfg.ranks):
        e2, t2 = _scan_layout(topk[s], 0, cfg.experts_per_rank)
        assert rc[s].tolist() == [e2.count(e) for e in range(cfg.experts_per_rank)]
        for j, t in enumerate(t2):
            assert rs[s, j] == t
            assert np.array_equal(rx[s, j], x[s][t])
        assert not rx[s, len(t2):].any() and not rs[s, len(t2):].any()


def test_dispatch_single_rank_all_experts_is_textbook_moe_sort():
    # R = 1 with every expert local: the layout is a stable sort of the
    # flattened (token, choice) expert ids.
    T, K, E = 64, 2, 16
    topk = synth.zipf_top2_routing(3, 0, T, E, K, 1.1)
    e1, t1 = oracle.dispatch_layout(topk, 0, E)
    flat = topk.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert e1.tolist() == flat[order].tolist()
    assert t1.tolist() == (order // K).tolist()


def test_dispatch_counts_and_rows_full_routing():
    x = None
    cfg = C5
    topk = [synth.zipf_top2_routing(cfg.seed, s, cfg.tokens, cfg.num_experts, cfg.topk, cfg.zipf)
            for s in range(cfg.ranks)]
    total = sum(int(((t // cfg.experts_per_rank) == cfg.rank).sum()) for t in topk)
    layouts = [oracle.dispatch_layout(topk[s], cfg.rank, cfg.experts_per_rank) for s in range(cfg.ranks)]
    assert sum(len(l[1]) for l in layouts) == total
    for e_loc, tok in layouts:
        assert len(tok) <= cfg.cap
        keys = e_loc.astype(np.int64) * cfg.tokens + tok
        assert np.all(np.diff(keys) > 0)  # strictly sorted by (expert, token), no duplicates


def test_slices_are_indexed_by_source_rank():
    # The receiver's slice index is the sender's rank (the Aboleth README's
    # all-to-all puts at recv offset RANK * BYTES and sets flag RANK).
    cfg, (x, topk, w) = _tiny_dispatch(R=3, T=8)
    rx, rs, rc = oracle.dispatch(x, topk, 1, cfg.experts_per_rank, cfg.cap)
    for s in range(3):
        for j in range(int(rc[s].sum())):
            assert np.array_equal(rx[s, j], x[s][rs[s, j]])


def test_grouped_gemm_rows_fsum():
    cfg, (x, topk, w) = _tiny_dispatch(R=2, T=16, H=24, E=2, num_experts=4)
    rx, rs, rc = oracle.dispatch(x, topk, 0, cfg.experts_per_rank, cfg.cap)
    y = oracle.grouped_gemm(rx, rc, w)
    for s in range(2):
        bounds = np.cumsum(rc[s])
        n_valid = int(bounds[-1])
        for j in range(n_valid):
            e = int(np.searchsorted(bounds, j, side="right"))
            for c in range(w.shape[2]):
                exact, mag = pins.fsum_entry(rx[s, j], w[e][:, c])
                assert abs(y[s, j, c] - exact) <= 24 * 2.0 ** -53 * mag + 1e-300
        assert not y[s, n_valid:].any()
        rows = list(range(0, n_valid, 3))
        assert np.array_equal(oracle.grouped_gemm_rows(rx, rc, w, s, rows), y[s, rows])


def test_grouped_gemm_small_integers_exact():
    cfg = synth.DispatchCfg("si", 2, 32, 16, 8, 2, 8, 4, 1.1, 1.0, 1.0, 9)
    x, topk, w = synth.dispatch_inputs(cfg, "smallint")
    rx, rs, rc = oracle.dispatch(x, topk, 0, cfg.experts_per_rank, cfg.cap)
    y = oracle.grouped_gemm(rx, rc, w)
    xi = pins.bf16_ints(rx)
    wi = pins.bf16_ints(w)
    for s in range(2):
        r0 = 0
        for e in range(cfg.experts_per_rank):
            r1 = r0 + int(rc[s, e])
            assert np.array_equal(y[s, r0:r1], (xi[s, r0:r1] @ wi[e]).astype(np.float64))
            r0 = r1


def test_dispatch_refuses_rows_past_the_slice_capacity():
    """A slice holds tokens * min(topk, experts_per_rank) rows, which is every
    routed pair when a token's choices are distinct experts.  Routing that
    repeats a local expert with topk > experts_per_rank asks for more: the
    oracle refuses it (the library clips it and reports OVL_ESHAPE)."""
    T = 6
    x = [np.zeros((T, 8), np.uint16)] * 2
    ok = [np.array([[2, 3, 0]] * T, np.int32)] * 2        # 2 local rows per token: 2T = cap
    recv_x, src, cnt = oracle.dispatch(x, ok, 1, 2, 2 * T)
    assert cnt.sum() == 2 * 2 * T
    bad = [np.array([[2, 2, 2]] * T, np.int32)] * 2       # 3 rows per token for expert 2
    with pytest.raises(ValueError):
        oracle.dispatch(x, bad, 1, 2, 2 * T)
