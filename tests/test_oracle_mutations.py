"""The pins bite: mistakes planted in copies of the oracle's arithmetic (on
the CPU) make the independent checks fail, and the golden fixtures from the
pages hold."""

import os

import numpy as np

import oracle
import synth
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def _sample(m, n, count=64, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, m, count), rng.integers(0, n, count)


# --------------------------------------------------------- planted GEMM mistakes

def _ag_case():
    cfg = synth.CONFIGS["ag_r2_128x256x256"]
    shards, b = synth.ag_inputs(cfg)
    g = oracle.all_gather(shards)
    return g, b


def test_correct_oracle_passes_the_fsum_pin():
    g, b = _ag_case()
    c = oracle.gemm(g, b)
    rows, cols = _sample(*c.shape)
    assert pins.check_entries_fsum(c, g, b, rows, cols)[0]


def test_transposed_operand_is_caught():
    g, b = _ag_case()
    bad = oracle.bf16_to_f64(g) @ oracle.bf16_to_f64(b).T  # B is square here
    rows, cols = _sample(*bad.shape)
    assert not pins.check_entries_fsum(bad, g, b, rows, cols)[0]


def test_dropped_last_k_term_is_caught():
    g, b = _ag_case()
    bad = oracle.bf16_to_f64(g[:, :-1]) @ oracle.bf16_to_f64(b[:-1])
    rows, cols = _sample(*bad.shape)
    assert not pins.check_entries_fsum(bad, g, b, rows, cols)[0]


def test_float32_accumulation_is_caught():
    g, b = _ag_case()
    bad = (oracle.bf16_to_f32(g) @ oracle.bf16_to_f32(b)).astype(np.float64)
    rows, cols = _sample(*bad.shape, count=256)
    assert not pins.check_entries_fsum(bad, g, b, rows, cols)[0]


def test_wrong_gather_order_is_caught():
    cfg = synth.AgGemmCfg("t", 3, 2, 5, 3, 2, 2, 1.0, 1.0, 3, False)
    shards, b = synth.ag_inputs(cfg)
    bad = oracle.all_gather(shards[::-1])
    assert not all(np.array_equal(bad[2 * s:2 * s + 2], shards[s]) for s in range(3))


def test_sign_error_in_partials_is_caught():
    cfg = synth.GemmRsCfg("t", 4, 16, 8, 8, 4, 4, 1.0, 1.0, 1.0, 21, 0)
    a, b, parts = synth.rs_inputs(cfg, "smallint")
    loc = oracle.gemm(a, b)
    bad = loc[:4].copy()
    for p in range(1, 4):
        bad -= parts[p]
    prod = pins.bf16_ints(a) @ pins.bf16_ints(b)
    want = prod[:4] + sum(parts[p].astype(np.int64) for p in range(1, 4))
    assert not np.array_equal(bad, want.astype(np.float64))


def test_layout_sorted_by_token_first_is_caught():
    topk = synth.zipf_top2_routing(1, 0, 32, 4, 2, 1.1)
    tok, ch = np.nonzero(topk < 2)
    e_loc = topk[tok, ch]
    order = np.lexsort((e_loc, tok))  # wrong: token-major
    e_list, t_list = [], []
    for e in range(2):
        for t in range(32):
            for c in range(2):
                if topk[t, c] == e:
                    e_list.append(e)
                    t_list.append(t)
    assert tok[order].tolist() != t_list


# --------------------------------------------------------- golden fixtures

def test_golden_signal_slot_stride():
    for dtype, nbytes, per_slot in _rows("signal_slot_stride.txt"):
        assert 64 // int(nbytes) == int(per_slot)
        if dtype == "int64":
            buf = oracle.expected_flags(6, 64, 2).view(np.int64)
            assert np.flatnonzero(buf).tolist() == [int(per_slot) * u for u in range(6)]


def test_golden_alltoall_slices_indexed_by_sender():
    cfg = synth.DispatchCfg("g", 4, 16, 4, 3, 2, 8, 2, 1.1, 1.0, 1.0, 31)
    x, topk, w = synth.dispatch_inputs(cfg)
    for rank_s, pid, peer, slot, flag in _rows("alltoall_peer_map.txt"):
        rank_s, peer, slot = int(rank_s), int(peer), int(slot)
        assert peer != rank_s and slot == rank_s and int(flag) == rank_s
        rx, rs, rc = oracle.dispatch(x, topk, peer, cfg.experts_per_rank, cfg.cap)
        e_loc, tok = oracle.dispatch_layout(topk[rank_s], peer, cfg.experts_per_rank)
        assert rs[slot, :len(tok)].tolist() == tok.tolist()
        for j, t in enumerate(tok):
            assert np.array_equal(rx[slot, j], x[rank_s][t])
