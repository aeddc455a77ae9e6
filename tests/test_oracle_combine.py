"""Pins of the MoE combine oracle (CPU): the dispatch -> expert GEMM ->
combine chain against a dense per-token MoE forward, the reverse put as a
copy, one-hot gates, and planted mistakes."""

import numpy as np
import pytest

import oracle
import synth
from oracle.bf16 import bf16_to_f64


def _chain(R, T, H, N, topk, E, rank, seed):
    """Inputs for every rank, the combine at `rank` built from the dispatch
    and grouped GEMM of every rank, and the dense reference."""
    cfg = synth.DispatchCfg("pin", R, T, H, N, topk, R * E, E, 1.1, 1.0, 0.25, seed, rank)
    x = [synth.normal_bf16(seed, 4, s, (T, H)) for s in range(R)]
    w_all = np.stack([synth.normal_bf16(seed, 6, e, (H, N), 0.25) for e in range(R * E)])
    topk_idx = [synth.zipf_top2_routing(seed, s, T, R * E, topk, 1.1) for s in range(R)]
    gates, _ = synth.combine_inputs(cfg)
    cap = cfg.cap
    # what every rank q computes for the rows it receives
    ys = []
    for q in range(R):
        rx, rs, rc = oracle.dispatch(x, topk_idx, q, E, cap)
        ys.append((oracle.grouped_gemm(rx, rc, w_all[q * E:(q + 1) * E]), rc))
    y, rc = ys[rank]
    ret_in = [None if q == rank else ys[q][0][rank] for q in range(R)]  # q's rows for this rank's tokens
    ret_out, out = oracle.combine(y, rc, ret_in, topk_idx[rank], gates, rank, E)
    dense = np.zeros((T, N))
    xf = bf16_to_f64(x[rank])
    for t in range(T):
        for k in range(topk):
            dense[t] += float(gates[t, k]) * (xf[t] @ bf16_to_f64(w_all[topk_idx[rank][t, k]]))
    return dict(y=y, rc=rc, ret_in=ret_in, ret_out=ret_out, out=out, dense=dense, topk=topk_idx[rank],
                gates=gates, E=E, R=R, rank=rank)


@pytest.mark.parametrize("R,T,H,N,topk,E,rank,seed", [
    (3, 20, 16, 8, 2, 2, 1, 3),
    (4, 33, 24, 16, 2, 3, 0, 7),
    (1, 17, 8, 8, 2, 4, 0, 5),     # one rank: every expert local, the textbook MoE combine
])
def test_chain_equals_dense_moe(R, T, H, N, topk, E, rank, seed):
    c = _chain(R, T, H, N, topk, E, rank, seed)
    np.testing.assert_allclose(c["out"], c["dense"], rtol=1e-12, atol=1e-12)


def test_reverse_put_is_the_slice_rows():
    c = _chain(3, 20, 16, 8, 2, 2, 1, 3)
    for s in range(3):
        if s == 1:
            assert c["ret_out"][s] is None
            continue
        n = int(c["rc"][s].sum())
        assert c["ret_out"][s].shape == (n, 8)
        assert np.array_equal(c["ret_out"][s], c["y"][s, :n])


def test_one_hot_gates_pick_the_expert_row():
    c = _chain(3, 20, 16, 8, 2, 2, 2, 11)
    pos, owner = oracle.combine_positions(c["topk"], 3, 2)
    for k in range(2):
        g = np.zeros_like(c["gates"])
        g[:, k] = 1
        _, out = oracle.combine(c["y"], c["rc"], c["ret_in"], c["topk"], g, 2, 2)
        for t in range(20):
            q = owner[t, k]
            row = c["y"][2, pos[t, k]] if q == 2 else c["ret_in"][q][pos[t, k]]
            assert np.array_equal(out[t], row)


def test_positions_cover_every_slice_row_once():
    topk = synth.zipf_top2_routing(9, 0, 300, 16, 2, 1.1)
    pos, owner = oracle.combine_positions(topk, 4, 4)
    for q in range(4):
        got = np.sort(pos[owner == q])
        assert np.array_equal(got, np.arange(len(got)))


def test_planted_mistakes_fail_the_dense_pin():
    c = _chain(3, 20, 16, 8, 2, 2, 1, 3)
    # gates of the two choices swapped
    _, out = oracle.combine(c["y"], c["rc"], c["ret_in"], c["topk"], c["gates"][:, ::-1], 1, 2)
    assert not np.allclose(out, c["dense"])
    # a peer's returned rows taken from the wrong peer
    wrong = list(c["ret_in"])
    wrong[0], wrong[2] = wrong[2], wrong[0]
    _, out = oracle.combine(c["y"], c["rc"], wrong, c["topk"], c["gates"], 1, 2)
    assert not np.allclose(out, c["dense"])


def test_choices_that_are_not_experts_contribute_nothing():
    c = _chain(3, 20, 16, 8, 2, 2, 1, 3)
    topk = c["topk"].copy()
    topk[5, 1] = -1
    topk[9, 0] = 6  # past the 6 experts
    # the layout of the remaining choices is what the dispatch gives them
    _, out = oracle.combine(c["y"], c["rc"], c["ret_in"], topk, c["gates"], 1, 2)
    pos, owner = oracle.combine_positions(topk, 3, 2)
    for t, keep in ((5, 0), (9, 1)):
        q = owner[t, keep]
        row = c["y"][1, pos[t, keep]] if q == 1 else c["ret_in"][q][pos[t, keep]]
        np.testing.assert_allclose(out[t], float(c["gates"][t, keep]) * row, rtol=1e-15)
