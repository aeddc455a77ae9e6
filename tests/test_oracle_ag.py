"""Pins for the AllGather -> GEMM oracle (CPU only)."""

import numpy as np
import pytest

import oracle
import synth
from tests import pins

C1 = synth.CONFIGS["ag_r2_128x256x256"]
C2 = synth.CONFIGS["ag_r8_8192x3584x4096"]
C4 = synth.CONFIGS["ag_r8_skinny_128x7168x8192"]


def _tiny(seed=7, R=2, Ms=3, K=5, N=4, kind="normal"):
    cfg = synth.AgGemmCfg("tiny", R, Ms, K, N, 2, 2, 1.0, 0.5, seed, False)
    return synth.ag_inputs(cfg, kind)


def test_bf16_decoder_matches_ieee_table():
    u = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_to_f64(u)
    ref = pins.decode_table()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_gather_is_concatenation_in_rank_order_bruteforce():
    shards, _ = _tiny(R=3, Ms=4, K=6)
    g = oracle.all_gather(shards)
    assert g.dtype == np.uint16 and g.shape == (12, 6)
    for s in range(3):
        for i in range(4):
            for k in range(6):
                assert g[s * 4 + i, k] == shards[s][i, k]


def test_gemm_matches_bruteforce_tiny():
    for seed in range(5):
        shards, b = _tiny(seed=seed)
        g, c = oracle.ag_gemm(shards, b)
        ref = pins.brute_gemm(g, b)
        assert np.allclose(c, np.array(ref), rtol=0, atol=1e-15 * np.abs(ref).max())


def test_small_config_every_entry_within_fsum_bound():
    shards, b = synth.ag_inputs(C1)
    g, c = oracle.ag_gemm(shards, b)
    assert c.shape == (C1.m, C1.n)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, C1.m, 400)
    cols = rng.integers(0, C1.n, 400)
    ok, msg = pins.check_entries_fsum(c, g, b, rows, cols)
    assert ok, msg


def test_gemm_entries_matches_fsum_at_large_shape():
    # One shard of the 8-rank 8192x3584x4096 workload, sampled entries only.
    shard = synth.normal_bf16(C2.seed, 1, 3, (64, C2.k))
    b = synth.normal_bf16(C2.seed, 2, 0, (C2.k, 96), C2.b_sigma)
    rows = np.arange(0, 64, 7)
    cols = (rows * 5) % 96
    vals = oracle.gemm_entries(shard, b, rows, cols)
    ok, msg = pins.check_entries_fsum(vals, shard, b, rows, cols)
    assert ok, msg


def test_identity_b_reproduces_gathered_operand():
    # B[k][n] = [k == n]: C must be the gathered operand (zero-padded when N > K).
    for K, N in ((8, 5), (5, 8), (6, 6)):
        cfg = synth.AgGemmCfg("id", 2, 3, K, N, 3, 3, 1.0, 1.0, 11, False)
        shards, b = synth.ag_inputs(cfg, "identity_b")
        g, c = oracle.ag_gemm(shards, b)
        want = np.zeros((6, N))
        d = min(K, N)
        want[:, :d] = pins.decode_np(g[:, :d])
        assert np.array_equal(c, want)


def test_small_integers_exact_against_integer_product():
    shards, b = synth.ag_inputs(C1, "smallint")
    g, c = oracle.ag_gemm(shards, b)
    exact = pins.bf16_ints(g) @ pins.bf16_ints(b)  # int64 product: exact
    assert np.array_equal(c, exact.astype(np.float64))


def test_block_rows_of_product_are_per_shard_products():
    # gather(A) @ B == stack(shard_s @ B): catches a gather in the wrong order.
    shards, b = _tiny(R=4, Ms=2, K=7, N=3)
    _, c = oracle.ag_gemm(shards, b)
    for s in range(4):
        part = np.array(pins.brute_gemm(shards[s], b))
        assert np.allclose(c[2 * s:2 * s + 2], part, rtol=0, atol=1e-14)


def test_single_rank_reduces_to_plain_gemm():
    shards, b = _tiny(R=1, Ms=5, K=4, N=3)
    g, c = oracle.ag_gemm(shards, b)
    assert np.array_equal(g, shards[0])
    assert np.allclose(c, np.array(pins.brute_gemm(shards[0], b)), rtol=0, atol=1e-14)


@pytest.mark.parametrize("cfg,tpf,want", [
    (C1, 0, (4, 2, 1)),      # 2 ranks x 2 panels of 32 rows, all of K
    (C2, 0, (32, 4, 1)),     # 8 ranks x 4 panels of 256 rows
    (C2, 1, (512, 4, 16)),   # ... split into 16 K-batches of 256 columns
    (C4, 0, (8, 1, 1)),      # 16-row shards < 128-row tile: one unit per shard
    (C4, 4, (128, 1, 16)),   # ... in 16 K-batches of 512 columns
])
def test_flag_units(cfg, tpf, want):
    assert oracle.ag_flag_units(cfg.ranks, cfg.shard_m, cfg.k, cfg.tile_m, cfg.tile_n, tpf) == want


def test_flag_units_ragged_cover_every_row_and_column_once():
    # 3 ranks of 100 rows, 48-row panels (48, 48, 4), K = 200 in batches of
    # 2 x 40 = 80 columns (80, 80, 40): 3 * 3 * 3 units.
    units, panels, batches = oracle.ag_flag_units(3, 100, 200, 48, 40, 2)
    assert (units, panels, batches) == (27, 3, 3)
    covered = np.zeros((300, 200), dtype=np.int32)
    for u in range(units):
        b = u % batches
        s, p = divmod(u // batches, panels)
        r0 = s * 100 + p * 48
        r1 = min(r0 + 48, (s + 1) * 100)
        covered[r0:r1, b * 80:min(200, (b + 1) * 80)] += 1
    assert (covered == 1).all()


def test_expected_flags_layout():
    buf = oracle.expected_flags(5, 8, 3)
    assert buf.view(np.int64).tolist() == [3, 3, 3, 3, 3]
    buf = oracle.expected_flags(3, 128, 9)
    v = buf.view(np.int64)
    assert v[0] == 9 and v[16] == 9 and v[32] == 9
    assert np.count_nonzero(buf) == np.count_nonzero(oracle.expected_flags(3, 8, 9))
