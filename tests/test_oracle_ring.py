"""Pins of the ring all-reduce oracle (CPU): the float64 sum within the
float32 rounding bound of a ring-ordered sum, exact small integers, one
result on every rank, the ring's summation order on inputs where the order
decides the bits, the trivial rank counts, and planted mistakes."""

import numpy as np
import pytest

import oracle
import synth

U32 = 2.0 ** -24  # unit roundoff of float32


def _inputs(R, n, seed, kind="normal"):
    if kind == "smallint":
        return [synth.small_int_f32(seed, 10, r, (n,), -1000, 1000) for r in range(R)]
    return [synth.normal_f32(synth.stream_key(seed, 10, r), n, 1.0) for r in range(R)]


def _within_ring_bound(outs, inputs):
    """|out - sum| <= (R - 1) u sum|x| (+ a hair for the bound's second-order
    terms): what a sequential float32 sum over R terms can be off by."""
    R = len(inputs)
    ref = oracle.allreduce_sum(inputs)
    mag = np.sum(np.abs(np.stack(inputs).astype(np.float64)), axis=0)
    tol = (R - 1) * U32 * mag * (1 + 1e-6) + 1e-300
    return all(np.all(np.abs(o.astype(np.float64) - ref) <= tol) for o in outs)


@pytest.mark.parametrize("R,n,seed", [(2, 64, 1), (3, 101, 2), (5, 1000, 3), (8, 4099, 4), (8, 8, 5), (7, 3, 6)])
def test_sum_within_float32_bound_and_identical_on_every_rank(R, n, seed):
    x = _inputs(R, n, seed)
    outs = oracle.ring_allreduce(x)
    assert _within_ring_bound(outs, x)
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("R,n", [(2, 10), (4, 77), (8, 1024)])
def test_small_integers_are_exact(R, n):
    x = _inputs(R, n, 7, "smallint")
    ref = np.sum(np.stack(x).astype(np.int64), axis=0)
    for o in oracle.ring_allreduce(x):
        assert np.array_equal(o.astype(np.int64), ref)


def _order_case():
    """Three ranks, chunks of two elements; in chunk c the rank two places
    after c holds 2^24 and the other two hold 1.  Summed in ring order from
    chunk c's first owner, (1 + 1) + 2^24 = 2^24 + 2 exactly; any other start
    or direction adds 1 to 2^24 first, which rounds back to 2^24 (ties to
    even), and ends at 2^24."""
    R, n = 3, 6
    x = [np.ones(n, dtype=np.float32) for _ in range(R)]
    for c, (lo, hi) in enumerate(oracle.ring_chunk_bounds(n, R)):
        x[(c + 2) % R][lo:hi] = 2.0 ** 24
    return x


def test_ring_order_decides_the_bits():
    outs = oracle.ring_allreduce(_order_case())
    for o in outs:
        assert np.all(o == np.float32(2.0 ** 24 + 2))


def test_planted_reverse_direction_is_caught():
    # the ring run the other way round: relabel rank r as -r
    x = _order_case()
    rev = [x[(-r) % 3] for r in range(3)]
    outs = oracle.ring_allreduce(rev)
    assert not all(np.all(o == np.float32(2.0 ** 24 + 2)) for o in outs)


def test_planted_dropped_rank_and_shifted_chunk_are_caught():
    x = _inputs(5, 1000, 8)
    good = oracle.ring_allreduce(x)
    dropped = [o - x[3] for o in good]  # one rank's contribution missing
    assert not _within_ring_bound(dropped, x)
    shifted = [np.roll(o, 200) for o in good]  # every chunk delivered one chunk over
    assert not _within_ring_bound(shifted, x)


def test_one_rank_is_the_identity_and_empty_is_empty():
    x = _inputs(1, 33, 9)
    (o,) = oracle.ring_allreduce(x)
    assert np.array_equal(o.view(np.uint32), x[0].view(np.uint32))
    outs = oracle.ring_allreduce([np.zeros(0, np.float32)] * 4)
    assert all(o.shape == (0,) for o in outs)


@pytest.mark.parametrize("n,R", [(0, 3), (1, 8), (7, 8), (16, 8), (1001, 7), (4096, 8)])
def test_chunks_cover_the_vector_once_from_even_starts(n, R):
    b = oracle.ring_chunk_bounds(n, R)
    assert len(b) == R
    covered = np.zeros(n, dtype=np.int64)
    for lo, hi in b:
        assert lo % 2 == 0 or lo == n
        covered[lo:hi] += 1
    assert np.all(covered == 1)
