"""Pins of the FP8 (E4M3) oracle (CPU): the decoder against the format's
stated values, the encoder against a brute-force nearest-code search with
ties to even, the per-row quantizer's scale and error bound, the FP8
dispatch against the bf16 layout, and the FP8 grouped GEMM against exact
sums."""

import math

import numpy as np
import pytest

import oracle
import synth

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decoder_matches_the_format():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    stated = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
              0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for c, v in stated.items():
        assert d[c] == v, hex(c)
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert len(FINITE) == 254
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E are increasing
    # each normal binade holds 8 evenly spaced values, one ulp = 2^(e-10)
    for e in range(1, 16):
        vals = d[e * 8:(e + 1) * 8] if e < 15 else d[120:127]
        assert np.allclose(np.diff(vals), 2.0 ** (e - 10))


def _brute(v):
    vals = oracle.e4m3_decode(FINITE)
    out = []
    for x in np.asarray(v, dtype=np.float64):
        dist = np.abs(vals - x)
        best = dist.min()
        cands = FINITE[dist == best]
        if len(cands) > 1:  # a tie: the even code (even mantissa), sign of x
            cands = cands[(cands & 1) == 0]
            cands = cands[(cands >= 0x80) == (x < 0)] if x != 0 else cands[:1]
        out.append(int(cands[0]))
    return np.array(out, dtype=np.uint8)


def test_encoder_is_the_nearest_code_with_ties_to_even():
    rng = np.random.default_rng(5)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 3000))
    v = (mags * rng.choice([-1.0, 1.0], 3000)).astype(np.float32)
    vals = np.sort(oracle.e4m3_decode(FINITE[FINITE < 0x80]))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in float32: ties
    v = np.concatenate([v, mids, -mids, np.float32([0, 448, -448, 2.0 ** -10, 2.0 ** -11])])
    got = oracle.e4m3_encode(v)
    want = _brute(v)
    zero = v == 0
    assert np.array_equal(got[~zero], want[~zero])
    assert np.all(oracle.e4m3_decode(got[zero]) == 0)


def test_encoder_round_trips_every_finite_code():
    d = oracle.e4m3_decode(FINITE).astype(np.float32)
    got = oracle.e4m3_encode(d)
    assert np.array_equal(got[d != 0], FINITE[d != 0])


def test_quantizer_scale_and_error_bound():
    x = synth.normal_bf16(3, 11, 0, (64, 300))
    x[5] = 0  # a zero row
    q, s = oracle.quantize_rows(x)
    xf = oracle.bf16_to_f64(x)
    amax = np.abs(xf).max(axis=1)
    assert s[5] == 1 and not q[5].any()
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448)).astype(np.float32))
    dq = oracle.e4m3_decode(q) * s[:, None].astype(np.float64)
    # the largest element of a row lands on +-448
    assert np.all(np.abs(oracle.e4m3_decode(q[nz])).max(axis=1) == 448)
    # half an ulp of the code (2^-4 relative for normals, 2^-10 absolute below
    # 2^-6), in units of the scale, plus float32 rounding of x * (448 / amax)
    bound = s[:, None] * (2.0 ** -4 * np.abs(xf) / s[:, None] + 2.0 ** -10) + 1e-6 * np.abs(xf)
    assert np.all(np.abs(dq - xf) <= bound)


def test_fp8_dispatch_is_the_bf16_layout_with_scales():
    cfg = synth.DispatchCfg("fp8pin", 3, 40, 32, 16, 2, 6, 2, 1.1, 1.0, 0.25, 9, 1)
    x, topk, _ = synth.dispatch_inputs(cfg)
    q = [oracle.quantize_rows(v) for v in x]
    rx8, rs8, src8, rc8 = oracle.dispatch_fp8([a for a, _ in q], [b for _, b in q], topk, 1, 2, cfg.cap)
    rx, src, rc = oracle.dispatch(x, topk, 1, 2, cfg.cap)
    assert np.array_equal(src8, src) and np.array_equal(rc8, rc)
    for s in range(3):
        n = int(rc[s].sum())
        assert np.array_equal(rx8[s, :n], q[s][0][src[s, :n]])
        assert np.array_equal(rs8[s, :n], q[s][1][src[s, :n]])
        assert not rx8[s, n:].any() and not rs8[s, n:].any()


def _gemm_case(kind):
    rng = np.random.default_rng(7)
    R, cap, H, E, N = 2, 12, 64, 2, 24
    counts = np.array([[5, 4], [0, 7]], dtype=np.int32)
    if kind == "smallint":
        codes = oracle.e4m3_encode(np.arange(-8, 9, dtype=np.float32))
        rx8 = rng.choice(codes, (R, cap, H)).astype(np.uint8)
        w8 = rng.choice(codes, (E, N, H)).astype(np.uint8)
        rs = np.ones((R, cap), np.float32)
        ws = np.ones((E, N), np.float32)
    else:
        rx8 = rng.choice(FINITE, (R, cap, H)).astype(np.uint8)
        w8 = rng.choice(FINITE, (E, N, H)).astype(np.uint8)
        rs = rng.uniform(0.001, 0.01, (R, cap)).astype(np.float32)
        ws = rng.uniform(0.001, 0.01, (E, N)).astype(np.float32)
    return rx8, rs, counts, w8, ws


def test_fp8_grouped_gemm_against_exact_sums():
    rx8, rs, rc, w8, ws = _gemm_case("normal")
    y = oracle.grouped_gemm_fp8(rx8, rs, rc, w8, ws)
    xd, wd = oracle.e4m3_decode(rx8), oracle.e4m3_decode(w8)
    for s in range(2):
        r0 = 0
        for e in range(2):
            for j in range(r0, r0 + rc[s][e]):
                for n in (0, 7, 23):
                    exact = math.fsum(xd[s, j] * wd[e, n]) * float(rs[s, j]) * float(ws[e, n])
                    assert abs(y[s, j, n] - exact) <= 1e-12 * max(1.0, abs(exact))
            r0 += rc[s][e]
        assert not y[s, int(rc[s].sum()):].any()


def test_fp8_grouped_gemm_small_integers_exact_and_transposed_weight_caught():
    rx8, rs, rc, w8, ws = _gemm_case("smallint")
    y = oracle.grouped_gemm_fp8(rx8, rs, rc, w8, ws)
    xi = oracle.e4m3_decode(rx8).astype(np.int64)
    wi = oracle.e4m3_decode(w8).astype(np.int64)
    assert np.array_equal(y[0, :5], (xi[0, :5] @ wi[0].T).astype(np.float64))
    assert np.array_equal(y[1, :7], (xi[1, :7] @ wi[1].T).astype(np.float64))
    # a weight read as [hidden][n] instead of [n][hidden] does not give these sums
    square = w8[:, :, :24]
    bad = oracle.e4m3_decode(rx8[0, :5, :24]) @ oracle.e4m3_decode(square[0])
    good = oracle.e4m3_decode(rx8[0, :5, :24]) @ oracle.e4m3_decode(square[0]).T
    assert not np.array_equal(bad, good)


@pytest.mark.parametrize("bad", [449.0, -500.0, float("nan")])
def test_encoder_refuses_values_out_of_range(bad):
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.float32([bad]))
