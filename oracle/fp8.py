"""FP8 (e4m3) dispatch and grouped GEMM (TEST INFRASTRUCTURE ONLY).

The Aboleth README measures its compiled MoE dispatch and combine on "one
FP8 layer" and says no more about the format.  The reading taken here:

  - tokens and expert weights travel and multiply as OCP FP8 E4M3 codes
    (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; subnormals
    below 2^-6; no infinities; S.1111.111 is NaN; the largest finite value
    is 448), which gfx950's matrix cores take directly;
  - one float32 scale per row: a token row x (or a weight column, stored as
    a row of the transposed weight) with amax = max |x| gets
    scale = amax / 448 and codes q = E4M3(min(max(x * (448 / amax), -448),
    448)), rounded to nearest, ties to the even code, both quotients in
    float32; a row of zeros gets scale 1 and zero codes;
  - the dispatch moves the codes and the row's scale (the bf16 layout, with
    rows of `hidden` bytes);
  - the grouped GEMM computes y[i][n] = (sum_k q_x[i][k] q_w[n][k]) * sx[i]
    * sw[n], the sum exact (float64 here).

`e4m3_decode` is the format's definition; `e4m3_encode` rounds float32
values by the rule above.  The pins hold the encoder to a brute-force search
over all 256 codes and the decoder to the format's stated values.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f32
from .dispatch import dispatch_layout

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return sign * v


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of float32 values already within [-448, 448]: round to
    nearest, ties to the even code (even mantissa)."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("values must be finite and within +-448")
    a = np.abs(v)
    # exponent of the binade (a = f * 2^x with f in [0.5, 1): floor(log2 a) =
    # x - 1, exactly), clamped to the subnormal range below 2^-6
    _, x2 = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(x2.astype(np.int64) - 1, -6)
    ulp = np.ldexp(1.0, (e - 3).astype(np.int32))  # 3 mantissa bits
    steps = a / ulp                                 # exact: a power-of-two scaling
    lo = np.floor(steps)
    frac = steps - lo
    up = (frac > 0.5) | ((frac == 0.5) & (lo % 2 == 1))
    n = (lo + up).astype(np.int64)                  # multiple of ulp, in [8, 16] (normal) or [0, 8]
    # n == 16 carries into the next binade
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    normal = (e > -6) | (n >= 8)
    code = np.where(normal, ((e + 7) << 3) | (n - 8), n)
    out = np.where(a == 0, 0, code)
    return (out | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows(rows_bf16):
    """(codes uint8 [rows][cols], scales float32 [rows]) of bf16 rows (uint16
    bit patterns), by the per-row rule of the module docstring."""
    x = bf16_to_f32(np.asarray(rows_bf16))
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    amax = amax.astype(np.float32)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1))
    scale = np.where(pos, safe / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    inv = np.where(pos, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(v), scale


def dispatch_fp8(x8, x_scale, topk_idx, rank: int, experts_per_rank: int, cap: int):
    """The dispatch of FP8 rows to `rank`: (recv_x8 uint8 [R][cap][hidden],
    recv_scale float32 [R][cap], recv_src, recv_count), the layout of the
    bf16 dispatch (oracle.dispatch) with each row's scale beside it."""
    R = len(x8)
    H = x8[0].shape[1]
    recv_x8 = np.zeros((R, cap, H), dtype=np.uint8)
    recv_scale = np.zeros((R, cap), dtype=np.float32)
    recv_src = np.zeros((R, cap), dtype=np.int32)
    recv_count = np.zeros((R, experts_per_rank), dtype=np.int32)
    for s in range(R):
        e_loc, tok = dispatch_layout(topk_idx[s], rank, experts_per_rank)
        if len(tok) > cap:
            raise ValueError("slice capacity exceeded")
        recv_x8[s, :len(tok)] = np.asarray(x8[s])[tok]
        recv_scale[s, :len(tok)] = np.asarray(x_scale[s])[tok]
        recv_src[s, :len(tok)] = tok
        recv_count[s] = np.bincount(e_loc, minlength=experts_per_rank)
    return recv_x8, recv_scale, recv_src, recv_count


def grouped_gemm_fp8(recv_x8, recv_scale, recv_count, w8, w_scale):
    """y float64 [R][cap][n]: every received row of local expert e times the
    transposed FP8 weight w8[e] ([n][hidden] codes) with both row scales;
    rows past a slice's count are zero."""
    R, cap, _ = recv_x8.shape
    E, N, _ = w8.shape
    y = np.zeros((R, cap, N))
    wd = [e4m3_decode(w8[e]) for e in range(E)]
    for s in range(R):
        r0 = 0
        for e in range(E):
            c = int(recv_count[s][e])
            if c:
                xd = e4m3_decode(recv_x8[s, r0:r0 + c])
                y[s, r0:r0 + c] = (xd @ wd[e].T) * recv_scale[s, r0:r0 + c, None].astype(np.float64) \
                    * w_scale[e][None, :].astype(np.float64)
            r0 += c
    return y
