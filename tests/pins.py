"""Independent checks that pin the oracle to facts outside it.

Each returns (ok, detail) so that the mutation tests can assert that a
planted mistake makes a check fail.  None of them calls the oracle.
"""

from __future__ import annotations

import math

import numpy as np


def _decode_one(v: int) -> float:
    """One bf16 bit pattern -> float, by the IEEE layout written out (sign,
    8-bit exponent, 7-bit fraction), independently of the oracle's decoder."""
    sign = -1.0 if v & 0x8000 else 1.0
    exp = (v >> 7) & 0xFF
    frac = v & 0x7F
    if exp == 0:
        return sign * frac * 2.0 ** (-133)
    if exp == 0xFF:
        return float("nan") if frac else sign * float("inf")
    return sign * (1.0 + frac / 128.0) * 2.0 ** (exp - 127)


_TABLE = None


def decode_table() -> np.ndarray:
    global _TABLE
    if _TABLE is None:
        _TABLE = np.array([_decode_one(v) for v in range(65536)], dtype=np.float64)
    return _TABLE


def decode_np(u16) -> np.ndarray:
    """bf16 bits -> float64 array via the 65536-entry table."""
    return decode_table()[np.asarray(u16, dtype=np.uint16)]


def decode_bf16(u16) -> list:
    return decode_np(u16).reshape(-1).tolist()


def fsum_entry(a_row_u16, b_col_u16):
    """(correctly rounded exact sum, sum of |products|) of one dot product."""
    a = decode_bf16(a_row_u16)
    b = decode_bf16(b_col_u16)
    prods = [x * y for x, y in zip(a, b)]  # each exact: 8-bit x 8-bit significands
    return math.fsum(prods), math.fsum(abs(p) for p in prods)


def check_entries_fsum(c, a_u16, b_u16, rows, cols, row_of=None):
    """c[i] (or c[rows[i], cols[i]] for 2-D c) against exact sums, within the
    float64 summation bound K * 2**-53 * sum|ab| (plus one ulp of the exact sum)."""
    a_u16 = np.asarray(a_u16)
    b_u16 = np.asarray(b_u16)
    k = a_u16.shape[1]
    worst = 0.0
    for i, (r, cc) in enumerate(zip(rows, cols)):
        got = float(c[i]) if np.ndim(c) == 1 else float(c[r, cc])
        ar = a_u16[r if row_of is None else row_of(r)]
        exact, mag = fsum_entry(ar, b_u16[:, cc])
        bound = k * 2.0 ** -53 * mag + abs(exact) * 2.0 ** -52
        if abs(got - exact) > bound:
            return False, f"entry ({r},{cc}): got {got!r}, exact {exact!r}, bound {bound:.3e}"
        worst = max(worst, abs(got - exact))
    return True, f"max err {worst:.3e}"


def brute_gemm(a_u16, b_u16):
    """Triple loop over Python floats with math.fsum per entry."""
    a = np.asarray(a_u16)
    b = np.asarray(b_u16)
    m, k = a.shape
    n = b.shape[1]
    A = [decode_bf16(a[i]) for i in range(m)]
    B = [decode_bf16(b[:, j]) for j in range(n)]
    return [[math.fsum(A[i][t] * B[j][t] for t in range(k)) for j in range(n)] for i in range(m)]


def bf16_ints(u16) -> np.ndarray:
    """Integer values of bf16 bits that hold small integers, as int64."""
    v = decode_np(u16)
    iv = np.rint(v).astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v), "not integer-valued"
    return iv
