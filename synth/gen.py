"""Counter-based generators (numpy, vectorised, chunked).

Every value is a pure function of (seed, tensor id, sub id, element index),
so any slice of any tensor can be regenerated without drawing the rest.

* Bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014).  Element i of a stream with key k is
  mix(k + (i + 1) * GOLDEN), the i-th output of a SplitMix64 generator whose
  state starts at k.
* Uniforms: the top 53 bits, centred: (x >> 11) + 0.5, times 2**-53, so a
  uniform is never 0 or 1.
* Normals: Box and Muller (1958), cosine branch only; element i uses the
  uniform pair (2i, 2i + 1) of its stream.
* bf16: the float32 value rounded to nearest, ties to even, on its bits.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20

_MASK64 = (1 << 64) - 1


def _mix_py(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int, sub_id: int = 0) -> int:
    """64-bit key of the stream (seed, tensor_id, sub_id)."""
    k = _mix_py(seed * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019)
    k = _mix_py(k ^ ((tensor_id & 0xFFFF) << 40) ^ (sub_id & 0xFFFFFFFFFF))
    return k


def raw_u64(key: int, start: int, count: int) -> np.ndarray:
    """Elements [start, start + count) of the stream as uint64."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * GOLDEN
    return _mix(z)


def uniform(key: int, start: int, count: int) -> np.ndarray:
    """Uniforms in (0, 1), float64."""
    x = raw_u64(key, start, count) >> np.uint64(11)
    return (x.astype(np.float64) + 0.5) * (2.0 ** -53)


def normal_f32(key: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """`count` normals N(0, sigma^2), rounded once to float32."""
    out = np.empty(count, dtype=np.float32)
    for c0 in range(0, count, _CHUNK):
        n = min(_CHUNK, count - c0)
        u = uniform(key, 2 * c0, 2 * n)
        u1, u2 = u[0::2], u[1::2]
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
        out[c0:c0 + n] = (z * sigma).astype(np.float32)
    return out


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: int, tensor_id: int, sub_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits (uint16 array of `shape`) of N(0, sigma^2) draws."""
    count = int(np.prod(shape))
    key = stream_key(seed, tensor_id, sub_id)
    out = np.empty(count, dtype=np.uint16)

    def chunk(c0):
        n = min(_CHUNK, count - c0)
        u = uniform(key, 2 * c0, 2 * n)
        z = np.sqrt(-2.0 * np.log(u[0::2])) * np.cos(2.0 * np.pi * u[1::2])
        out[c0:c0 + n] = bf16_rne((z * sigma).astype(np.float32))

    starts = range(0, count, _CHUNK)
    if count > _CHUNK:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(chunk, starts))
    else:
        for c0 in starts:
            chunk(c0)
    return out.reshape(shape)


def small_int_f32(seed: int, tensor_id: int, sub_id: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """float32 integers drawn uniformly from [lo, hi]."""
    count = int(np.prod(shape))
    key = stream_key(seed, tensor_id, sub_id)
    span = hi - lo + 1
    vals = np.empty(count, dtype=np.float32)
    for c0 in range(0, count, _CHUNK):
        n = min(_CHUNK, count - c0)
        u = uniform(key, c0, n)
        vals[c0:c0 + n] = (lo + np.floor(u * span)).astype(np.float32)
    return vals.reshape(shape)


def small_int_bf16(seed: int, tensor_id: int, sub_id: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from [lo, hi] (exact in bf16 for |v| <= 256)."""
    return bf16_rne(small_int_f32(seed, tensor_id, sub_id, shape, lo, hi))


def permutation(seed: int, tensor_id: int, sub_id: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates shuffle of range(n) (Durstenfeld's form), int32."""
    perm = np.arange(n, dtype=np.int32)
    if n <= 1:
        return perm
    u = uniform(stream_key(seed, tensor_id, sub_id), 0, n)
    for i in range(n - 1, 0, -1):
        j = int(u[i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def zipf_top2_routing(seed: int, source: int, tokens: int, num_experts: int = 64,
                      topk: int = 2, exponent: float = 1.1) -> np.ndarray:
    """Top-k expert ids per token, int32 [tokens][topk].

    Expert e has popularity p_e proportional to (e + 1) ** -exponent; a token
    picks `topk` distinct experts by sampling without replacement in
    proportion to p (Gumbel top-k: the k largest of ln p_e + G, with
    G = -ln(-ln U)).  Equal keys go to the lower expert id.
    """
    logp = -exponent * np.log(np.arange(1, num_experts + 1, dtype=np.float64))
    u = uniform(stream_key(seed, 5, source), 0, tokens * num_experts).reshape(tokens, num_experts)
    keys = logp[None, :] - np.log(-np.log(u))
    order = np.argsort(-keys, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :topk].astype(np.int32))


def zipf_topk_gates(seed: int, source: int, tokens: int, num_experts: int = 64, topk: int = 2,
                    exponent: float = 1.1) -> np.ndarray:
    """Gate weights of the routing `zipf_top2_routing` draws, float32
    [tokens][topk]: the chosen experts' keys (ln p_e + G, the same draws)
    taken as router logits and normalised by a softmax over the top-k."""
    logp = -exponent * np.log(np.arange(1, num_experts + 1, dtype=np.float64))
    u = uniform(stream_key(seed, 5, source), 0, tokens * num_experts).reshape(tokens, num_experts)
    keys = logp[None, :] - np.log(-np.log(u))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :topk]
    top = np.take_along_axis(keys, order, axis=1)
    e = np.exp(top - top.max(axis=1, keepdims=True))
    return np.ascontiguousarray((e / e.sum(axis=1, keepdims=True)).astype(np.float32))
