"""The workloads, as concrete seeded synthetic inputs.

Stream ids: A shard s -> (1, s); B -> (2, 0); peer partial p -> (3, p);
tokens of source s -> (4, s); routing draws of source s -> (5, s); expert
weight e -> (6, e); producer order of epoch e -> (7, e); rows a peer returns
to the combine -> (8, q); ring all-reduce vector of rank r -> (10, r).  Seeds
are 1000 + i for the i-th workload below.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import (normal_bf16, normal_f32, small_int_bf16, small_int_f32, permutation, stream_key,
                  zipf_top2_routing, zipf_topk_gates)


@dataclass(frozen=True)
class AgGemmCfg:
    name: str
    ranks: int
    shard_m: int
    k: int
    n: int
    tile_m: int
    tile_n: int
    a_sigma: float
    b_sigma: float
    seed: int
    random_order: bool
    epochs: int = 1

    @property
    def m(self) -> int:
        return self.ranks * self.shard_m

    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


@dataclass(frozen=True)
class GemmRsCfg:
    name: str
    ranks: int
    m: int
    k: int
    n: int
    tile_m: int
    tile_n: int
    a_sigma: float
    b_sigma: float
    p_sigma: float
    seed: int
    rank: int = 0

    @property
    def block_m(self) -> int:
        return self.m // self.ranks

    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


@dataclass(frozen=True)
class DispatchCfg:
    name: str
    ranks: int
    tokens: int
    hidden: int
    n: int
    topk: int
    num_experts: int
    experts_per_rank: int
    zipf: float
    x_sigma: float
    w_sigma: float
    seed: int
    rank: int = 0
    tile_m: int = 256
    tile_n: int = 128

    @property
    def cap(self) -> int:
        return self.tokens * min(self.topk, self.experts_per_rank)


@dataclass(frozen=True)
class RingCfg:
    name: str
    ranks: int
    n: int        # fp32 elements per rank
    tile: int     # elements per signalled tile
    sigma: float
    seed: int


CONFIGS = {
    # R=2 ranks of 64x256 bf16 N(0,1) shards; B 256x256 N(0,1)/16; tile 32x32.
    "ag_r2_128x256x256": AgGemmCfg("ag_r2_128x256x256", 2, 64, 256, 256, 32, 32,
                                   1.0, 1.0 / 16, 1000, False, 1),
    # R=8 ranks of 1024x4096 shards (M=8192); B 4096x3584 N(0,0.02); tile 256.
    "ag_r8_8192x3584x4096": AgGemmCfg("ag_r8_8192x3584x4096", 8, 1024, 4096, 3584, 256, 256,
                                      1.0, 0.02, 1001, True, 5),
    # A 8192x1792 times B 1792x4096, R=8 row blocks of 1024, 7 fp32 peer partials.
    "rs_r8_8192x4096x1792": GemmRsCfg("rs_r8_8192x4096x1792", 8, 8192, 1792, 4096, 256, 256,
                                      1.0, 0.02, 1.0, 1002),
    # Decode-like skinny: R=8 shards of 16x8192 (M=128); B 8192x7168; tile 128.
    "ag_r8_skinny_128x7168x8192": AgGemmCfg("ag_r8_skinny_128x7168x8192", 8, 16, 8192, 7168, 128, 128,
                                            1.0, 0.02, 1003, True, 1),
    # MoE: 8 sources x 4096 tokens, hidden 4096, top-2 of 64 Zipf(1.1) experts,
    # 8 local experts with W 4096x1408.
    "a2a_r8_t4096_h4096_e64": DispatchCfg("a2a_r8_t4096_h4096_e64", 8, 4096, 4096, 1408, 2, 64, 8,
                                          1.1, 1.0, 0.02, 1004),
    # Ring all-reduce: 8 ranks x 32 MiB fp32 (8M elements, a gradient bucket),
    # N(0,1); chunks of 1M elements in 64 tiles of 16K (64 KiB).
    "ring_r8_n8m": RingCfg("ring_r8_n8m", 8, 8 << 20, 16 << 10, 1.0, 1005),
}


# ---------------------------------------------------------------- AG-GEMM inputs

def ag_inputs(cfg: AgGemmCfg, kind: str = "normal"):
    """(shards, b): R uint16 arrays [shard_m][k] and one uint16 [k][n].

    kind: "normal" (the workload), "smallint" (integers in [-4, 4], so fp32
    accumulation is exact) or "identity_b" (normal A, B[k][n] = [k == n]).
    """
    R, Ms, K, N = cfg.ranks, cfg.shard_m, cfg.k, cfg.n
    if kind == "smallint":
        shards = [small_int_bf16(cfg.seed, 1, s, (Ms, K)) for s in range(R)]
        b = small_int_bf16(cfg.seed, 2, 0, (K, N))
    else:
        shards = [normal_bf16(cfg.seed, 1, s, (Ms, K), cfg.a_sigma) for s in range(R)]
        if kind == "identity_b":
            b = np.zeros((K, N), dtype=np.uint16)
            d = min(K, N)
            b[np.arange(d), np.arange(d)] = 0x3F80  # 1.0 in bf16
        else:
            b = normal_bf16(cfg.seed, 2, 0, (K, N), cfg.b_sigma)
    return shards, b


def producer_order(seed: int, epoch: int, panels: int, batches: int, shuffle: bool = True,
                   kind: str = "panels") -> np.ndarray:
    """Order in which the producer moves flag units, int32 of length panels*batches.

    Unit u = panel * batches + batch.  kind="panels": a seeded permutation of
    the panels, each panel's K-batches in ascending order; kind="units": a
    seeded permutation of all units; shuffle=False: identity.
    """
    n_units = panels * batches
    if not shuffle:
        return np.arange(n_units, dtype=np.int32)
    if kind == "units":
        return permutation(seed, 7, epoch, n_units)
    pp = permutation(seed, 7, epoch, panels)
    return (pp[:, None].astype(np.int64) * batches + np.arange(batches)[None, :]).reshape(-1).astype(np.int32)


# ---------------------------------------------------------------- GEMM-RS inputs

def rs_inputs(cfg: GemmRsCfg, kind: str = "normal"):
    """(a, b, partials): uint16 [m][k], uint16 [k][n], list of R float32
    [m/R][n] peer partials (None at the own rank)."""
    M, K, N, R = cfg.m, cfg.k, cfg.n, cfg.ranks
    bm = M // R
    if kind == "smallint":
        a = small_int_bf16(cfg.seed, 1, 0, (M, K))
        b = small_int_bf16(cfg.seed, 2, 0, (K, N))
        parts = [None if p == cfg.rank else small_int_f32(cfg.seed, 3, p, (bm, N), -64, 64)
                 for p in range(R)]
    else:
        a = normal_bf16(cfg.seed, 1, 0, (M, K), cfg.a_sigma)
        b = normal_bf16(cfg.seed, 2, 0, (K, N), cfg.b_sigma)
        parts = [None if p == cfg.rank else
                 normal_f32(stream_key(cfg.seed, 3, p), bm * N, cfg.p_sigma).reshape(bm, N)
                 for p in range(R)]
    return a, b, parts


# ---------------------------------------------------------------- dispatch inputs

def dispatch_inputs(cfg: DispatchCfg, kind: str = "normal"):
    """(x, topk, w): R uint16 [tokens][hidden], R int32 [tokens][topk] global
    expert ids, uint16 [experts_per_rank][hidden][n] local expert weights."""
    R, T, H, N = cfg.ranks, cfg.tokens, cfg.hidden, cfg.n
    if kind == "smallint":
        x = [small_int_bf16(cfg.seed, 4, s, (T, H)) for s in range(R)]
        w = np.stack([small_int_bf16(cfg.seed, 6, e, (H, N)) for e in range(cfg.experts_per_rank)])
    else:
        x = [normal_bf16(cfg.seed, 4, s, (T, H), cfg.x_sigma) for s in range(R)]
        w = np.stack([normal_bf16(cfg.seed, 6, e, (H, N), cfg.w_sigma) for e in range(cfg.experts_per_rank)])
    topk = [zipf_top2_routing(cfg.seed, s, T, cfg.num_experts, cfg.topk, cfg.zipf) for s in range(R)]
    return x, topk, w


# ---------------------------------------------------------------- combine inputs

def combine_inputs(cfg: DispatchCfg, kind: str = "normal"):
    """(gates, ret_in) for the combine at rank cfg.rank: gates float32
    [tokens][topk] of this rank's own tokens (routing of source cfg.rank),
    and for every peer q != rank the rows q returns for those tokens, float32
    [cap][n] (None at the own rank): what q's experts computed for the
    tokens it received from this rank, in q's slice order."""
    R, T, N = cfg.ranks, cfg.tokens, cfg.n
    cap = cfg.cap
    gates = zipf_topk_gates(cfg.seed, cfg.rank, T, cfg.num_experts, cfg.topk, cfg.zipf)
    if kind == "smallint":
        # dyadic gates (1..4)/4 and small integers: every product and sum exact in fp32
        gates = (small_int_f32(cfg.seed, 9, cfg.rank, (T, cfg.topk), 1, 4) / 4).astype(np.float32)
        ret = [None if q == cfg.rank else small_int_f32(cfg.seed, 8, q, (cap, N), -16, 16) for q in range(R)]
    else:
        ret = [None if q == cfg.rank else normal_f32(stream_key(cfg.seed, 8, q), cap * N, 1.0).reshape(cap, N)
               for q in range(R)]
    return gates, ret


# ---------------------------------------------------------------- ring all-reduce inputs

def ring_inputs(cfg: RingCfg, kind: str = "normal"):
    """R float32 [n] vectors, one per rank."""
    if kind == "smallint":
        return [small_int_f32(cfg.seed, 10, r, (cfg.n,), -1000, 1000) for r in range(cfg.ranks)]
    return [normal_f32(stream_key(cfg.seed, 10, r), cfg.n, cfg.sigma) for r in range(cfg.ranks)]
