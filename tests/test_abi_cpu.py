"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and its host logic (plans, validation, sizes, schedule) behaves.  Nothing here
reaches a kernel launch: every call either touches no device or fails its
argument checks first."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ovl.h")


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for want in ("ag_gemm_plan", "ag_gemm_run", "gemm_rs_run", "a2a_dispatch_grouped_gemm_run",
                 "ovl_flags_reset", "ovl_check"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ovl().lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(ovl().EXPORTS) <= set(declared_functions())


def test_strerror():
    o = ovl()
    assert o.strerror(0) == "ok"
    assert "epoch" in o.strerror(o.OVL_EEPOCH)
    assert o.strerror(-99) == "unknown status"


@pytest.mark.parametrize("args,status", [
    ((0, 0, 64, 256, 256, 32, 32, 0, 8), "OVL_EINVAL"),        # no ranks
    ((2, 2, 64, 256, 256, 32, 32, 0, 8), "OVL_EINVAL"),        # rank out of range
    ((17, 0, 64, 256, 256, 32, 32, 0, 8), "OVL_EUNSUPPORTED"),  # more than 16 ranks
    ((2, 0, 0, 256, 256, 32, 32, 0, 8), "OVL_ESHAPE"),         # empty shard
    ((2, 0, 64, 250, 256, 32, 32, 0, 8), "OVL_EALIGN"),        # K not a multiple of 8
    ((2, 0, 64, 256, 252, 32, 32, 0, 8), "OVL_EALIGN"),        # N not a multiple of 8
    ((2, 0, 64, 256, 256, 32, 30, 1, 8), "OVL_EALIGN"),        # K-tile not a multiple of 8
    ((2, 0, 64, 256, 256, 32, 32, 0, 12), "OVL_EALIGN"),       # flag stride
    ((2, 0, 64, 256, 256, 32, 32, -1, 8), "OVL_ESHAPE"),       # negative tiles per flag
    ((8, 0, 1 << 18, 4096, 256, 256, 256, 0, 8), "OVL_EUNSUPPORTED"),  # gathered operand > 1 GiB
    ((2, 0, 64, 256, 256, 32, 32, 0, 8, 17), "OVL_EINVAL"),     # more than 16 producers per unit
    ((2, 0, 64, 256, 256, 32, 32, 0, 8, -1), "OVL_EINVAL"),     # negative producers per unit
])
def test_plan_rejects(args, status):
    o = ovl()
    with pytest.raises(o.OvlError) as e:
        o.ag_gemm_plan(*args)
    assert e.value.status == getattr(o, status)


@pytest.mark.parametrize("name,tpf,stride", [
    ("ag_r2_128x256x256", 0, 8), ("ag_r2_128x256x256", 1, 128),
    ("ag_r8_8192x3584x4096", 1, 8), ("ag_r8_skinny_128x7168x8192", 4, 64),
])
def test_plan_sizes_match_the_flag_unit_definition(name, tpf, stride):
    cfg = synth.CONFIGS[name]
    p = ovl().ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, tpf, stride)
    units, _, _ = oracle.ag_flag_units(cfg.ranks, cfg.shard_m, cfg.k, cfg.tile_m, cfg.tile_n, tpf)
    assert p.num_units == units
    assert p.flags_bytes == units * stride
    assert p.workspace_bytes >= ovl().ERROR_RECORD_BYTES


@pytest.mark.parametrize("name,tpf,W", [("ag_r8_8192x3584x4096", 1, 4), ("ag_r8_skinny_128x7168x8192", 4, 2),
                                        ("ag_r2_128x256x256", 1, 16)])
def test_split_unit_plans_add_one_counter_per_unit(name, tpf, W):
    cfg = synth.CONFIGS[name]
    o = ovl()
    one = o.ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, tpf, 8)
    many = o.ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, tpf, 8, W)
    assert many.num_units == one.num_units and many.flags_bytes == one.flags_bytes
    assert many.workspace_bytes == one.workspace_bytes + -(-one.num_units * 8 // 256) * 256


def test_ragged_plan_sizes():
    p = ovl().ag_gemm_plan(3, 1, 100, 200, 136, 48, 40, 2, 8)
    assert p.num_units == oracle.ag_flag_units(3, 100, 200, 48, 40, 2)[0] == 27


def _consumer_order(plan, order):
    lib = ovl().lib()
    lib.ag_gemm_consumer_order.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ag_gemm_consumer_order.restype = ctypes.c_int32
    lib.ag_gemm_row_tiles.argtypes = [ctypes.c_void_p]
    lib.ag_gemm_row_tiles.restype = ctypes.c_int32
    T = lib.ag_gemm_row_tiles(plan.handle)
    out = np.zeros(T, dtype=np.int32)
    arg = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    st = lib.ag_gemm_consumer_order(plan.handle, None if arg is None else arg.ctypes.data, out.ctypes.data)
    return st, out


def _golden(name):
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(x) for x in line.split()])
    return rows


def test_consumer_order_follows_the_swizzle_golden():
    # 8 ranks x 4 panels of 256 rows (32 row tiles).  With producers moving
    # the shards in the order rank, rank+1, ..., the consumer order is the
    # pages' swizzle pid -> (pid + rank * tiles_per_pe) % total_tiles.
    cfg = synth.CONFIGS["ag_r8_8192x3584x4096"]
    golden = _golden("swizzle_start_tile.txt")
    for rank in range(8):
        plan = ovl().ag_gemm_plan(8, rank, cfg.shard_m, cfg.k, cfg.n, 256, 256, 0, 8)
        shards = [(rank + j) % 8 for j in range(8)]
        order = np.array([s * 4 + p for s in shards for p in range(4)], dtype=np.int32)
        st, got = _consumer_order(plan, order)
        assert st == 0
        assert got.tolist() == [(pid + rank * 4) % 32 for pid in range(32)]
        for r, pid, swz in golden:
            if r == rank:
                assert got[pid] == swz


def test_consumer_order_is_a_permutation_with_own_rows_first():
    plan = ovl().ag_gemm_plan(4, 2, 192, 384, 320, 64, 64, 2, 8)
    order = synth.producer_order(5, 1, 4 * 3, plan.num_units // 12, True, "units")
    st, got = _consumer_order(plan, order)
    assert st == 0
    T = len(got)
    assert sorted(got.tolist()) == list(range(T))
    own = [rt for rt in range(T) if rt * 128 >= 2 * 192 and min((rt + 1) * 128, 768) <= 3 * 192]
    assert got[:len(own)].tolist() == own


def test_consumer_order_rejects_bad_units():
    plan = ovl().ag_gemm_plan(2, 0, 64, 256, 256, 32, 32, 0, 8)
    st, _ = _consumer_order(plan, np.array([0, 1, 2, 9], dtype=np.int32))
    assert st == ovl().OVL_EINVAL


def test_run_argument_errors_come_before_any_device_work():
    o = ovl()
    plan = o.ag_gemm_plan(2, 0, 64, 256, 256, 32, 32, 0, 8)
    # Null shard array, null workspace: rejected before the device is touched.
    st = o.lib().ag_gemm_run(plan.handle, None, None, None, None, None, None, 1, None, None, None)
    assert st == o.OVL_EINVAL
    desc = o.gemm_rs_desc(8, 0, 8192, 4096, 1792, tile_m=128)
    st = o.gemm_rs_run(desc, 16, 16, [16] * 8, [16] * 8, 16, 16, 16, 16, 1, raise_on_error=False, stream=0)
    assert st == o.OVL_EUNSUPPORTED
    desc = o.gemm_rs_desc(3, 0, 1000, 256, 256)  # m not a multiple of ranks
    st = o.gemm_rs_run(desc, 16, 16, [16] * 3, [16] * 3, 16, 16, 16, 16, 1, raise_on_error=False, stream=0)
    assert st == o.OVL_ESHAPE
    ad = o.a2a_desc(17, 0, 16, 64, 64, 2, 17 * 2, 2)
    st = o.a2a_dispatch_grouped_gemm_run(ad, [16] * 17, [16] * 17, 16, 16, 16, 16, 16, 16, 16, 1,
                                         raise_on_error=False, stream=0)
    assert st == o.OVL_EUNSUPPORTED
    ad = o.a2a_desc(2, 0, 16, 60, 64, 2, 4, 2)  # hidden not a multiple of 8
    st = o.a2a_dispatch_grouped_gemm_run(ad, [16] * 2, [16] * 2, 16, 16, 16, 16, 16, 16, 16, 1,
                                         raise_on_error=False, stream=0)
    assert st == o.OVL_EALIGN


@pytest.mark.parametrize("tile", [(128, 256), (256, 128), (512, 512), (64, 64), (0, 256), (0, 0)])
def test_gemm_rs_refuses_tiles_it_does_not_implement(tile):
    """gemm_rs_run implements 256 x 256 and 128 x 128 tiles; every other pair
    is refused with OVL_EUNSUPPORTED before any device work, and the size
    queries return 0 for it."""
    o = ovl()
    desc = o.gemm_rs_desc(8, 0, 8192, 4096, 1792, tile_m=tile[0], tile_n=tile[1])
    st = o.gemm_rs_run(desc, 16, 16, [16] * 8, [16] * 8, 16, 16, 16, 16, 1, raise_on_error=False, stream=0)
    assert st == o.OVL_EUNSUPPORTED
    assert o.gemm_rs_flags_bytes(desc) == 0 and o.gemm_rs_workspace_bytes(desc) == 0


def test_gemm_rs_tile_sizes():
    """Flag and workspace sizes follow the tile: one flag per tile of each
    block (8192 x 4096 over 8 ranks: 4 x 16 tiles of 256, 8 x 32 of 128)."""
    o = ovl()
    for tile, tpb in ((256, 64), (128, 256)):
        d = o.gemm_rs_desc(8, 0, 8192, 4096, 1792, tile, tile)
        assert o.gemm_rs_flags_bytes(d) == 8 * tpb * 8
        assert o.gemm_rs_workspace_bytes(d) == o.ERROR_RECORD_BYTES + 8 * tpb


@pytest.mark.parametrize("f8,tile,ok", [
    (False, (0, 0), True), (False, (256, 256), True), (False, (256, 128), False), (False, (128, 128), False),
    (True, (0, 0), True), (True, (256, 256), True), (True, (256, 128), False), (True, (128, 64), False),
])
def test_dispatch_tile_arguments(f8, tile, ok):
    """The grouped-GEMM tile of the dispatch descriptor: 0 x 0 (default) or
    the implemented one (256 x 256 for bf16 and FP8 rows) pass the argument
    checks; any other pair is refused with OVL_EUNSUPPORTED before any device
    work.  (An accepted tile fails later on the null row buffers, with
    OVL_EINVAL: no device is touched either way.)"""
    o = ovl()
    ad = o.a2a_desc(2, 0, 16, 64, 64, 2, 4, 2, 8, tile[0], tile[1])
    lib = o.lib()
    if f8:
        st = lib.a2a_dispatch_grouped_gemm_fp8_run(ctypes.byref(ad), None, None, None, None, None, None, None,
                                                   None, None, None, None, None, 1, None, None)
    else:
        st = lib.a2a_dispatch_grouped_gemm_run(ctypes.byref(ad), None, None, None, None, None, None, None, None,
                                               None, 1, None, None)
    assert st == (o.OVL_EINVAL if ok else o.OVL_EUNSUPPORTED)


def test_flag_and_workspace_sizes():
    o = ovl()
    d = o.gemm_rs_desc(8, 0, 8192, 4096, 1792)
    assert o.gemm_rs_flags_bytes(d) == 8 * 64 * 8
    assert o.gemm_rs_workspace_bytes(d) == o.ERROR_RECORD_BYTES + 8 * 64
    ad = o.a2a_desc(8, 0, 4096, 4096, 1408, 2, 64, 8, 128)
    assert o.a2a_flags_bytes(ad) == 8 * 128
    assert o.a2a_workspace_bytes(ad) >= o.ERROR_RECORD_BYTES + 8 * 8
    # the trace holds slices, 64 producers and 8 int64 per possible work item:
    # m-tiles <= 8 * 8192 / 256 + 8, n-tiles of 256 columns: 6
    assert o.a2a_trace_bytes(ad) == 8 * (8 + 64 + 8 * (8 * 8192 // 256 + 8) * 6)


@pytest.mark.parametrize("name,tpf,splits", [
    ("ag_r2_128x256x256", 0, 1),            # K too short to split
    ("ag_r8_8192x3584x4096", 1, 1),         # enough 256x256 tiles
    ("ag_r8_skinny_128x7168x8192", 4, 4),   # 56 tiles of 128x128: K in 4 ranges
])
def test_split_k_plan(name, tpf, splits):
    cfg = synth.CONFIGS[name]
    p = ovl().ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, tpf, 8)
    assert p.splits == splits
    if splits > 1:
        m = cfg.ranks * cfg.shard_m
        tiles = -(-m // 128) * -(-cfg.n // 128)
        counters = -(-tiles * 16 // 256) * 256
        assert p.workspace_bytes == 256 + counters + splits * m * cfg.n * 4
    else:
        assert p.workspace_bytes == 256
