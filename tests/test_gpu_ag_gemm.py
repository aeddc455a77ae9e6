"""GPU parity of the AllGather -> GEMM path against the oracle (through the C-ABI)."""

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gemm_tol
from tests.gpu_util import dev, host, say, zeros_bytes, zeros_f32, zeros_u16, max_err

pytestmark = pytest.mark.gpu


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


# A bf16 quiet NaN.  Before every run that copies (every mode but
# GEMM_ONLY) the gathered buffer is filled with it, so that a consumer that
# reads a unit before its producer has written it turns its rows of C into
# NaN, which the comparison with the oracle cannot miss (a gathered buffer
# left over from an earlier run would hold the right bits already).
NAN_BF16 = 0x7FC0


class AgCase:
    def __init__(self, cfg, kind="normal", tiles_per_flag=0, flag_stride=8, rank=0, unit_producers=1):
        o = ovl()
        self.cfg = cfg
        self.shards, self.b = synth.ag_inputs(cfg, kind)
        self.plan = o.ag_gemm_plan(cfg.ranks, rank, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n,
                                   tiles_per_flag, flag_stride, unit_producers)
        self.units, self.panels, self.batches = oracle.ag_flag_units(cfg.ranks, cfg.shard_m, cfg.k, cfg.tile_m,
                                                                     cfg.tile_n, tiles_per_flag)
        assert self.plan.num_units == self.units
        assert self.plan.flags_bytes == self.units * flag_stride
        self.stride = flag_stride
        self.d_shards = [dev(s) for s in self.shards]
        self.d_b = dev(self.b)
        self.g = zeros_u16(cfg.m, cfg.k)
        self.c = zeros_f32(cfg.m, cfg.n)
        self.flags = zeros_bytes(self.plan.flags_bytes)
        self.ws = zeros_bytes(self.plan.workspace_bytes)
        o.ovl_flags_reset(self.flags, self.plan.flags_bytes, self.ws, self.plan.workspace_bytes)

    def order(self, epoch, kind="panels"):
        return synth.producer_order(self.cfg.seed, epoch, self.cfg.ranks * self.panels, self.batches, True, kind)

    def run(self, epoch, order=None, mode=0, producers=0, spin_limit=0, jitter=0, poison=True):
        o = ovl()
        d_order = dev(order) if order is not None else None
        if poison and mode != o.MODE_GEMM_ONLY:
            self.g.fill_(NAN_BF16)
        say(f"  ag_gemm_run {self.cfg.name} epoch={epoch} mode={mode} order={'none' if order is None else 'set'}"
            f" jitter={jitter}")
        o.ag_gemm_run(self.plan, self.d_shards, self.d_b, self.g, self.c, self.flags, self.ws, epoch, d_order,
                      mode=mode, producers=producers, spin_limit=spin_limit, jitter=jitter)
        return o.ovl_check(self.ws, raise_on_error=False)

    def check_gathered_and_flags(self, epoch):
        g = host(self.g, np.uint16)
        assert np.array_equal(g, oracle.all_gather(self.shards)), "gathered != concatenation of shards"
        fl = host(self.flags)[: self.plan.flags_bytes]
        assert np.array_equal(fl, oracle.expected_flags(self.units, self.stride, epoch)), "flag bytes differ"


def _full_check(case, c_ref=None):
    """Every element of C against the oracle's float64 product."""
    if c_ref is None:
        _, c_ref = oracle.ag_gemm(case.shards, case.b)
    c = host(case.c)
    assert np.isfinite(c).all(), "C holds NaN or Inf: a unit was read before it was written"
    tol = gemm_tol(case.cfg.k, float(np.abs(c_ref).max()))
    err = max_err(c, c_ref)
    assert err <= tol, f"max err {err} > tol {tol}"
    return c


def _exact_check(case, c_ref=None):
    """Small-integer inputs: every element of C equals the exact product."""
    if c_ref is None:
        _, c_ref = oracle.ag_gemm(case.shards, case.b)
    assert np.array_equal(host(case.c), c_ref.astype(np.float32))


def _small(name, R, Ms, K, N, tm, tn, seed=5):
    return synth.AgGemmCfg(name, R, Ms, K, N, tm, tn, 1.0, 1.0 / 16, seed, True)


# ------------------------------------------------------------------ small / ragged

def test_small_fused_matches_oracle():
    case = AgCase(synth.CONFIGS["ag_r2_128x256x256"])
    st, det = case.run(1)
    assert st == 0, det
    case.check_gathered_and_flags(1)
    _full_check(case)


@pytest.mark.parametrize("mode", [0, 3])
def test_small_integers_bit_exact(mode):
    case = AgCase(synth.CONFIGS["ag_r2_128x256x256"], "smallint")
    st, det = case.run(1, mode=mode)
    assert st == 0, det
    _, c_ref = oracle.ag_gemm(case.shards, case.b)
    assert np.array_equal(host(case.c), c_ref.astype(np.float32))


@pytest.mark.parametrize("shape", [
    # R, shard_m, K, N, tile_m, tile_n, tiles_per_flag
    (3, 100, 200, 136, 48, 40, 2),   # ragged panels, ragged K-batch, ragged N tile
    (2, 300, 520, 264, 256, 64, 1),  # 256-row panels with a short last panel
    (5, 16, 64, 8, 128, 32, 0),      # shards shorter than the tile: unit = whole shard
    (1, 129, 8, 16, 64, 8, 1),       # one rank, K of one vector
])
def test_ragged_shapes_match_oracle(shape):
    R, Ms, K, N, tm, tn, tpf = shape
    cfg = _small("ragged", R, Ms, K, N, tm, tn)
    case = AgCase(cfg, tiles_per_flag=tpf)
    order = case.order(1, "units")
    st, det = case.run(1, order)
    assert st == 0, det
    case.check_gathered_and_flags(1)
    _full_check(case)


# ------------------------------------------------------------------ split K

def _counters_are_zero(case):
    tiles = -(-case.cfg.m // 128) * -(-case.cfg.n // 128)  # split plans use 128x128 tiles
    cnt = host(case.ws)[256: 256 + 16 * tiles].view(np.int64)
    return not cnt.any()


@pytest.mark.parametrize("mode", [0, 3, 2])
def test_split_k_small_integers_bit_exact(mode):
    # 64 x 256 output in two 128x128 tiles, K = 2048 in 8 ranges of 256.
    cfg = _small("splitk", 4, 16, 2048, 256, 16, 128, seed=11)
    case = AgCase(cfg, "smallint", tiles_per_flag=2)
    assert case.plan.splits == 8
    _, c_ref = oracle.ag_gemm(case.shards, case.b)
    if mode == 2:  # GEMM only: the gathered operand must already be there
        assert case.run(1, case.order(1, "units"), mode=1)[0] == 0
    for epoch in (2, 3):
        st, det = case.run(epoch, case.order(epoch, "units"), mode=mode)
        assert st == 0, det
        assert np.array_equal(host(case.c), c_ref.astype(np.float32))
        assert _counters_are_zero(case)
    if mode != 2:
        case.check_gathered_and_flags(3)


def test_split_k_ragged_orders_and_modes_agree():
    # 150 x 200 output (2 x 2 tiles of 128, ragged), K = 1000 in ranges of
    # 256, 256, 256, 232; flag batches of 120 columns straddle the ranges.
    cfg = _small("splitk_ragged", 3, 50, 1000, 200, 50, 40, seed=12)
    case = AgCase(cfg, tiles_per_flag=3)
    assert case.plan.splits == 4
    first = None
    for epoch in range(1, 5):
        st, det = case.run(epoch, case.order(epoch, "units"), mode=0 if epoch < 4 else 3)
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        assert _counters_are_zero(case)
        c = host(case.c).copy()
        if first is None:
            first = _full_check(case).copy()
        assert np.array_equal(c.view(np.uint32), first.view(np.uint32)), "C bits changed with producer order"


def test_epochs_reuse_flags_without_reset():
    case = AgCase(synth.CONFIGS["ag_r2_128x256x256"], tiles_per_flag=2, flag_stride=128)
    first = None
    for epoch in range(1, 6):
        st, det = case.run(epoch, case.order(epoch, "units"))
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        c = host(case.c).copy()
        if first is None:
            first = c
            _full_check(case)
        assert np.array_equal(c.view(np.uint32), first.view(np.uint32)), "C bits changed with producer order"


def test_epoch_rules():
    o = ovl()
    case = AgCase(synth.CONFIGS["ag_r2_128x256x256"])
    with pytest.raises(o.OvlError) as e:
        case.run(0)
    assert e.value.status == o.OVL_EEPOCH
    assert case.run(3)[0] == 0
    for bad in (3, 2):
        with pytest.raises(o.OvlError) as e:
            case.run(bad)
        assert e.value.status == o.OVL_EEPOCH
    o.ovl_flags_reset(case.flags, case.plan.flags_bytes, case.ws, case.plan.workspace_bytes)
    assert case.run(1)[0] == 0
    case.check_gathered_and_flags(1)


def test_missing_unit_times_out():
    # A producer order that repeats one unit and omits another leaves the
    # omitted unit unsignalled: its waiters must give up with OVL_ETIMEOUT.
    o = ovl()
    case = AgCase(synth.CONFIGS["ag_r2_128x256x256"])
    order = np.arange(case.units, dtype=np.int32)
    missing = case.units - 1
    order[missing] = 0
    st, det = case.run(1, order, spin_limit=2000)
    assert st == o.OVL_ETIMEOUT
    assert det[1] == missing and det[3] == 1


def test_modes_compose_to_the_same_bits():
    o = ovl()
    cfg = _small("modes", 4, 192, 384, 320, 64, 64)
    case = AgCase(cfg, tiles_per_flag=2)
    assert case.run(1, case.order(1))[0] == 0
    fused = host(case.c).copy()
    case.c.zero_()
    assert case.run(2, mode=o.MODE_BARRIER)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), fused.view(np.uint32))
    case.c.zero_()
    case.g.zero_()
    assert case.run(3, case.order(3), mode=o.MODE_COPY_ONLY)[0] == 0
    case.check_gathered_and_flags(3)
    assert case.run(4, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), fused.view(np.uint32))
    _full_check(case)


# ------------------------------------------------------------------ 256 x 256 consumer tile, ragged

@pytest.mark.parametrize("kind", ["normal", "smallint"])
def test_ragged_big_tile_orders_and_modes(kind):
    """The 256 x 256 consumer tile (the headline's) at a ragged size the
    oracle finishes at once: 4000 x 2056 x 520 is 16 x 9 tiles with short
    last rows and columns, shards of 1000 rows straddle the tiles, and
    K-batches of 128 columns end in an 8-column batch.  Every element of C
    is compared, over random unit orders, producer jitter, BARRIER and
    COPY_ONLY + GEMM_ONLY, and the bits must not move."""
    o = ovl()
    cfg = _small("ragged_big", 4, 1000, 520, 2056, 256, 64, seed=31)
    case = AgCase(cfg, kind, tiles_per_flag=2)
    assert case.plan.tile_rows == 256 and case.plan.splits == 1
    _, c_ref = oracle.ag_gemm(case.shards, case.b)
    check = _exact_check if kind == "smallint" else _full_check
    bits = None
    for epoch, jitter in ((1, 0), (2, 0), (3, 300)):
        st, det = case.run(epoch, case.order(epoch, "units"), jitter=jitter)
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        check(case, c_ref)
        c = host(case.c).view(np.uint32)
        if bits is None:
            bits = c.copy()
        assert np.array_equal(c, bits), "C bits changed with producer order"
    case.c.zero_()
    assert case.run(4, mode=o.MODE_BARRIER)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), bits)
    case.c.zero_()
    assert case.run(5, case.order(5, "units"), mode=o.MODE_COPY_ONLY)[0] == 0
    case.check_gathered_and_flags(5)
    assert case.run(6, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), bits)


def test_producer_jitter_leaves_the_bits_alone():
    """Producers that pause a hashed, uneven time before every unit (a test
    aid of the call) deliver units in a shuffled order: the consumers must
    still produce exactly the bits of an unjittered run."""
    cfg = _small("jitter", 8, 256, 1024, 1024, 256, 128, seed=32)
    case = AgCase(cfg, tiles_per_flag=2)
    assert case.run(1, case.order(1))[0] == 0
    bits = host(case.c).view(np.uint32).copy()
    _full_check(case)
    for epoch, jitter in ((2, 64), (3, 400), (4, 1000)):
        case.c.zero_()
        st, det = case.run(epoch, case.order(epoch, "units"), jitter=jitter)
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        assert np.array_equal(host(case.c).view(np.uint32), bits)


def test_more_panels_than_the_bootstrap_table():
    """16 shards of 65 panels (1040 flag units, more than the bootstrap
    table holds): the bootstrap is off and every unit is moved by the
    producers; gathered, flags and C in full."""
    cfg = _small("many_panels", 16, 1040, 128, 64, 16, 64, seed=33)
    case = AgCase(cfg)
    assert case.units == 16 * 65
    for epoch in (1, 2):
        st, det = case.run(epoch, case.order(epoch, "units"))
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        _full_check(case)


@pytest.mark.parametrize("mode", [0, 3])
def test_flag_ahead_of_the_epoch_is_reported_and_parity_catches_the_early_read(mode):
    """The checker bites on early consumption.  Every unit flag is preset to
    epoch + 1 (as a signal of a later run would leave it) and the producer
    order leaves out the units of one peer panel, so they are never copied.
    The consumers then find their flags already set, do not wait, and read
    that panel's rows of `gathered` while they still hold the NaN fill: the
    run reports OVL_EEPOCH (a flag above the awaited epoch), the panel's
    rows of C are NaN, and the comparison with the oracle fails.  The same
    order with the flags reset and the units all moved passes."""
    import torch
    o = ovl()
    cfg = _small("early", 4, 256, 512, 512, 64, 64, seed=34)
    case = AgCase(cfg, tiles_per_flag=2)
    shard, panel = 2, 1  # rows [576, 640): not the own rank's
    order = case.order(1, "units")
    dropped = np.isin(order // case.batches, [shard * case.panels + panel])
    assert dropped.sum() == case.batches
    order[dropped] = -1
    case.flags.view(torch.int64).fill_(2)
    st, det = case.run(1, order, mode=mode)
    assert st == o.OVL_EEPOCH, (st, det)
    assert det[0] == (1 if mode == 0 else 2) and det[2] == 2 and det[3] == 1, det
    c = host(case.c)
    r0 = shard * cfg.shard_m + panel * 64
    assert np.isnan(c[r0:r0 + 64]).all(), "the panel that never moved was not read early"
    with pytest.raises(AssertionError):
        _full_check(case)
    o.ovl_flags_reset(case.flags, case.plan.flags_bytes, case.ws, case.plan.workspace_bytes)
    case.c.zero_()
    st, det = case.run(1, case.order(1, "units"), mode=mode)
    assert st == 0, det
    _full_check(case)


# ------------------------------------------------------------------ split units (signal ADD)

@pytest.mark.parametrize("W", [2, 4, 7])
def test_split_unit_arrivals_match_one_publisher(W):
    """Each flag unit moved by W producer workgroups that each add an arrival
    to the unit's counter, the arrival completing a multiple of W setting the
    flag: gathered and flags bit-exact and C bit-identical to the
    one-publisher plan, over epochs that skip values (the counter is never
    reset), random orders, jitter, BARRIER and COPY_ONLY + GEMM_ONLY."""
    o = ovl()
    cfg = _small("split_units", 4, 1000, 520, 2056, 256, 64, seed=35)
    one = AgCase(cfg, tiles_per_flag=2)
    assert one.run(1, one.order(1, "units"))[0] == 0
    bits = host(one.c).view(np.uint32).copy()
    _full_check(one)
    case = AgCase(cfg, tiles_per_flag=2, unit_producers=W)
    assert case.plan.workspace_bytes > one.plan.workspace_bytes
    for epoch, jitter in ((1, 0), (2, 0), (5, 200), (9, 0)):
        case.c.zero_()
        st, det = case.run(epoch, case.order(epoch, "units"), jitter=jitter)
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        assert np.array_equal(host(case.c).view(np.uint32), bits), f"epoch {epoch}"
    case.c.zero_()
    assert case.run(10, mode=o.MODE_BARRIER)[0] == 0
    case.check_gathered_and_flags(10)
    assert np.array_equal(host(case.c).view(np.uint32), bits)
    assert case.run(11, case.order(11, "units"), mode=o.MODE_COPY_ONLY)[0] == 0
    case.check_gathered_and_flags(11)
    case.c.zero_()
    assert case.run(12, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), bits)
    # every counter holds W arrivals per run that moved units (6 runs); the
    # plan has no K split, so the counters follow the 256-byte error record
    assert case.plan.splits == 1
    cnt = host(case.ws)[256: 256 + case.units * 8].view(np.int64)
    assert (cnt == 6 * W).all(), np.unique(cnt)


def test_full_size_split_units_match_one_publisher():
    """The headline workload with 4 producers per 256 x 256 flag unit: the
    same gathered, flags and C bits as one publisher per unit."""
    cfg = synth.CONFIGS["ag_r8_8192x3584x4096"]
    one = AgCase(cfg, tiles_per_flag=1)
    assert one.run(1, one.order(1))[0] == 0
    bits = host(one.c).view(np.uint32).copy()
    case = AgCase(cfg, tiles_per_flag=1, unit_producers=4)
    for epoch in (1, 2):
        st, det = case.run(epoch, case.order(epoch))
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        assert np.array_equal(host(case.c).view(np.uint32), bits)


# ------------------------------------------------------------------ full sizes

@pytest.mark.parametrize("name,tpf", [("ag_r8_8192x3584x4096", 1), ("ag_r8_skinny_128x7168x8192", 4)])
def test_full_size_random_orders_and_modes(name, tpf):
    """The workloads at full size, in the bench's launch configuration:
    gathered and flags bit-exact, every element of C within the bound, and
    C bit-identical over three seeded producer orders, BARRIER and
    GEMM_ONLY."""
    o = ovl()
    cfg = synth.CONFIGS[name]
    case = AgCase(cfg, tiles_per_flag=tpf)
    _, c_ref = oracle.ag_gemm(case.shards, case.b)
    bits = None
    for epoch in range(1, 4):
        st, det = case.run(epoch, case.order(epoch))
        assert st == 0, det
        case.check_gathered_and_flags(epoch)
        c = host(case.c)
        if bits is None:
            bits = c.view(np.uint32).copy()
            _full_check(case, c_ref)
        else:
            assert np.array_equal(c.view(np.uint32), bits)
    case.c.zero_()
    assert case.run(4, mode=o.MODE_BARRIER)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), bits)
    case.c.zero_()
    assert case.run(5, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.c).view(np.uint32), bits)


@pytest.mark.parametrize("name,tpf", [("ag_r8_8192x3584x4096", 1), ("ag_r8_skinny_128x7168x8192", 4)])
def test_full_size_small_integers_exact(name, tpf):
    """Small integers: fp32 accumulation is exact, so every element of C
    must equal the oracle's product bit for bit (every index, swizzle and
    tile bug shows)."""
    cfg = synth.CONFIGS[name]
    case = AgCase(cfg, "smallint", tiles_per_flag=tpf)
    st, det = case.run(1, case.order(1))
    assert st == 0, det
    case.check_gathered_and_flags(1)
    _exact_check(case)


# ------------------------------------------------------------------ device trace

def test_trace_records_publishes_and_waits_in_causal_order():
    """A traced run gives the same bits as an untraced one, and its records
    hold together: every unit is published, every item ends after it starts
    and after the publish of every unit its rows and K range need, and its
    waits fit inside it."""
    import ctypes
    import torch
    o = ovl()
    cfg = _small("ag_trace", 4, 256, 512, 2048, 256, 256, seed=9)
    case = AgCase(cfg, tiles_per_flag=1)
    plan = case.plan
    assert plan.splits == 1  # enough tiles for the consumers: one item per tile
    order = case.order(1, "units")
    assert case.run(1, order)[0] == 0
    c_plain = host(case.c).copy()
    trace = torch.zeros(plan.trace_bytes // 8, dtype=torch.int64, device="cuda")
    case.c.zero_()
    case.g.zero_()
    say("  traced run")
    o.ag_gemm_run(plan, case.d_shards, case.d_b, case.g, case.c, case.flags, case.ws, 2, dev(order), trace=trace)
    st, det = o.ovl_check(case.ws, raise_on_error=False)
    assert st == 0, det
    assert np.array_equal(host(case.c).view(np.uint32), c_plain.view(np.uint32))
    tr = host(trace)
    units = plan.num_units
    pub = tr[:units]
    items = tr[units:].reshape(-1, 6)
    assert np.all(pub > 0), "a unit without a publish time"
    assert np.all(items[:, 0] > 0) and np.all(items[:, 1] >= items[:, 0])
    assert np.all((items[:, 2] >= 0) & (items[:, 2] <= items[:, 1] - items[:, 0]))
    # the shader clock over the 100 MHz ticks: a plausible clock (0.5 to 3 GHz)
    ghz = (items[:, 5] - items[:, 4]).sum() / ((items[:, 1] - items[:, 0]).sum() * 10.0)
    assert 0.5 < ghz < 3.0, ghz
    # consumer order (host copy of the device rule) -> each item's row tile
    lib = o.lib()
    lib.ag_gemm_row_tiles.argtypes = [ctypes.c_void_p]
    lib.ag_gemm_row_tiles.restype = ctypes.c_int32
    lib.ag_gemm_consumer_order.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ag_gemm_consumer_order.restype = ctypes.c_int32
    row_tiles = lib.ag_gemm_row_tiles(plan.handle.value)
    bm = cfg.m // row_tiles
    tiles_n = len(items) // row_tiles
    o32 = np.ascontiguousarray(order.astype(np.int32))
    sorted_rt = np.zeros(row_tiles, dtype=np.int32)
    assert lib.ag_gemm_consumer_order(plan.handle.value, o32.ctypes.data, sorted_rt.ctypes.data) == 0
    for j, rec in enumerate(items):
        rt = int(sorted_rt[j // tiles_n])
        s = rt * bm // cfg.shard_m  # the shard holding the tile's rows (one panel per shard here)
        if s == 0:  # the own shard: nothing to wait for
            assert rec[2] == 0
            continue
        need = [s * case.batches + bt for bt in range(case.batches)]
        assert pub[need].max() <= rec[1], f"item {j} ended before its units were published"
