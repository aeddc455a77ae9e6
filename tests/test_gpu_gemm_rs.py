"""GPU parity of the GEMM -> ReduceScatter path against the oracle (through the C-ABI)."""

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gemm_tol
from tests.gpu_util import dev, host, say, zeros_bytes, zeros_f32, max_err

pytestmark = pytest.mark.gpu


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


TILES = (256, 128)  # the implemented tiles (tile_m = tile_n)


class RsCase:
    def __init__(self, cfg, kind="normal", tile=256):
        o = ovl()
        self.cfg = cfg
        self.a, self.b, self.parts = synth.rs_inputs(cfg, kind)
        R, bm = cfg.ranks, cfg.block_m
        self.desc = o.gemm_rs_desc(R, cfg.rank, cfg.m, cfg.n, cfg.k, tile, tile, 8)
        self.fbytes = o.gemm_rs_flags_bytes(self.desc)
        self.tpb = self.fbytes // 8 // R
        self.d_a, self.d_b = dev(self.a), dev(self.b)
        self.peer_out = [None if p == cfg.rank else zeros_f32(bm, cfg.n) for p in range(R)]
        self.peer_in = [None if p == cfg.rank else dev(self.parts[p]) for p in range(R)]
        self.out = zeros_f32(bm, cfg.n)
        self.out_flags = zeros_bytes(self.fbytes)
        self.in_flags = zeros_bytes(self.fbytes)
        self.ws = zeros_bytes(o.gemm_rs_workspace_bytes(self.desc))
        o.ovl_flags_reset(self.out_flags, self.fbytes, self.ws, self.ws.numel())

    def set_in_flags(self, epoch):
        v = self.in_flags.view(dtype=__import__("torch").int64).view(self.cfg.ranks, self.tpb)
        v.fill_(epoch)
        v[self.cfg.rank].zero_()

    def poison(self):
        """NaN in every output, so that an element the run fails to write shows."""
        self.out.fill_(float("nan"))
        for t in self.peer_out:
            if t is not None:
                t.fill_(float("nan"))

    def run(self, epoch, mode=0, spin_limit=0):
        o = ovl()
        say(f"  gemm_rs_run {self.cfg.name} tile={self.desc.tile_m} epoch={epoch} mode={mode}")
        o.gemm_rs_run(self.desc, self.d_a, self.d_b, self.peer_out, self.peer_in, self.out, self.out_flags,
                      self.in_flags, self.ws, epoch, mode=mode, spin_limit=spin_limit)
        return o.ovl_check(self.ws, raise_on_error=False)


def _small(R=4, rank=1, bm=300, n=264, k=200, seed=9):
    return synth.GemmRsCfg("rs_small", R, R * bm, k, n, 256, 256, 1.0, 0.25, 1.0, seed, rank)


@pytest.mark.parametrize("tile", TILES)
def test_small_ragged_matches_oracle(tile):
    cfg = _small()
    case = RsCase(cfg, tile=tile)
    case.set_in_flags(1)
    case.poison()
    st, det = case.run(1)
    assert st == 0, det
    loc, outb, own = oracle.gemm_rs(case.a, case.b, case.parts, cfg.rank, cfg.ranks)
    tol = gemm_tol(cfg.k, float(np.abs(loc).max()))
    for p in range(cfg.ranks):
        if p != cfg.rank:
            assert max_err(host(case.peer_out[p]), outb[p]) <= tol
    assert max_err(host(case.out), own) <= gemm_tol(cfg.k, float(np.abs(own).max()))
    fl = host(case.out_flags)[: case.fbytes]
    assert np.array_equal(fl, oracle.rs_expected_flags(cfg.ranks, cfg.rank, case.tpb, 8, 1))


@pytest.mark.parametrize("tile", TILES)
def test_small_integers_bit_exact(tile):
    cfg = _small(R=8, rank=0, bm=256, n=512, k=320)
    case = RsCase(cfg, "smallint", tile=tile)
    case.set_in_flags(1)
    assert case.run(1)[0] == 0
    loc, outb, own = oracle.gemm_rs(case.a, case.b, case.parts, cfg.rank, cfg.ranks)
    assert np.array_equal(host(case.out), own.astype(np.float32))
    for p in range(1, 8):
        assert np.array_equal(host(case.peer_out[p]), outb[p].astype(np.float32))


@pytest.mark.parametrize("tile", TILES)
def test_single_rank_is_plain_gemm(tile):
    cfg = _small(R=1, rank=0, bm=520, n=136, k=64)
    case = RsCase(cfg, tile=tile)
    st, det = case.run(1)
    assert st == 0, det
    ref = oracle.gemm(case.a, case.b)
    assert max_err(host(case.out), ref) <= gemm_tol(cfg.k, float(np.abs(ref).max()))


@pytest.mark.parametrize("tile", TILES)
def test_withheld_partial_times_out(tile):
    o = ovl()
    cfg = _small()
    case = RsCase(cfg, tile=tile)
    case.set_in_flags(1)
    v = case.in_flags.view(dtype=__import__("torch").int64).view(cfg.ranks, case.tpb)
    v[3, 2] = 0  # peer 3 never sent tile 2 of this rank's block
    st, det = case.run(1, spin_limit=2000)
    assert st == o.OVL_ETIMEOUT
    # The reduce job that needs the withheld partial gives up (site 3: in
    # flag 3*tpb + 2, observed 0, awaited 1).
    assert det == (3, 3 * case.tpb + 2, 0, 1), det


def _check_all(case, exact=False):
    """Every element of the own block and of every outbound partial."""
    cfg = case.cfg
    loc, outb, own = oracle.gemm_rs(case.a, case.b, case.parts, cfg.rank, cfg.ranks)
    got_own = host(case.out)
    if exact:
        assert np.array_equal(got_own, own.astype(np.float32))
    else:
        assert np.isfinite(got_own).all()
        assert max_err(got_own, own) <= gemm_tol(cfg.k, float(np.abs(own).max()))
    tol = gemm_tol(cfg.k, float(np.abs(loc).max()))
    for p in range(cfg.ranks):
        if p == cfg.rank:
            continue
        got = host(case.peer_out[p])
        if exact:
            assert np.array_equal(got, outb[p].astype(np.float32)), f"partial for peer {p}"
        else:
            assert max_err(got, outb[p]) <= tol, f"partial for peer {p}"
    fl = host(case.out_flags)[: case.fbytes]
    assert np.array_equal(fl, oracle.rs_expected_flags(cfg.ranks, cfg.rank, case.tpb, 8, case.last_epoch))


@pytest.mark.parametrize("kind,tile", [("normal", 256), ("smallint", 256), ("normal", 128), ("smallint", 128)])
def test_full_size(kind, tile):
    """8192 x 4096 x 1792 over 8 ranks in the bench's launch configuration
    (256 x 256 tiles) and with 128 x 128 tiles: the own block and all 7
    outbound partials compared in full (bit for bit with small integers),
    flags exact, and GEMM_ONLY gives the same bits."""
    cfg = synth.CONFIGS["rs_r8_8192x4096x1792"]
    case = RsCase(cfg, kind, tile=tile)
    case.set_in_flags(1)
    case.poison()
    st, det = case.run(1)
    assert st == 0, det
    case.last_epoch = 1
    _check_all(case, exact=kind == "smallint")
    first = host(case.out).view(np.uint32).copy()
    case.poison()
    assert case.run(2, mode=ovl().MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.out).view(np.uint32), first)
