"""GPU parity of the all-to-all dispatch -> grouped expert GEMM path (through the C-ABI)."""

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gemm_tol
from tests.gpu_util import dev, host, say, zeros_bytes, max_err

pytestmark = pytest.mark.gpu


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


class A2aCase:
    def __init__(self, cfg, kind="normal", topk=None):
        import torch
        o = ovl()
        self.cfg = cfg
        self.x, self.topk, self.w = synth.dispatch_inputs(cfg, kind)
        if topk is not None:
            self.topk = topk
        R, cap = cfg.ranks, cfg.cap
        self.desc = o.a2a_desc(R, cfg.rank, cfg.tokens, cfg.hidden, cfg.n, cfg.topk, cfg.num_experts,
                               cfg.experts_per_rank, 8)
        self.fbytes = o.a2a_flags_bytes(self.desc)
        self.d_x = [dev(a) for a in self.x]
        self.d_topk = [dev(t) for t in self.topk]
        self.d_w = dev(self.w)
        self.recv_x = torch.zeros(R, cap, cfg.hidden, dtype=torch.int16, device="cuda")
        self.recv_src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
        self.recv_count = torch.zeros(R, cfg.experts_per_rank, dtype=torch.int32, device="cuda")
        self.y = torch.zeros(R, cap, cfg.n, dtype=torch.float32, device="cuda")
        self.flags = zeros_bytes(self.fbytes)
        self.ws = zeros_bytes(o.a2a_workspace_bytes(self.desc))
        o.ovl_flags_reset(self.flags, self.fbytes, self.ws, self.ws.numel())

    def run(self, epoch, mode=0, producers=0):
        o = ovl()
        say(f"  a2a_run {self.cfg.name} epoch={epoch} mode={mode}")
        o.a2a_dispatch_grouped_gemm_run(self.desc, self.d_x, self.d_topk, self.d_w, self.recv_x, self.recv_src,
                                        self.recv_count, self.y, self.flags, self.ws, epoch, mode=mode,
                                        producers=producers)
        return o.ovl_check(self.ws, raise_on_error=False)

    def oracle_layout(self):
        c = self.cfg
        return oracle.dispatch(self.x, self.topk, c.rank, c.experts_per_rank, c.cap)

    def check_layout(self, epoch):
        rx, rs, rc = self.oracle_layout()
        assert np.array_equal(host(self.recv_count), rc), "recv_count differs"
        assert np.array_equal(host(self.recv_src), rs), "recv_src differs"
        assert np.array_equal(host(self.recv_x, np.uint16), rx), "recv_x differs"
        fl = host(self.flags)[: self.fbytes]
        assert np.array_equal(fl, oracle.expected_flags(self.cfg.ranks, 8, epoch)), "flags differ"
        return rx, rs, rc


def _cfg(name, R=2, T=64, H=64, N=128, topk=2, E=4, rank=0, seed=3):
    return synth.DispatchCfg(name, R, T, H, N, topk, R * E, E, 1.1, 1.0, 0.25, seed, rank)


@pytest.mark.parametrize("cfg", [
    _cfg("a2a_small"),
    _cfg("a2a_ragged", R=3, T=100, H=200, N=136, E=3, rank=1, seed=5),
    _cfg("a2a_skewed", R=4, T=300, H=72, N=256, E=2, rank=3, seed=8),
    _cfg("a2a_rows_2k", R=3, T=90, H=1024, N=136, E=3, rank=1, seed=6),  # 4 rows per copy slot
])
def test_small_matches_oracle(cfg):
    case = A2aCase(cfg)
    st, det = case.run(1)
    assert st == 0, det
    rx, rs, rc = case.check_layout(1)
    y_ref = oracle.grouped_gemm(rx, rc, case.w)
    y = host(case.y)
    assert max_err(y, y_ref) <= gemm_tol(cfg.hidden, float(np.abs(y_ref).max()))


def test_small_integers_bit_exact_and_modes_agree():
    o = ovl()
    cfg = _cfg("a2a_int", R=4, T=200, H=128, N=256, E=2, rank=2)
    case = A2aCase(cfg, "smallint")
    assert case.run(1)[0] == 0
    rx, rs, rc = case.check_layout(1)
    y_ref = oracle.grouped_gemm(rx, rc, case.w)
    first = host(case.y).copy()
    assert np.array_equal(first, y_ref.astype(np.float32))
    case.recv_x.zero_()
    case.y.zero_()
    assert case.run(2, mode=o.MODE_COPY_ONLY)[0] == 0
    case.check_layout(2)
    assert case.run(3, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.y).view(np.uint32), first.view(np.uint32))
    for producers in (1, 3, 64):
        assert case.run(4 + producers, producers=producers)[0] == 0
        case.check_layout(4 + producers)
        assert np.array_equal(host(case.y).view(np.uint32), first.view(np.uint32))


def test_own_slice_tiles_read_in_place_match_the_copy():
    # Every own token picks local expert 0, so that expert's first two
    # m-tiles (256 rows each) hold own-slice rows only: the fused launch
    # reads them from the own tokens in place, the GEMM-only launch from the
    # copied slice.  Small integers: both must equal the oracle bit for bit.
    o = ovl()
    cfg = _cfg("a2a_own", R=2, T=600, H=128, N=256, topk=1, E=2, rank=0, seed=9)
    rng = np.random.default_rng(11)
    topk = [np.zeros((cfg.tokens, 1), dtype=np.int32),
            rng.integers(0, 2 * cfg.experts_per_rank, (cfg.tokens, 1)).astype(np.int32)]
    case = A2aCase(cfg, "smallint", topk=topk)
    for epoch, producers in ((1, 0), (2, 1)):
        case.y.zero_()
        assert case.run(epoch, producers=producers)[0] == 0
        rx, rs, rc = case.check_layout(epoch)
        assert rc[0, 0] == cfg.tokens  # the own slice: all to local expert 0
        y_ref = oracle.grouped_gemm(rx, rc, case.w)
        assert np.array_equal(host(case.y), y_ref.astype(np.float32))
    fused = host(case.y).view(np.uint32).copy()
    case.y.zero_()
    assert case.run(3, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.y).view(np.uint32), fused)


def test_slices_with_nothing_routed_complete():
    # Every token of every source picks experts of other ranks only.
    cfg = _cfg("a2a_empty", R=3, T=40, E=2, rank=1)
    topk = [np.tile(np.array([[0, 5]], dtype=np.int32), (cfg.tokens, 1)) for _ in range(3)]
    case = A2aCase(cfg, topk=topk)
    st, det = case.run(1)
    assert st == 0, det
    case.check_layout(1)
    assert not host(case.y).any()


def test_zero_tokens():
    cfg = _cfg("a2a_zero", R=2, T=0, E=2, rank=0)
    case = A2aCase(cfg)
    st, det = case.run(1)
    assert st == 0, det
    fl = host(case.flags)[: case.fbytes]
    assert np.array_equal(fl, oracle.expected_flags(2, 8, 1))
    assert not host(case.recv_count).any()


def test_full_size_layout_exact_and_rows_sampled():
    cfg = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]
    case = A2aCase(cfg)
    st, det = case.run(1)
    assert st == 0, det
    rx, rs, rc = case.check_layout(1)
    y = host(case.y)
    rng = np.random.default_rng(2)
    for s in (0, 3, 7):
        n_valid = int(rc[s].sum())
        rows = rng.choice(n_valid, size=min(48, n_valid), replace=False)
        ref = oracle.grouped_gemm_rows(rx, rc, case.w, s, rows)
        assert max_err(y[s, rows], ref) <= gemm_tol(cfg.hidden, float(np.abs(ref).max()))
        assert not y[s, n_valid:].any()
    first = y.view(np.uint32).copy()
    assert case.run(2)[0] == 0
    assert np.array_equal(host(case.y).view(np.uint32), first)
