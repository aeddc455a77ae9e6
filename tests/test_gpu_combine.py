"""GPU parity of the MoE combine (reverse all-to-all + gate-weighted sum)
against the oracle, through the C-ABI, after the dispatch + grouped GEMM."""

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gemm_tol
from tests.gpu_util import dev, host, say, zeros_bytes, max_err
from tests.test_gpu_dispatch import A2aCase, _cfg

pytestmark = pytest.mark.gpu


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


class CombineCase:
    """The dispatch + grouped GEMM at `rank`, then the combine there."""

    def __init__(self, cfg, kind="normal"):
        import torch
        o = ovl()
        self.cfg = cfg
        self.a2a = A2aCase(cfg, kind)
        st, det = self.a2a.run(1)
        assert st == 0, det
        self.gates, self.ret_in = synth.combine_inputs(cfg, kind)
        R, cap, N = cfg.ranks, cfg.cap, cfg.n
        self.d_gates = dev(self.gates)
        self.d_ret_in = [None if q == cfg.rank else dev(self.ret_in[q]) for q in range(R)]
        self.ret_out = [None if q == cfg.rank else torch.zeros(cap, N, dtype=torch.float32, device="cuda")
                        for q in range(R)]
        self.out = torch.zeros(cfg.tokens, N, dtype=torch.float32, device="cuda")
        self.fbytes = o.a2a_combine_flags_bytes(self.a2a.desc)
        self.out_flags = zeros_bytes(self.fbytes)
        self.in_flags = zeros_bytes(self.fbytes)
        self.ws = zeros_bytes(o.a2a_combine_workspace_bytes(self.a2a.desc))
        o.ovl_flags_reset(self.out_flags, self.fbytes, self.ws, self.ws.numel())

    def set_in_flags(self, epoch):
        v = self.in_flags.view(dtype=__import__("torch").int64)[: self.cfg.ranks]
        v.fill_(epoch)
        v[self.cfg.rank] = 0

    def run(self, epoch, mode=0, spin_limit=0):
        o = ovl()
        say(f"  a2a_combine_run {self.cfg.name} epoch={epoch} mode={mode}")
        o.a2a_combine_run(self.a2a.desc, self.a2a.y, self.a2a.recv_count, self.ret_out, self.d_ret_in,
                          self.a2a.d_topk[self.cfg.rank], self.d_gates, self.out, self.out_flags, self.in_flags,
                          self.ws, epoch, mode=mode, spin_limit=spin_limit)
        return o.ovl_check(self.ws, raise_on_error=False)

    def reference(self):
        """Oracle chain from the inputs: dispatch, grouped GEMM, combine."""
        c = self.cfg
        rx, rs, rc = self.a2a.oracle_layout()
        y = oracle.grouped_gemm(rx, rc, self.a2a.w)
        ret_out, out = oracle.combine(y, rc, self.ret_in, self.a2a.topk[c.rank], self.gates, c.rank,
                                      c.experts_per_rank)
        return y, rc, ret_out, out

    def check_out_flags(self, epoch):
        fl = host(self.out_flags)[: self.fbytes].view(np.int64)
        for q in range(self.cfg.ranks):
            assert fl[q] == (0 if q == self.cfg.rank else epoch), fl


@pytest.mark.parametrize("cfg", [
    _cfg("cb_small", R=3, T=50, H=64, N=128, E=2, rank=1, seed=21),
    _cfg("cb_ragged", R=4, T=77, H=72, N=136, E=3, rank=3, seed=22),
    _cfg("cb_top5", R=3, T=70, H=64, N=136, topk=5, E=4, rank=2, seed=25),
    _cfg("cb_top8", R=2, T=45, H=64, N=2312, topk=8, E=5, rank=0, seed=26),
])
def test_combine_matches_oracle(cfg):
    case = CombineCase(cfg)
    case.set_in_flags(1)
    st, det = case.run(1)
    assert st == 0, det
    y_ref, rc, ret_out_ref, out_ref = case.reference()
    y_gpu = host(case.a2a.y)
    for s in range(cfg.ranks):
        if s == cfg.rank:
            continue
        n = int(rc[s].sum())
        got = host(case.ret_out[s])
        assert np.array_equal(got[:n].view(np.uint32), y_gpu[s, :n].view(np.uint32)), "reverse put is not a copy"
        assert not got[n:].any()
        assert max_err(got[:n], ret_out_ref[s]) <= gemm_tol(cfg.hidden, float(np.abs(y_ref).max()))
    # gates sum to 1: the GEMM bound of the local rows, plus fp32 rounding of the sum
    tol = gemm_tol(cfg.hidden, float(np.abs(y_ref).max())) + 1e-5 * float(np.abs(out_ref).max())
    assert max_err(host(case.out), out_ref) <= tol
    case.check_out_flags(1)


def test_small_integers_bit_exact_and_modes_agree():
    o = ovl()
    cfg = _cfg("cb_int", R=4, T=60, H=64, N=128, E=2, rank=2, seed=23)
    case = CombineCase(cfg, "smallint")
    case.set_in_flags(1)
    assert case.run(1)[0] == 0
    _, _, _, out_ref = case.reference()
    first = host(case.out).copy()
    assert np.array_equal(first, out_ref.astype(np.float32))
    for r in case.ret_out:
        if r is not None:
            r.zero_()
    case.out.zero_()
    assert case.run(2, mode=o.MODE_COPY_ONLY)[0] == 0
    case.check_out_flags(2)
    assert not host(case.out).any()
    assert case.run(3, mode=o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.out).view(np.uint32), first.view(np.uint32))


def test_withheld_return_times_out():
    o = ovl()
    cfg = _cfg("cb_withheld", R=3, T=40, H=64, N=128, E=2, rank=0, seed=24)
    case = CombineCase(cfg)
    case.set_in_flags(1)
    case.in_flags.view(dtype=__import__("torch").int64)[2] = 0  # peer 2 never returned its rows
    st, det = case.run(1, spin_limit=2000)
    assert st == o.OVL_ETIMEOUT
    assert det == (7, 2, 0, 1), det
    case.check_out_flags(1)  # the reverse puts still completed


def test_zero_tokens_sets_every_out_flag():
    cfg = _cfg("cb_zero", R=3, T=0, E=2, rank=1)
    case = CombineCase(cfg)
    case.set_in_flags(1)
    st, det = case.run(1)
    assert st == 0, det
    case.check_out_flags(1)


def test_full_size():
    """The combine at the MoE workload, after the full-size dispatch and
    grouped GEMM: every reverse put bit-exact (a copy of the GPU's own y
    rows), and every token of `out` against the oracle's chain (dispatch,
    grouped GEMM, combine) within the GEMM bound plus fp32 rounding of the
    gate-weighted sum."""
    cfg = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]
    case = CombineCase(cfg)
    case.set_in_flags(1)
    case.out.fill_(float("nan"))
    for r in case.ret_out:
        if r is not None:
            r.fill_(float("nan"))
    st, det = case.run(1)
    assert st == 0, det
    y_ref, rc, ret_out_ref, out_ref = case.reference()
    y_gpu = host(case.a2a.y)
    for s in range(cfg.ranks):
        if s == cfg.rank:
            continue
        n = int(rc[s].sum())
        got = host(case.ret_out[s])
        assert np.array_equal(got[:n].view(np.uint32), y_gpu[s, :n].view(np.uint32)), f"reverse put to {s}"
        assert np.isnan(got[n:]).all(), f"rows past the count sent to {s}"
    case.check_out_flags(1)
    out = host(case.out)
    assert np.isfinite(out).all()
    tol = gemm_tol(cfg.hidden, float(np.abs(y_ref).max())) + 1e-5 * float(np.abs(out_ref).max())
    assert max_err(out, out_ref) <= tol
