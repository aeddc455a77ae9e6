"""GPU parity of the ring all-reduce with per-tile signals against the
oracle's step-by-step ring simulation, through the C-ABI: every rank's
output bit-exact (the float32 sums are formed in the ring's order on both
sides), every flag slot holding the epoch, FUSED and BARRIER alike."""

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, host, say, zeros_bytes

pytestmark = pytest.mark.gpu


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


class RingCase:
    def __init__(self, R, n, tile, inputs=None, seed=11, kind="normal", flag_stride=8):
        import torch
        o = ovl()
        self.R, self.n = R, n
        cfg = synth.RingCfg("case", R, n, tile, 1.0, seed)
        self.x = inputs if inputs is not None else synth.ring_inputs(cfg, kind)
        self.desc = o.ring_desc(R, n, tile, flag_stride)
        self.d_in = [dev(v) for v in self.x]
        self.d_out = [torch.zeros(max(n, 4), dtype=torch.float32, device="cuda") for _ in range(R)]
        self.fbytes = o.ring_allreduce_flags_bytes(self.desc)
        self.flags = zeros_bytes(self.fbytes)
        self.ws = zeros_bytes(o.ring_allreduce_workspace_bytes(self.desc))
        o.ovl_flags_reset(self.flags, self.fbytes, self.ws, self.ws.numel())
        self.stride = flag_stride // 8

    def run(self, epoch, mode=0, spin_limit=0):
        o = ovl()
        say(f"[ring] R={self.R} n={self.n} tile={self.desc.tile} epoch={epoch} mode={mode}")
        o.ring_allreduce_run(self.desc, self.d_in, self.d_out, self.flags, self.ws, epoch, mode=mode,
                             spin_limit=spin_limit)
        return o.ovl_check(self.ws, raise_on_error=False)

    def outputs(self):
        return [host(t)[: self.n] for t in self.d_out]

    def check(self, epoch):
        ref = oracle.ring_allreduce(self.x)
        for r, got in enumerate(self.outputs()):
            assert np.array_equal(got.view(np.uint32), ref[r].view(np.uint32)), f"rank {r}"
        fl = host(self.flags)[: self.fbytes].view(np.int64)[:: self.stride]
        assert np.all(fl == epoch), np.unique(fl)


@pytest.mark.parametrize("R,n,tile", [
    (2, 64, 16),
    (3, 101, 8),      # odd length: a lone last element
    (5, 1000, 32),    # ragged tiles
    (8, 7, 2),        # empty chunks
    (8, 4099, 64),
    (4, 4096, 4096),  # one tile per chunk
])
@pytest.mark.parametrize("mode", [0, 3])
def test_matches_ring_oracle_bit_exact(R, n, tile, mode):
    case = RingCase(R, n, tile)
    st, det = case.run(1, mode)
    assert st == 0, det
    case.check(1)


def test_ring_order_on_the_device():
    x = [np.ones(6, dtype=np.float32) for _ in range(3)]
    for c, (lo, hi) in enumerate(oracle.ring_chunk_bounds(6, 3)):
        x[(c + 2) % 3][lo:hi] = 2.0 ** 24
    case = RingCase(3, 6, 2, inputs=x)
    assert case.run(1)[0] == 0
    for got in case.outputs():
        assert np.all(got == np.float32(2.0 ** 24 + 2))


def test_small_integers_exact_and_epochs_continue_without_reset():
    case = RingCase(6, 3000, 128, kind="smallint", flag_stride=64)
    ref = np.sum(np.stack(case.x).astype(np.int64), axis=0)
    for epoch, mode in ((1, 0), (2, 3), (3, 0)):
        for t in case.d_out:
            t.zero_()
        st, det = case.run(epoch, mode)
        assert st == 0, det
        for got in case.outputs():
            assert np.array_equal(got.astype(np.int64), ref)
        case.check(epoch)


def test_one_rank_copies_and_empty_vectors_do_nothing():
    case = RingCase(1, 333, 16)
    assert case.run(1)[0] == 0
    assert np.array_equal(case.outputs()[0].view(np.uint32), case.x[0].view(np.uint32))
    empty = RingCase(4, 0, 16, inputs=[np.zeros(0, np.float32)] * 4)
    assert empty.run(1)[0] == 0


def test_argument_errors():
    import torch
    o = ovl()
    case = RingCase(3, 100, 10)
    assert o.ring_allreduce_run(case.desc, case.d_in, case.d_out, case.flags, case.ws, 0,
                                raise_on_error=False) == o.OVL_EEPOCH
    inplace = list(case.d_in)
    assert o.ring_allreduce_run(case.desc, case.d_in, inplace, case.flags, case.ws, 1,
                                raise_on_error=False) == o.OVL_EINVAL
    shared = [case.d_out[0]] * 3
    assert o.ring_allreduce_run(case.desc, case.d_in, shared, case.flags, case.ws, 1,
                                raise_on_error=False) == o.OVL_EINVAL
    bad_tile = o.ring_desc(3, 100, 7)
    assert o.ring_allreduce_run(bad_tile, case.d_in, case.d_out, case.flags, case.ws, 1,
                                raise_on_error=False) == o.OVL_ESHAPE
    assert o.ring_allreduce_run(case.desc, case.d_in, case.d_out, case.flags, case.ws, 1, mode=o.MODE_GEMM_ONLY,
                                raise_on_error=False) == o.OVL_EINVAL
    # nothing was enqueued by the refused calls: the epoch sequence is untouched
    assert case.run(1)[0] == 0
    case.check(1)
    del torch


def test_full_size_bit_exact():
    cfg = synth.CONFIGS["ring_r8_n8m"]
    case = RingCase(cfg.ranks, cfg.n, cfg.tile, inputs=synth.ring_inputs(cfg))
    st, det = case.run(1)
    assert st == 0, det
    case.check(1)
    st, det = case.run(2, mode=ovl().MODE_BARRIER)
    assert st == 0, det
    case.check(2)
