"""The allocation-free AG-GEMM call (ag_gemm_run_noalloc) against the
workspace call (ag_gemm_run) through the C-ABI: the same gathered bits, flag
bytes and C bits on the same inputs, and C within the oracle's bound, on
calls in a row whose second is smaller (the library's scratch keeps the
first call's contents, and what must start at zero is cleared by the call)."""

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


def _cfg(name, R, Ms, K, N, tm, tn, seed):
    return synth.AgGemmCfg(name, R, Ms, K, N, tm, tn, 1.0, 1.0 / 16, seed, True)


def _run_both(cfg, tpf, epoch=1, unit_producers=1):
    """Runs the workspace call and the allocation-free call on the same
    inputs and order; returns both results and the oracle's C."""
    o = ovl()
    shards, b = synth.ag_inputs(cfg)
    plan = o.ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, tpf, 8, unit_producers)
    units, panels, batches = oracle.ag_flag_units(cfg.ranks, cfg.shard_m, cfg.k, cfg.tile_m, cfg.tile_n, tpf)
    order = dev(synth.producer_order(cfg.seed, epoch, cfg.ranks * panels, batches, True, "units"))
    d_shards, d_b = [dev(s) for s in shards], dev(b)
    out = []
    for noalloc in (False, True):
        g = zeros_u16(cfg.m, cfg.k)
        g.fill_(0x7FC0)  # NaN: an early read shows
        c = zeros_f32(cfg.m, cfg.n)
        flags = zeros_bytes(plan.flags_bytes)
        o.ovl_flags_reset(flags, plan.flags_bytes, None, 0)  # a new flag buffer: epochs start at 1
        say(f"  {cfg.name} splits={plan.splits} noalloc={noalloc}")
        if noalloc:
            o.ag_gemm_run_noalloc(plan, d_shards, d_b, g, c, flags, epoch, order)
            st, det = o.ovl_check(None, raise_on_error=False)
        else:
            ws = zeros_bytes(plan.workspace_bytes)
            o.ag_gemm_run(plan, d_shards, d_b, g, c, flags, ws, epoch, order)
            st, det = o.ovl_check(ws, raise_on_error=False)
        assert st == 0, det
        out.append((host(g, np.uint16), host(c), host(flags)[: plan.flags_bytes]))
    _, c_ref = oracle.ag_gemm(shards, b)
    expected_flags = oracle.expected_flags(units, 8, epoch)
    return plan, out, c_ref, oracle.all_gather(shards), expected_flags


def _check(cfg, plan, out, c_ref, g_ref, f_ref):
    (g0, c0, f0), (g1, c1, f1) = out
    assert np.array_equal(g1, g0) and np.array_equal(g1, g_ref)
    assert np.array_equal(f1, f0) and np.array_equal(f1, f_ref)
    assert np.array_equal(c1.view(np.uint32), c0.view(np.uint32)), "C differs from the workspace call"
    assert max_err(c1, c_ref) <= gemm_tol(cfg.k, float(np.abs(c_ref).max()))


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    # 1: split K in 8 ranges (128 x 2048 output, K = 4096): the partials and
    #    counters live in the scratch.
    big = _cfg("noalloc_split8", 8, 16, 4096, 2048, 16, 256, seed=51)
    plan, out, c_ref, g_ref, f_ref = _run_both(big, tpf=2)
    assert plan.splits == 8
    _check(big, plan, out, c_ref, g_ref, f_ref)
    # 2: a smaller split plan (64 x 512 output, K = 1024 in 4 ranges): the
    #    scratch still holds call 1's partials beyond its own.
    small = _cfg("noalloc_split4", 2, 32, 1024, 512, 32, 128, seed=52)
    plan, out, c_ref, g_ref, f_ref = _run_both(small, tpf=1)
    assert 1 < plan.splits < 8
    _check(small, plan, out, c_ref, g_ref, f_ref)
    # 3: smaller still, no split (the R = 2 128 x 256 x 256 workload).
    tiny = synth.CONFIGS["ag_r2_128x256x256"]
    plan, out, c_ref, g_ref, f_ref = _run_both(tiny, tpf=1)
    assert plan.splits == 1
    _check(tiny, plan, out, c_ref, g_ref, f_ref)


def test_noalloc_reports_a_timeout_in_its_own_record_and_recovers():
    """A unit left out of the producer order: the allocation-free call's
    waits give up into the scratch's error record (ovl_check(NULL)); the next
    call clears it and succeeds."""
    o = ovl()
    cfg = synth.CONFIGS["ag_r2_128x256x256"]
    shards, b = synth.ag_inputs(cfg)
    plan = o.ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n, 0, 8)
    order = np.arange(plan.num_units, dtype=np.int32)
    order[-1] = -1
    g, c = zeros_u16(cfg.m, cfg.k), zeros_f32(cfg.m, cfg.n)
    flags = zeros_bytes(plan.flags_bytes)
    o.ovl_flags_reset(flags, plan.flags_bytes, None, 0)
    d_shards, d_b = [dev(s) for s in shards], dev(b)
    say("  noalloc with a missing unit")
    o.ag_gemm_run_noalloc(plan, d_shards, d_b, g, c, flags, 1, dev(order), spin_limit=2000)
    st, det = o.ovl_check(None, raise_on_error=False)
    assert st == o.OVL_ETIMEOUT and det[1] == plan.num_units - 1, det
    o.ovl_flags_reset(flags, plan.flags_bytes, None, 0)
    o.ag_gemm_run_noalloc(plan, d_shards, d_b, g, c, flags, 1, None)
    st, det = o.ovl_check(None, raise_on_error=False)
    assert st == 0, det
    _, c_ref = oracle.ag_gemm(shards, b)
    assert max_err(host(c), c_ref) <= gemm_tol(cfg.k, float(np.abs(c_ref).max()))


def test_noalloc_split_units_start_their_counters_at_zero():
    """Several producers per unit: the arrival counters live in the scratch,
    which the previous call (with another producer count) left behind; each
    call clears them, so calls with 4, then 3 producers per unit both match
    the workspace call."""
    cfg = _cfg("noalloc_units", 4, 300, 512, 768, 64, 128, seed=53)
    for W in (4, 3):
        plan, out, c_ref, g_ref, f_ref = _run_both(cfg, tpf=1, unit_producers=W)
        _check(cfg, plan, out, c_ref, g_ref, f_ref)
