"""Race evidence on the CPU: the signal protocols of the library, modelled with
std::thread and C++ release/acquire atomics (tests/protocol_model.cpp) and
run under ThreadSanitizer.

The model moves the data with plain loads and stores, so any consumer read
that the protocol does not order after its producer's write is a data race
ThreadSanitizer reports, whatever the timing ("Triton-distributed
Semantics", Token-Based Data Dependency: a load hoisted above its wait is
the bug to rule out).  The AllGather -> GEMM model is driven by the
library's own plan tables: its unit geometry, seeded producer orders, and
the consumer order from the library's host mirror of its device rule
(ag_gemm_consumer_order).  Each planted protocol bug (a wait skipped, a flag
set before the copy, relaxed ordering, an arrival before its copy) must be
reported; the real protocols must run clean, over several epochs without a
reset, with random pauses."""

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "protocol_model.cpp")
TSAN_OPTIONS = "halt_on_error=0 exitcode=66 report_signal_unsafe=0"


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("model") / "protocol_model")
    subprocess.run([cxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC, "-o", exe], check=True)
    return exe


def _run(exe, text, tmp_path, mutation=None):
    inp = tmp_path / "input.txt"
    inp.write_text(text)
    env = dict(os.environ, TSAN_OPTIONS=TSAN_OPTIONS)
    cmd = [exe, str(inp)] + ([mutation] if mutation else [])
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    return r.returncode, r.stderr


def _consumer_order(plan, order):
    lib = ovl().lib()
    out = np.zeros(plan.row_tiles, dtype=np.int32)
    o32 = np.ascontiguousarray(order, dtype=np.int32)
    assert lib.ag_gemm_consumer_order(plan.handle, ctypes.c_void_p(o32.ctypes.data),
                                      ctypes.c_void_p(out.ctypes.data)) == 0
    return out


def _ag_input(R=4, rank=1, shard_m=128, K=96, N=40, tile_m=32, tile_n=16, tpf=2, W=1, P=3, C=4, epochs=3,
              seed=7):
    """The model's input from the library's plan of the same problem: the
    flag units, seeded producer orders (new per epoch) and, for each, the
    consumer order of the plan's row tiles (rows of the plan's consumer
    tile; rank 1's rows form row tile 1, an own tile)."""
    o = ovl()
    plan = o.ag_gemm_plan(R, rank, shard_m, K, N, tile_m, tile_n, tpf, 8)
    unit_rows = min(tile_m, shard_m)
    panels = -(-shard_m // unit_rows)
    batch_cols = min(K, tpf * tile_n) if tpf else K
    batches = -(-K // batch_cols)
    assert plan.num_units == R * panels * batches
    assert plan.row_tiles == -(-R * shard_m // plan.tile_rows)
    lines = [f"ag {R} {rank} {shard_m} {K} {N} {unit_rows} {panels} {batch_cols} {batches} "
             f"{plan.tile_rows} 16 {W} {P} {C} {epochs} {seed}"]
    for e in range(1, epochs + 1):
        order = synth.producer_order(seed, e, R * panels, batches, True, "units")
        lines.append(" ".join(map(str, order.tolist())))
        lines.append(" ".join(map(str, _consumer_order(plan, order).tolist())))
    return "\n".join(lines) + "\n"


def test_ag_protocol_is_race_free(model, tmp_path):
    rc, err = _run(model, _ag_input(), tmp_path)
    assert "ThreadSanitizer" not in err, err[-3000:]
    assert rc == 0, err[-2000:]


def test_ag_split_unit_arrivals_are_race_free(model, tmp_path):
    """Four workgroups per unit, arrivals on a monotone counter (signal
    ADD), the arrival completing a multiple of four publishes (SET)."""
    rc, err = _run(model, _ag_input(W=4, P=5), tmp_path)
    assert "ThreadSanitizer" not in err, err[-3000:]
    assert rc == 0, err[-2000:]


@pytest.mark.parametrize("mutation,W", [("skip_wait", 1), ("publish_early", 1), ("relaxed", 1),
                                        ("add_no_release", 4)])
def test_ag_planted_protocol_bugs_are_reported(model, tmp_path, mutation, W):
    rc, err = _run(model, _ag_input(W=W, P=5 if W > 1 else 3), tmp_path, mutation)
    assert "WARNING: ThreadSanitizer: data race" in err, (rc, err[-2000:])


def _a2a_input(R=4, rank=2, T=48, H=8, N=6, topk=2, E=3, chunk=4, tile=8, P=2, C=3, seed=11):
    x, topk_idx, _ = synth.dispatch_inputs(
        synth.DispatchCfg("model", R, T, 8, 8, topk, R * E, E, 1.1, 1.0, 0.25, seed, rank))
    lines = [f"a2a {R} {rank} {T} {H} {N} {topk} {E} {chunk} {tile} {P} {C} {seed}"]
    for s in range(R):
        lines.append(" ".join(map(str, np.asarray(topk_idx[s]).reshape(-1).tolist())))
    return "\n".join(lines) + "\n"


def test_dispatch_protocol_is_race_free(model, tmp_path):
    rc, err = _run(model, _a2a_input(), tmp_path)
    assert "ThreadSanitizer" not in err, err[-3000:]
    assert rc == 0, err[-2000:]


def test_dispatch_arrival_before_copy_is_reported(model, tmp_path):
    rc, err = _run(model, _a2a_input(), tmp_path, "arrive_early")
    assert "WARNING: ThreadSanitizer: data race" in err, (rc, err[-2000:])


RS_INPUT = "rs 4 1 40 24 36 16 3 5\n"


def test_gemm_rs_protocol_is_race_free(model, tmp_path):
    rc, err = _run(model, RS_INPUT, tmp_path)
    assert "ThreadSanitizer" not in err, err[-3000:]
    assert rc == 0, err[-2000:]


def test_gemm_rs_reduce_without_own_wait_is_reported(model, tmp_path):
    rc, err = _run(model, RS_INPUT, tmp_path, "no_own_wait")
    assert "WARNING: ThreadSanitizer: data race" in err, (rc, err[-2000:])
