"""Every workgroup barrier of the library's kernels runs with the whole
wavefront active: checked on the gfx950 assembly hipcc makes of each source
(the same flags as the library build), with the dataflow of exec_check.py.

A barrier reached while some lanes of a wavefront are masked off counts the
wavefront as arrived, so those lanes fall one barrier behind the rest of the
workgroup.  The compiler can produce that from source that looks correct: a
loop whose every iteration starts and ends with a thread-0 branch can be
threaded into a nested loop in which the other lanes run on through the
barriers while thread 0 takes the outer path (a dispatch ticket loop hung
on exactly this).  The synthetic kernels below pin the check: it reports the
barrier of a thread-0 branch, of a thread-strided loop and of that threaded
ticket loop, and passes the same loop with a barrier after its trailing
thread-0 branch.
"""

import concurrent.futures as cf
import glob
import os
import shutil

import pytest

from tests import exec_check as ec
from tests import kloop_check as kc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_overlap_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


HIPCC = _hipcc()
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not found")


def _flags():
    from communication_overlap_amd import build as B

    return [f for f in B.FLAGS if f not in ("-fPIC", "-Wall")] + ["-w"]


def _compile_and_check(src):
    asm = ec.device_asm(HIPCC, src, _flags())
    bad, n, _ = ec.check_asm(asm)
    waits, loops = kc.kloop_waits(asm)
    return os.path.basename(src), bad, n, waits, loops


@pytest.fixture(scope="module")
def library_checks():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ProcessPoolExecutor(min(8, len(srcs))) as ex:
        return list(ex.map(_compile_and_check, srcs))


def test_every_library_barrier_runs_with_full_exec(library_checks):
    report = [f"{name}: {fn}: asm lines {[ln for ln, _ in sites]}"
              for name, bad, _, _, _ in library_checks for fn, sites in bad.items()]
    assert not report, "barriers under a partial EXEC:\n" + "\n".join(report)
    # The kernels that synchronise workgroups were all seen.
    seen = {name: n for name, _, n, _, _ in library_checks}
    for name in ("ag_gemm.hip", "a2a.hip", "gemm_rs.hip", "combine.hip", "ring.hip"):
        assert seen[name] > 0, name


def test_no_compiler_wait_ahead_of_a_k_step(library_checks):
    """No GEMM K-loop of the library starts a step with a vector-memory wait
    of the compiler's (kloop_check.py says why that loses the prefetch)."""
    report = [f"{name}: {fn}: loop at asm line {ln}: {w}"
              for name, _, _, waits, _ in library_checks for fn, sites in waits.items() for ln, w in sites]
    assert not report, "\n".join(report)
    loops = {name: n for name, _, _, _, n in library_checks}
    # every kernel instantiation's tile loop was found
    for name, least in (("ag_gemm.hip", 9), ("a2a.hip", 8), ("gemm_rs.hip", 4)):
        assert loops[name] >= least, (name, loops[name])


_LOOPS = """
    .type k,@function
k:
    s_mov_b32 s0, 0
.LBB0_1:
    ds_read_b128 v[0:3], v8
    s_waitcnt vmcnt(%s)
    ds_read_b128 v[4:7], v8 offset:16
    v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
    s_waitcnt vmcnt(2)
    s_barrier
    s_cbranch_scc1 .LBB0_1
.LBB0_2:
    s_waitcnt vmcnt(0)
    v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
    s_cbranch_scc0 .LBB0_2
    s_endpgm
.Lfunc_end0:
"""


def test_kloop_check_reports_a_wait_ahead_of_the_first_mfma():
    bad, n = kc.kloop_waits(_LOOPS % "5")
    assert n == 2
    assert [w for _, w in bad["k"]] == [["vmcnt(5)"], ["vmcnt(0)"]]
    # A wait after the step's first MFMA (the step-end wait) is not reported.
    ok = (_LOOPS % "5").replace("    s_waitcnt vmcnt(5)\n", "")
    ok = ok.replace(".LBB0_2:\n    s_waitcnt vmcnt(0)\n", ".LBB0_2:\n")
    assert kc.kloop_waits(ok) == ({}, 2)


SYNTHETIC = r"""
#include <hip/hip_runtime.h>
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__global__ void k_branch(int* out) {
  if (threadIdx.x == 0) { out[0] = 1; __syncthreads(); }
  out[threadIdx.x + 1] = 2;
}

__global__ void k_strided(int* out, int n) {
  __shared__ int s[256];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    s[threadIdx.x] = i;
    __syncthreads();
    out[i] = s[(threadIdx.x + 1) & 255];
  }
}

__global__ void k_ticket_threaded(int* ticket, int* out, int total) {
  __shared__ int sh;
  for (;;) {
    if (threadIdx.x == 0) sh = atomicAdd(ticket, 1);
    __syncthreads();
    const int t = uni(sh);
    __syncthreads();
    if (t >= total) break;
    out[t * blockDim.x + threadIdx.x] = t;
    if (threadIdx.x == 0) atomicAdd(out, 1);
  }
}

__global__ void k_ticket_separated(int* ticket, int* out, int total) {
  __shared__ int sh;
  for (;;) {
    if (threadIdx.x == 0) sh = atomicAdd(ticket, 1);
    __syncthreads();
    const int t = uni(sh);
    __syncthreads();
    if (t >= total) break;
    out[t * blockDim.x + threadIdx.x] = t;
    if (threadIdx.x == 0) atomicAdd(out, 1);
    __syncthreads();
  }
}

__global__ void k_uniform_branch(int* out, int n) {
  __shared__ int s[256];
  if (n > 4) {
    s[threadIdx.x] = n;
    __syncthreads();
  }
  out[threadIdx.x] = s[threadIdx.x ^ 1];
}
"""


def test_checker_reports_planted_divergent_barriers(tmp_path):
    src = tmp_path / "synthetic.hip"
    src.write_text(SYNTHETIC)
    asm = ec.device_asm(HIPCC, str(src), _flags())
    bad, n, nf = ec.check_asm(asm)
    names = {fn: sites for fn, sites in bad.items()}

    def flagged(kernel):
        return any(kernel in fn for fn in names)

    assert nf == 5 and n >= 8
    assert flagged("k_branch")
    assert flagged("k_strided")
    assert flagged("k_ticket_threaded")
    assert not flagged("k_ticket_separated")
    assert not flagged("k_uniform_branch")
