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
    bad, n, _ = ec.check_asm(ec.device_asm(HIPCC, src, _flags()))
    return os.path.basename(src), bad, n


def test_every_library_barrier_runs_with_full_exec():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ProcessPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(_compile_and_check, srcs))
    report = [f"{name}: {fn}: asm lines {[ln for ln, _ in sites]}"
              for name, bad, _ in results for fn, sites in bad.items()]
    assert not report, "barriers under a partial EXEC:\n" + "\n".join(report)
    # The kernels that synchronise workgroups were all seen.
    seen = {name: n for name, _, n in results}
    for name in ("ag_gemm.hip", "a2a.hip", "gemm_rs.hip", "combine.hip", "ring.hip"):
        assert seen[name] > 0, name


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
