"""ctypes binding of libovl.so: the same entry points as include/ovl.h.

Argument marshalling only.  Tensors are passed as raw device pointers
(their data_ptr()), streams as their HIP handle; every step of the path runs
in the library's kernels.  There is no fallback: if the library is missing,
loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, byref, c_char_p, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libovl.so")

OVL_OK = 0
OVL_EINVAL = -1
OVL_ESHAPE = -2
OVL_EALIGN = -3
OVL_EEPOCH = -4
OVL_EHIP = -5
OVL_ETIMEOUT = -6
OVL_EUNSUPPORTED = -7

MODE_FUSED = 0
MODE_COPY_ONLY = 1
MODE_GEMM_ONLY = 2
MODE_BARRIER = 3

ERROR_RECORD_BYTES = 64

EXPORTS = (
    "ag_gemm_plan", "ag_gemm_plan_destroy", "ag_gemm_num_units", "ag_gemm_flags_bytes",
    "ag_gemm_workspace_bytes", "ag_gemm_splits", "ag_gemm_run",
    "gemm_rs_flags_bytes", "gemm_rs_workspace_bytes", "gemm_rs_run",
    "a2a_flags_bytes", "a2a_workspace_bytes", "a2a_trace_bytes", "a2a_dispatch_grouped_gemm_run",
    "a2a_combine_flags_bytes", "a2a_combine_workspace_bytes", "a2a_combine_run",
    "ovl_flags_reset", "ovl_check", "ovl_strerror", "ovl_copy",
    "ring_allreduce_flags_bytes", "ring_allreduce_workspace_bytes", "ring_allreduce_run",
    "fp8_quantize_rows", "a2a_dispatch_grouped_gemm_fp8_run", "ag_gemm_trace_bytes",
    "ag_gemm_row_tiles", "ag_gemm_tile_rows", "ag_gemm_consumer_order", "ag_gemm_run_noalloc",
)


class OvlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


class Opts(Structure):
    _fields_ = [("mode", c_uint32), ("producers", c_uint32), ("spin_limit", c_uint64), ("trace", c_void_p),
                ("jitter", c_uint32), ("reserved", c_uint32)]


class AgGemmDesc(Structure):
    _fields_ = [("ranks", c_int32), ("rank", c_int32), ("shard_m", c_int64), ("k", c_int64), ("n", c_int64),
                ("tile_m", c_int32), ("tile_n", c_int32), ("tiles_per_flag", c_int32), ("flag_stride", c_int32),
                ("unit_producers", c_int32)]


class GemmRsDesc(Structure):
    _fields_ = [("ranks", c_int32), ("rank", c_int32), ("m", c_int64), ("n", c_int64), ("k", c_int64),
                ("tile_m", c_int32), ("tile_n", c_int32), ("flag_stride", c_int32)]


class A2aDesc(Structure):
    _fields_ = [("ranks", c_int32), ("rank", c_int32), ("tokens", c_int64), ("hidden", c_int64), ("n", c_int64),
                ("topk", c_int32), ("num_experts", c_int32), ("experts_per_rank", c_int32),
                ("flag_stride", c_int32), ("tile_m", c_int32), ("tile_n", c_int32)]


class RingDesc(Structure):
    _fields_ = [("ranks", c_int32), ("n", c_int64), ("tile", c_int64), ("flag_stride", c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libovl.so once (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m communication_overlap_amd.build`")
    import torch  # noqa: F401  (loads the HIP runtime the library links against)
    L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    st = c_int32
    L.ag_gemm_plan.argtypes = [POINTER(AgGemmDesc), POINTER(c_void_p)]
    L.ag_gemm_plan.restype = st
    L.ag_gemm_plan_destroy.argtypes = [c_void_p]
    L.ag_gemm_plan_destroy.restype = st
    L.ag_gemm_num_units.argtypes = [c_void_p]
    L.ag_gemm_num_units.restype = c_int64
    L.ag_gemm_flags_bytes.argtypes = [c_void_p]
    L.ag_gemm_flags_bytes.restype = c_size_t
    L.ag_gemm_workspace_bytes.argtypes = [c_void_p]
    L.ag_gemm_workspace_bytes.restype = c_size_t
    L.ag_gemm_splits.argtypes = [c_void_p]
    L.ag_gemm_splits.restype = c_int32
    L.ag_gemm_trace_bytes.argtypes = [c_void_p]
    L.ag_gemm_trace_bytes.restype = c_size_t
    L.ag_gemm_row_tiles.argtypes = [c_void_p]
    L.ag_gemm_row_tiles.restype = c_int32
    L.ag_gemm_tile_rows.argtypes = [c_void_p]
    L.ag_gemm_tile_rows.restype = c_int32
    L.ag_gemm_run.argtypes = [c_void_p, POINTER(c_void_p), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_int64, c_void_p, POINTER(Opts), c_void_p]
    L.ag_gemm_run.restype = st
    L.ag_gemm_run_noalloc.argtypes = [c_void_p, POINTER(c_void_p), c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int64, c_void_p, POINTER(Opts), c_void_p]
    L.ag_gemm_run_noalloc.restype = st
    L.gemm_rs_flags_bytes.argtypes = [POINTER(GemmRsDesc)]
    L.gemm_rs_flags_bytes.restype = c_size_t
    L.gemm_rs_workspace_bytes.argtypes = [POINTER(GemmRsDesc)]
    L.gemm_rs_workspace_bytes.restype = c_size_t
    L.gemm_rs_run.argtypes = [POINTER(GemmRsDesc), c_void_p, c_void_p, POINTER(c_void_p), POINTER(c_void_p),
                              c_void_p, c_void_p, c_void_p, c_void_p, c_int64, POINTER(Opts), c_void_p]
    L.gemm_rs_run.restype = st
    L.a2a_flags_bytes.argtypes = [POINTER(A2aDesc)]
    L.a2a_flags_bytes.restype = c_size_t
    L.a2a_workspace_bytes.argtypes = [POINTER(A2aDesc)]
    L.a2a_workspace_bytes.restype = c_size_t
    L.a2a_trace_bytes.argtypes = [POINTER(A2aDesc)]
    L.a2a_trace_bytes.restype = c_size_t
    L.a2a_dispatch_grouped_gemm_run.argtypes = [POINTER(A2aDesc), POINTER(c_void_p), POINTER(c_void_p), c_void_p,
                                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_int64, POINTER(Opts), c_void_p]
    L.a2a_dispatch_grouped_gemm_run.restype = st
    L.a2a_combine_flags_bytes.argtypes = [POINTER(A2aDesc)]
    L.a2a_combine_flags_bytes.restype = c_size_t
    L.a2a_combine_workspace_bytes.argtypes = [POINTER(A2aDesc)]
    L.a2a_combine_workspace_bytes.restype = c_size_t
    L.a2a_combine_run.argtypes = [POINTER(A2aDesc), c_void_p, c_void_p, POINTER(c_void_p), POINTER(c_void_p),
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                  POINTER(Opts), c_void_p]
    L.a2a_combine_run.restype = st
    L.ovl_flags_reset.argtypes = [c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    L.ovl_flags_reset.restype = st
    L.ovl_check.argtypes = [c_void_p, POINTER(c_int64), c_void_p]
    L.ovl_check.restype = st
    L.ovl_strerror.argtypes = [c_int32]
    L.ovl_strerror.restype = c_char_p
    L.ovl_copy.argtypes = [c_void_p, c_void_p, c_size_t, c_int32, c_void_p]
    L.ovl_copy.restype = st
    L.ring_allreduce_flags_bytes.argtypes = [POINTER(RingDesc)]
    L.ring_allreduce_flags_bytes.restype = c_size_t
    L.ring_allreduce_workspace_bytes.argtypes = [POINTER(RingDesc)]
    L.ring_allreduce_workspace_bytes.restype = c_size_t
    L.ring_allreduce_run.argtypes = [POINTER(RingDesc), POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_void_p,
                                     c_int64, POINTER(Opts), c_void_p]
    L.ring_allreduce_run.restype = st
    L.fp8_quantize_rows.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p]
    L.fp8_quantize_rows.restype = st
    L.a2a_dispatch_grouped_gemm_fp8_run.argtypes = [POINTER(A2aDesc), POINTER(c_void_p), POINTER(c_void_p),
                                                    POINTER(c_void_p), c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                                    POINTER(Opts), c_void_p]
    L.a2a_dispatch_grouped_gemm_fp8_run.restype = st
    _lib = L
    return L


def strerror(status: int) -> str:
    try:
        return lib().ovl_strerror(status).decode()
    except ImportError:
        return f"status {status}"


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _opts(mode: int, producers: int, spin_limit: int, trace=None, jitter: int = 0) -> Opts:
    return Opts(mode, producers, spin_limit, _ptr(trace), jitter, 0)


def _check(status: int, where: str, raise_on_error: bool) -> int:
    if status != OVL_OK and raise_on_error:
        raise OvlError(status, where)
    return status


def _ptr_array(ts):
    arr = (c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


# ------------------------------------------------------------------ AG-GEMM

class AgGemmPlan:
    """Owns an ag_gemm_plan_t."""

    def __init__(self, ranks, rank, shard_m, k, n, tile_m, tile_n, tiles_per_flag=0, flag_stride=8,
                 unit_producers=1):
        self.desc = AgGemmDesc(ranks, rank, shard_m, k, n, tile_m, tile_n, tiles_per_flag, flag_stride,
                               unit_producers)
        h = c_void_p()
        _check(lib().ag_gemm_plan(byref(self.desc), byref(h)), "ag_gemm_plan", True)
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.ag_gemm_plan_destroy(h)
            self.handle = None

    @property
    def num_units(self) -> int:
        return lib().ag_gemm_num_units(self.handle)

    @property
    def flags_bytes(self) -> int:
        return lib().ag_gemm_flags_bytes(self.handle)

    @property
    def workspace_bytes(self) -> int:
        return lib().ag_gemm_workspace_bytes(self.handle)

    @property
    def splits(self) -> int:
        return lib().ag_gemm_splits(self.handle)

    @property
    def trace_bytes(self) -> int:
        return lib().ag_gemm_trace_bytes(self.handle)

    @property
    def tile_rows(self) -> int:
        """Rows of the consumer's output tile (chosen by the library)."""
        return lib().ag_gemm_tile_rows(self.handle)

    @property
    def row_tiles(self) -> int:
        return lib().ag_gemm_row_tiles(self.handle)


def ag_gemm_plan(*args, **kw) -> AgGemmPlan:
    return AgGemmPlan(*args, **kw)


def ag_gemm_run(plan: AgGemmPlan, shards, b, gathered, c, flags, workspace, epoch: int, producer_order=None,
                mode: int = MODE_FUSED, producers: int = 0, spin_limit: int = 0, stream=None,
                raise_on_error: bool = True, trace=None, jitter: int = 0) -> int:
    arr = _ptr_array(shards)
    o = _opts(mode, producers, spin_limit, trace, jitter)
    st = lib().ag_gemm_run(plan.handle, arr, _ptr(b), _ptr(gathered), _ptr(c), _ptr(flags), _ptr(workspace),
                           epoch, _ptr(producer_order), byref(o), _stream(stream))
    return _check(st, "ag_gemm_run", raise_on_error)


def ag_gemm_run_noalloc(plan: AgGemmPlan, shards, b, gathered, c, flags, epoch: int, producer_order=None,
                        mode: int = MODE_FUSED, producers: int = 0, spin_limit: int = 0, stream=None,
                        raise_on_error: bool = True, trace=None, jitter: int = 0) -> int:
    arr = _ptr_array(shards)
    o = _opts(mode, producers, spin_limit, trace, jitter)
    st = lib().ag_gemm_run_noalloc(plan.handle, arr, _ptr(b), _ptr(gathered), _ptr(c), _ptr(flags), epoch,
                                   _ptr(producer_order), byref(o), _stream(stream))
    return _check(st, "ag_gemm_run_noalloc", raise_on_error)


# ------------------------------------------------------------------ GEMM-RS

def gemm_rs_desc(ranks, rank, m, n, k, tile_m=256, tile_n=256, flag_stride=8) -> GemmRsDesc:
    return GemmRsDesc(ranks, rank, m, n, k, tile_m, tile_n, flag_stride)


def gemm_rs_flags_bytes(desc: GemmRsDesc) -> int:
    return lib().gemm_rs_flags_bytes(byref(desc))


def gemm_rs_workspace_bytes(desc: GemmRsDesc) -> int:
    return lib().gemm_rs_workspace_bytes(byref(desc))


def gemm_rs_run(desc: GemmRsDesc, a, b, peer_out, peer_in, out, out_flags, in_flags, workspace, epoch: int,
                mode: int = MODE_FUSED, producers: int = 0, spin_limit: int = 0, stream=None,
                raise_on_error: bool = True) -> int:
    o = _opts(mode, producers, spin_limit)
    st = lib().gemm_rs_run(byref(desc), _ptr(a), _ptr(b), _ptr_array(peer_out), _ptr_array(peer_in), _ptr(out),
                           _ptr(out_flags), _ptr(in_flags), _ptr(workspace), epoch, byref(o), _stream(stream))
    return _check(st, "gemm_rs_run", raise_on_error)


# ------------------------------------------------------------------ dispatch + grouped GEMM

def a2a_desc(ranks, rank, tokens, hidden, n, topk, num_experts, experts_per_rank, flag_stride=8,
             tile_m=0, tile_n=0) -> A2aDesc:
    return A2aDesc(ranks, rank, tokens, hidden, n, topk, num_experts, experts_per_rank, flag_stride, tile_m, tile_n)


def a2a_flags_bytes(desc: A2aDesc) -> int:
    return lib().a2a_flags_bytes(byref(desc))


def a2a_workspace_bytes(desc: A2aDesc) -> int:
    return lib().a2a_workspace_bytes(byref(desc))


def a2a_trace_bytes(desc: A2aDesc) -> int:
    return lib().a2a_trace_bytes(byref(desc))


def a2a_dispatch_grouped_gemm_run(desc: A2aDesc, x, topk_idx, w, recv_x, recv_src, recv_count, y, flags,
                                  workspace, epoch: int, mode: int = MODE_FUSED, producers: int = 0,
                                  spin_limit: int = 0, stream=None, raise_on_error: bool = True, trace=None) -> int:
    o = _opts(mode, producers, spin_limit, trace)
    st = lib().a2a_dispatch_grouped_gemm_run(byref(desc), _ptr_array(x), _ptr_array(topk_idx), _ptr(w),
                                             _ptr(recv_x), _ptr(recv_src), _ptr(recv_count), _ptr(y), _ptr(flags),
                                             _ptr(workspace), epoch, byref(o), _stream(stream))
    return _check(st, "a2a_dispatch_grouped_gemm_run", raise_on_error)


def fp8_quantize_rows(in_bf16, codes, scale, rows: int, cols: int, stream=None, raise_on_error: bool = True) -> int:
    st = lib().fp8_quantize_rows(_ptr(in_bf16), _ptr(codes), _ptr(scale), rows, cols, _stream(stream))
    return _check(st, "fp8_quantize_rows", raise_on_error)


def a2a_dispatch_grouped_gemm_fp8_run(desc: A2aDesc, x8, x_scale, topk_idx, w8, w_scale, recv_x8, recv_scale,
                                      recv_src, recv_count, y, flags, workspace, epoch: int, mode: int = MODE_FUSED,
                                      producers: int = 0, spin_limit: int = 0, stream=None,
                                      raise_on_error: bool = True, trace=None) -> int:
    o = _opts(mode, producers, spin_limit, trace)
    st = lib().a2a_dispatch_grouped_gemm_fp8_run(byref(desc), _ptr_array(x8), _ptr_array(x_scale),
                                                 _ptr_array(topk_idx), _ptr(w8), _ptr(w_scale), _ptr(recv_x8),
                                                 _ptr(recv_scale), _ptr(recv_src), _ptr(recv_count), _ptr(y),
                                                 _ptr(flags), _ptr(workspace), epoch, byref(o), _stream(stream))
    return _check(st, "a2a_dispatch_grouped_gemm_fp8_run", raise_on_error)


def a2a_combine_flags_bytes(desc: A2aDesc) -> int:
    return lib().a2a_combine_flags_bytes(byref(desc))


def a2a_combine_workspace_bytes(desc: A2aDesc) -> int:
    return lib().a2a_combine_workspace_bytes(byref(desc))


def a2a_combine_run(desc: A2aDesc, y, recv_count, ret_out, ret_in, topk_idx, gates, out, out_flags, in_flags,
                    workspace, epoch: int, mode: int = MODE_FUSED, spin_limit: int = 0, stream=None,
                    raise_on_error: bool = True) -> int:
    o = _opts(mode, 0, spin_limit)
    st = lib().a2a_combine_run(byref(desc), _ptr(y), _ptr(recv_count), _ptr_array(ret_out), _ptr_array(ret_in),
                               _ptr(topk_idx), _ptr(gates), _ptr(out), _ptr(out_flags), _ptr(in_flags),
                               _ptr(workspace), epoch, byref(o), _stream(stream))
    return _check(st, "a2a_combine_run", raise_on_error)


# ------------------------------------------------------------------ ring all-reduce

def ring_desc(ranks, n, tile, flag_stride=8) -> RingDesc:
    return RingDesc(ranks, n, tile, flag_stride)


def ring_allreduce_flags_bytes(desc: RingDesc) -> int:
    return lib().ring_allreduce_flags_bytes(byref(desc))


def ring_allreduce_workspace_bytes(desc: RingDesc) -> int:
    return lib().ring_allreduce_workspace_bytes(byref(desc))


def ring_allreduce_run(desc: RingDesc, inputs, outputs, flags, workspace, epoch: int, mode: int = MODE_FUSED,
                       spin_limit: int = 0, stream=None, raise_on_error: bool = True) -> int:
    o = _opts(mode, 0, spin_limit)
    st = lib().ring_allreduce_run(byref(desc), _ptr_array(inputs), _ptr_array(outputs), _ptr(flags),
                                  _ptr(workspace), epoch, byref(o), _stream(stream))
    return _check(st, "ring_allreduce_run", raise_on_error)


# ------------------------------------------------------------------ flags, errors, copy

def ovl_flags_reset(flags, flag_bytes: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().ovl_flags_reset(_ptr(flags), flag_bytes, _ptr(workspace), ws_bytes, _stream(stream)),
           "ovl_flags_reset", True)


def ovl_check(workspace, stream=None, raise_on_error: bool = True):
    """Returns (status, (site, flag index, observed, awaited))."""
    detail = (c_int64 * 4)()
    st = lib().ovl_check(_ptr(workspace), detail, _stream(stream))
    _check(st, "ovl_check", raise_on_error)
    return st, tuple(detail)


def ovl_copy(dst, src, nbytes: int, blocks: int = 0, stream=None) -> None:
    _check(lib().ovl_copy(_ptr(dst), _ptr(src), nbytes, blocks, _stream(stream)), "ovl_copy", True)
