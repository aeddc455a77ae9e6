"""GPU parity of the FP8 path through the C-ABI: the per-row E4M3
quantizer (codes and scales bit-exact against the oracle), and the FP8
dispatch -> FP8 grouped GEMM (received codes, scales, sources, counts and
flags bit-exact; outputs within the float32 accumulation bound of exact
code sums; small integers exact)."""

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gemm_tol
from tests.gpu_util import dev, host, say, zeros_bytes, max_err

pytestmark = pytest.mark.gpu


def fp8_tol(k, ref_absmax):
    """The GEMM bound the bf16 path meets, 2e-2 sqrt(K/4096) max|ref|.  The
    matrix core does not sum a step's 64 code products exactly (errors near
    2^-14 of the result were measured on N(0,1) data), so the float32
    accumulation bound of exact products does not hold; small-integer codes,
    whose sums are exact in any accumulator, are compared bit for bit."""
    return gemm_tol(k, ref_absmax)


def ovl():
    from communication_overlap_amd import ovl as _o
    return _o


def _quantize_on_gpu(rows_bf16):
    import torch
    o = ovl()
    r, c = rows_bf16.shape
    q = torch.zeros(max(r, 1), max(c, 16), dtype=torch.uint8, device="cuda")
    s = torch.zeros(max(r, 1), dtype=torch.float32, device="cuda")
    o.fp8_quantize_rows(dev(rows_bf16), q, s, r, c)
    return host(q)[:r, :c], host(s)[:r]


@pytest.mark.parametrize("rows,cols,sigma", [(7, 16, 1.0), (33, 272, 1.0), (64, 4096, 0.02), (5, 1024, 300.0)])
def test_quantizer_bit_exact(rows, cols, sigma):
    x = synth.normal_bf16(17, 12, cols, (rows, cols), sigma)
    x[rows // 2] = 0  # a zero row
    if rows > 3:  # a wide dynamic range in one row: subnormal codes
        x[1, ::3] = synth.normal_bf16(17, 13, 0, (1, len(range(0, cols, 3))), 1e-4)[0]
    say(f"[fp8] quantize {rows}x{cols} sigma={sigma}")
    q, s = _quantize_on_gpu(x)
    rq, rs = oracle.quantize_rows(x)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:5]
    if rows > 3 and sigma <= 1.0:
        assert np.any(((rq & 0x78) == 0) & ((rq & 7) != 0)), "no subnormal code exercised"


def _fp8_inputs(cfg, kind="normal"):
    """(x8, x_scale, topk, w8 [E][n][hidden], w_scale [E][n]) for a dispatch config."""
    x, topk, w = synth.dispatch_inputs(cfg, kind if kind == "normal" else "normal")
    E = cfg.experts_per_rank
    if kind == "smallint":
        codes = oracle.e4m3_encode(np.arange(-4, 5, dtype=np.float32))
        rng = np.random.default_rng(cfg.seed)
        x8 = [rng.choice(codes, (cfg.tokens, cfg.hidden)).astype(np.uint8) for _ in range(cfg.ranks)]
        xs = [np.ones(cfg.tokens, np.float32) for _ in range(cfg.ranks)]
        w8 = rng.choice(codes, (E, cfg.n, cfg.hidden)).astype(np.uint8)
        ws = np.ones((E, cfg.n), np.float32)
        return x8, xs, topk, w8, ws
    q = [oracle.quantize_rows(v) for v in x]
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))  # [E][n][hidden]
    wq = [oracle.quantize_rows(wt[e]) for e in range(E)]
    return [a for a, _ in q], [b for _, b in q], topk, np.stack([a for a, _ in wq]), np.stack([b for _, b in wq])


class Fp8Case:
    def __init__(self, cfg, kind="normal"):
        import torch
        o = ovl()
        self.cfg = cfg
        self.x8, self.xs, self.topk, self.w8, self.ws_ = _fp8_inputs(cfg, kind)
        R, cap = cfg.ranks, cfg.cap
        self.desc = o.a2a_desc(R, cfg.rank, cfg.tokens, cfg.hidden, cfg.n, cfg.topk, cfg.num_experts,
                               cfg.experts_per_rank, 8)
        self.fbytes = o.a2a_flags_bytes(self.desc)
        self.d_x8 = [dev(a) for a in self.x8]
        self.d_xs = [dev(a) for a in self.xs]
        self.d_topk = [dev(t) for t in self.topk]
        self.d_w8 = dev(self.w8)
        self.d_ws = dev(self.ws_)
        self.recv_x8 = torch.zeros(R, cap, cfg.hidden, dtype=torch.uint8, device="cuda")
        self.recv_scale = torch.zeros(R, cap, dtype=torch.float32, device="cuda")
        self.recv_src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
        self.recv_count = torch.zeros(R, cfg.experts_per_rank, dtype=torch.int32, device="cuda")
        self.y = torch.zeros(R, cap, cfg.n, dtype=torch.float32, device="cuda")
        self.flags = zeros_bytes(self.fbytes)
        self.ws = zeros_bytes(o.a2a_workspace_bytes(self.desc))
        o.ovl_flags_reset(self.flags, self.fbytes, self.ws, self.ws.numel())

    def run(self, epoch, mode=0):
        o = ovl()
        if mode != o.MODE_GEMM_ONLY and self.recv_x8.numel():
            # E4M3 NaN codes and NaN scales: a row read before its slice lands,
            # or a padding row written, shows.
            self.recv_x8.fill_(0x7F)
            self.recv_scale.fill_(float("nan"))
            self.poisoned = True
        say(f"[fp8] a2a {self.cfg.name} epoch={epoch} mode={mode}")
        o.a2a_dispatch_grouped_gemm_fp8_run(self.desc, self.d_x8, self.d_xs, self.d_topk, self.d_w8, self.d_ws,
                                            self.recv_x8, self.recv_scale, self.recv_src, self.recv_count, self.y,
                                            self.flags, self.ws, epoch, mode=mode)
        return o.ovl_check(self.ws, raise_on_error=False)

    def check_layout(self, epoch):
        c = self.cfg
        rx8, rs8, src, rc = oracle.dispatch_fp8(self.x8, self.xs, self.topk, c.rank, c.experts_per_rank, c.cap)
        assert np.array_equal(host(self.recv_count), rc)
        assert np.array_equal(host(self.recv_src), src)
        got_x, got_s = host(self.recv_x8), host(self.recv_scale)
        for s in range(c.ranks):
            n = int(rc[s].sum())
            assert np.array_equal(got_x[s, :n], rx8[s, :n]), f"codes of slice {s}"
            assert np.array_equal(got_s[s, :n].view(np.uint32), rs8[s, :n].view(np.uint32)), f"scales of slice {s}"
            if getattr(self, "poisoned", False):
                assert (got_x[s, n:] == 0x7F).all() and np.isnan(got_s[s, n:]).all(), f"padding of slice {s}"
            else:
                assert not got_x[s, n:].any() and not got_s[s, n:].any()
        assert np.array_equal(host(self.flags)[: self.fbytes], oracle.expected_flags(c.ranks, 8, epoch))
        return rx8, rs8, rc

    def check_y(self, rx8, rs8, rc):
        ref = oracle.grouped_gemm_fp8(rx8, rs8, rc, self.w8, self.ws_)
        got = host(self.y)
        assert max_err(got, ref) <= fp8_tol(self.cfg.hidden, float(np.abs(ref).max()))
        return got


def _cfg(name, R=2, T=64, H=64, N=128, topk=2, E=4, rank=0, seed=3):
    return synth.DispatchCfg(name, R, T, H, N, topk, R * E, E, 1.1, 1.0, 0.25, seed, rank)


@pytest.mark.parametrize("cfg", [
    _cfg("f8_small"),
    _cfg("f8_ragged", R=3, T=100, H=208, N=136, E=3, rank=1, seed=5),
    _cfg("f8_skewed", R=4, T=300, H=80, N=264, E=2, rank=3, seed=8),
    _cfg("f8_rows_1k", R=3, T=90, H=1024, N=136, E=3, rank=1, seed=6),  # 8 rows per copy slot
    _cfg("f8_rows_2k", R=2, T=77, H=2048, N=128, E=4, rank=0, seed=7),  # 4 rows per copy slot
])
def test_fp8_dispatch_and_gemm_match_oracle(cfg):
    case = Fp8Case(cfg)
    st, det = case.run(1)
    assert st == 0, det
    case.check_y(*case.check_layout(1))


def test_fp8_small_integers_exact_and_modes_agree():
    o = ovl()
    cfg = _cfg("f8_int", R=4, T=200, H=128, N=256, E=2, rank=2)
    case = Fp8Case(cfg, "smallint")
    assert case.run(1)[0] == 0
    rx8, rs8, rc = case.check_layout(1)
    ref = oracle.grouped_gemm_fp8(rx8, rs8, rc, case.w8, case.ws_)
    first = host(case.y).copy()
    assert np.array_equal(first, ref.astype(np.float32))
    case.y.zero_()
    assert case.run(2, o.MODE_COPY_ONLY)[0] == 0
    case.check_layout(2)
    assert case.run(3, o.MODE_GEMM_ONLY)[0] == 0
    assert np.array_equal(host(case.y).view(np.uint32), first.view(np.uint32))


def test_fp8_full_size():
    """The MoE workload at full size with FP8 rows: every token and weight
    row quantized on the device bit-exact against the oracle's encoder, the
    received codes, scales, sources, counts and flags bit-exact, and every
    received row of y within the bound of the oracle's FP8 grouped GEMM;
    rows past each slice's count never written."""
    import torch
    o = ovl()
    cfg = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]
    R, E, cap, H, N = cfg.ranks, cfg.experts_per_rank, cfg.cap, cfg.hidden, cfg.n
    x, topk, w = synth.dispatch_inputs(cfg)
    x8, xs = [], []
    for s in range(R):
        q = torch.zeros(cfg.tokens, H, dtype=torch.uint8, device="cuda")
        sc = torch.zeros(cfg.tokens, dtype=torch.float32, device="cuda")
        say(f"[fp8] quantize tokens of source {s}")
        o.fp8_quantize_rows(dev(x[s]), q, sc, cfg.tokens, H)
        rq, rs = oracle.quantize_rows(x[s])
        assert np.array_equal(host(q), rq) and np.array_equal(host(sc).view(np.uint32), rs.view(np.uint32)), s
        x8.append(q)
        xs.append(sc)
    wt_h = np.ascontiguousarray(np.transpose(w, (0, 2, 1))).reshape(E * N, H)
    w8 = torch.zeros(E * N, H, dtype=torch.uint8, device="cuda")
    wsc = torch.zeros(E * N, dtype=torch.float32, device="cuda")
    o.fp8_quantize_rows(dev(wt_h), w8, wsc, E * N, H)
    rq, rs = oracle.quantize_rows(wt_h)
    assert np.array_equal(host(w8), rq) and np.array_equal(host(wsc).view(np.uint32), rs.view(np.uint32))
    desc = o.a2a_desc(R, cfg.rank, cfg.tokens, H, N, cfg.topk, cfg.num_experts, E, 8)
    fb = o.a2a_flags_bytes(desc)
    recv_x8 = torch.full((R, cap, H), 0x7F, dtype=torch.uint8, device="cuda")
    recv_scale = torch.full((R, cap), float("nan"), dtype=torch.float32, device="cuda")
    recv_src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    recv_count = torch.zeros(R, E, dtype=torch.int32, device="cuda")
    y = torch.full((R, cap, N), float("nan"), dtype=torch.float32, device="cuda")
    flags = zeros_bytes(fb)
    ws = zeros_bytes(o.a2a_workspace_bytes(desc))
    o.ovl_flags_reset(flags, fb, ws, ws.numel())
    say("[fp8] full-size fused run")
    o.a2a_dispatch_grouped_gemm_fp8_run(desc, x8, xs, [dev(t) for t in topk], w8, wsc, recv_x8, recv_scale,
                                        recv_src, recv_count, y, flags, ws, 1)
    st, det = o.ovl_check(ws, raise_on_error=False)
    assert st == 0, det
    x8h = [host(t) for t in x8]
    xsh = [host(t) for t in xs]
    rx8, rs8, src_ref, rc_ref = oracle.dispatch_fp8(x8h, xsh, topk, cfg.rank, E, cap)
    assert np.array_equal(host(recv_count), rc_ref) and np.array_equal(host(recv_src), src_ref)
    assert np.array_equal(host(flags)[:fb], oracle.expected_flags(R, 8, 1))
    got_x, got_s, yh = host(recv_x8), host(recv_scale), host(y)
    ref = oracle.grouped_gemm_fp8(rx8, rs8, rc_ref, host(w8).reshape(E, N, H), host(wsc).reshape(E, N))
    tol = fp8_tol(H, float(np.abs(ref).max()))
    for s in range(R):
        n = int(rc_ref[s].sum())
        assert np.array_equal(got_x[s, :n], rx8[s, :n]) and (got_x[s, n:] == 0x7F).all(), s
        assert np.array_equal(got_s[s, :n].view(np.uint32), rs8[s, :n].view(np.uint32)), s
        assert np.isfinite(yh[s, :n]).all(), f"slice {s}: a row read before it landed"
        assert max_err(yh[s, :n], ref[s, :n]) <= tol, s
        assert np.isnan(yh[s, n:]).all(), f"slice {s}: rows past the count written"
