"""Benchmark of the tile-overlap hot path on one MI355X.

A step is one fused AllGather -> GEMM (producer copy + per-unit flags +
consumer MFMA GEMM, one persistent launch) on the R=8 workload: shards of
1024 x 4096 bf16 N(0,1) per rank (gathered M = 8192), B 4096 x 3584 bf16
N(0, 0.02^2), 256 x 256 tiles, one flag per (256-row panel, 256-column K-tile),
a new seeded random producer order every epoch, epochs increasing without
reset.  Prints one JSON line.

Beside the headline number it measures, each with the 256 MB last-level
cache flushed before every repetition: copy-only and GEMM-only times of the
same launch (for overlap efficiency), the GEMM -> ReduceScatter and skinny
AllGather -> GEMM workloads, and the CPU oracle on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # dense MFMA fp8, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E, published
METRIC = "fused AG-GEMM TFLOP/s (% bf16 MFMA peak) + overlap eff. vs copy+GEMM serial"

# HBM bytes per launch of the fused 8192x3584x4096 kernel, from two rocprofv3
# --pmc passes (FETCH_SIZE x 2.00 + WRITE_SIZE x 1.00, the factors a plain
# 256 MiB copy reads on the same counters), and the hash of the kernel
# sources they were taken on; reported only while the sources are unchanged.
TRAFFIC_BYTES = (213240 * 2.0 + 182931 * 1.0) * 1024
TRAFFIC_SOURCES_SHA = "a89794adead20ac5"
KERNEL_SOURCES = ("communication_overlap_amd/csrc/ag_gemm.hip", "communication_overlap_amd/csrc/gemm_core.h",
                  "communication_overlap_amd/csrc/device.h")


def kernel_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class Flusher:
    """Reads 512 MiB so that no operand is served from the 256 MB cache.

    A read leaves the cache holding clean lines.  A flush that writes leaves
    up to 256 MB of dirty lines, whose write-back then lands inside the next
    timed kernel (measured: a 256 MiB copy ran at 3.5 TB/s after a 512 MiB
    zero fill, 5.1-5.5 TB/s after a 512 MiB read)."""

    def __init__(self):
        import torch
        self.buf = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.sum()


def timed_reps(fn, reps, flush=None, warm=5):
    """Median / p10 / p90 of fn's device time in microseconds (HIP events on
    the current stream around fn only), after `warm` untimed calls."""
    import torch
    for _ in range(warm):
        if flush:
            flush()
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if flush:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    t = np.array(times)
    return {"median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90))}


class AgBench:
    def __init__(self, cfg, tiles_per_flag, unit_producers=1):
        import torch
        import synth
        from communication_overlap_amd import ovl
        self.ovl = ovl
        self.cfg = cfg
        shards, b = synth.ag_inputs(cfg)
        self.plan = ovl.ag_gemm_plan(cfg.ranks, 0, cfg.shard_m, cfg.k, cfg.n, cfg.tile_m, cfg.tile_n,
                                     tiles_per_flag, 8, unit_producers)
        units = self.plan.num_units
        pps = -(-cfg.shard_m // min(cfg.tile_m, cfg.shard_m))  # panels per shard
        batches = units // (cfg.ranks * pps)
        self.d_shards = [dev(s) for s in shards]
        self.d_b = dev(b)
        self.g = torch.zeros(cfg.m, cfg.k, dtype=torch.int16, device="cuda")
        self.c = torch.zeros(cfg.m, cfg.n, dtype=torch.float32, device="cuda")
        self.flags = torch.zeros(self.plan.flags_bytes, dtype=torch.uint8, device="cuda")
        self.ws = torch.zeros(self.plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        ovl.ovl_flags_reset(self.flags, self.plan.flags_bytes, self.ws, self.plan.workspace_bytes)
        n_panels = cfg.ranks * pps
        self.orders = [dev(synth.producer_order(cfg.seed, e, n_panels, batches, cfg.random_order))
                       for e in range(1, 6)]
        self.epoch = 0

    def run(self, mode=0, producers=0):
        self.epoch += 1
        self.ovl.ag_gemm_run(self.plan, self.d_shards, self.d_b, self.g, self.c, self.flags, self.ws,
                             self.epoch, self.orders[(self.epoch - 1) % 5], mode=mode, producers=producers)

    def check(self):
        st, det = self.ovl.ovl_check(self.ws, raise_on_error=False)
        if st != 0:
            raise RuntimeError(f"device error {st} {det}")


def trace_summary(ag, flush):
    """One traced fused launch (cache flushed): when the copy finished, how
    long consumers waited for flags, from the device's 100 MHz clock."""
    import torch
    trace = torch.zeros(ag.plan.trace_bytes // 8, dtype=torch.int64, device="cuda")
    flush()
    ag.epoch += 1
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    ag.ovl.ag_gemm_run(ag.plan, ag.d_shards, ag.d_b, ag.g, ag.c, ag.flags, ag.ws, ag.epoch,
                       ag.orders[(ag.epoch - 1) % 5], trace=trace)
    e1.record()
    e1.synchronize()
    ag.check()
    tr = trace.cpu().numpy()
    units = ag.plan.num_units
    pub, items = tr[:units], tr[units:].reshape(-1, 6)
    t0 = int(items[:, 0].min())
    us = lambda ticks: float(ticks) / 100.0  # noqa: E731  (100 MHz)
    busy = items[:, 1] - items[:, 0]
    return {"event_us": e0.elapsed_time(e1) * 1e3,
            "span_us": us(items[:, 1].max() - t0),
            "last_publish_us": us(pub.max() - t0),
            "items": int(len(items)),
            "consumer_wait_frac": float(items[:, 2].sum() / busy.sum()),
            "mean_wait_per_item_us": us(items[:, 2].mean()),
            "items_that_waited": int((items[:, 2] > 0).sum()),
            "sclk_GHz": float((items[:, 5] - items[:, 4]).sum() / (busy.sum() * 10.0)),
            "note": "times from the first item's start; waits = wave-0 flag polling inside the tiles"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _repeat(fn, seconds):
    """Runs fn whole, repeatedly, until `seconds` of wall time; (runs, s per run)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or runs >= 200:
            return runs, dt / runs


def cpu_baseline(cfg):
    """The oracle on the host cores: the headline workload (gather + float64
    GEMM) repeated whole for about 10 s, and every other workload timed whole
    for about 2 s each (the oracle as it is, untuned)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    shards, b = synth.ag_inputs(cfg)
    runs, per = _repeat(lambda: oracle.ag_gemm(shards, b), 10.0)
    per_config = {cfg.name: {"s_per_run": round(per, 4), "runs": runs,
                             "TFLOPs": round(cfg.flops() / per / 1e12, 4)}}
    for name in ("ag_r2_128x256x256", "ag_r8_skinny_128x7168x8192"):
        c = synth.CONFIGS[name]
        sh, bb = synth.ag_inputs(c)
        n, t = _repeat(lambda: oracle.ag_gemm(sh, bb), 2.0)
        per_config[name] = {"s_per_run": round(t, 5), "runs": n, "TFLOPs": round(c.flops() / t / 1e12, 4)}
    c = synth.CONFIGS["rs_r8_8192x4096x1792"]
    a, bb, parts = synth.rs_inputs(c)
    n, t = _repeat(lambda: oracle.gemm_rs(a, bb, parts, c.rank, c.ranks), 2.0)
    per_config[c.name] = {"s_per_run": round(t, 4), "runs": n, "TFLOPs": round(c.flops() / t / 1e12, 4)}
    c = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]
    x, topk, w = synth.dispatch_inputs(c)

    def moe():
        rx, rs, rc = oracle.dispatch(x, topk, c.rank, c.experts_per_rank, c.cap)
        oracle.grouped_gemm(rx, rc, w)

    n, t = _repeat(moe, 2.0)
    per_config[c.name] = {"s_per_run": round(t, 4), "runs": n, "what": "dispatch layout + copy + float64 grouped GEMM"}
    return {"value": cfg.flops() / per / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{runs} runs of the whole {cfg.m}x{cfg.n}x{cfg.k} workload (gather + float64 GEMM), "
                      f"{runs * per:.1f} s",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "per_config": per_config}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="repetitions of each side measurement")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the side workloads")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the flushed overlap measurements (then every launch of the headline kernel runs "
                         "back to back, as in the timed region: the run to profile for its average duration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the other ranks "
              "are emulated as buffers in the same HBM)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from communication_overlap_amd import ovl

    torch.cuda.set_device(0)
    ovl.lib()
    cfg = synth.CONFIGS["ag_r8_8192x3584x4096"]
    log(f"[bench] inputs {cfg.name}")
    ag = AgBench(cfg, tiles_per_flag=1)
    flush = Flusher()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        ag.run()
    ag.check()

    log(f"[bench] timing {args.steps} fused steps")
    # One HIP event pair on the launch stream brackets the K launches: the
    # average launch is their span over K.  (An event pair around every
    # launch left about 6 us between launches, 11 us under the profiler,
    # where the launches otherwise follow each other with no measurable gap.)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        ag.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ag.check()
    kern_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = cfg.flops() / (wall / args.steps) / 1e12
    achieved = cfg.flops() / (kern_us * 1e-6) / 1e12
    # The shader clock under the same back-to-back load, outside the timed
    # region: 10 more launches, then a traced one right behind them (left out
    # with --no-overlap, so that a profile of that run holds the warmup and
    # the timed launches only).
    b2b_trace = None
    if not args.no_overlap:
        for _ in range(10):
            ag.run()
        b2b_trace = trace_summary(ag, lambda: None)
        ag.check()

    overlap = None
    if not args.no_overlap:
        log("[bench] overlap: fused / copy-only / gemm-only, cache flushed")
        fused = timed_reps(lambda: ag.run(ovl.MODE_FUSED), args.reps, flush)
        copy_only = timed_reps(lambda: ag.run(ovl.MODE_COPY_ONLY), args.reps, flush)
        gemm_only = timed_reps(lambda: ag.run(ovl.MODE_GEMM_ONLY), args.reps, flush)
        ag.check()
        copy_bytes = 2 * cfg.m * cfg.k * 2
        overlap = {
            "fused_us": fused, "copy_only_us": copy_only, "gemm_only_us": gemm_only,
            "fused_over_copy_plus_gemm": fused["median_us"] / (copy_only["median_us"] + gemm_only["median_us"]),
            "fused_over_gemm_only": fused["median_us"] / gemm_only["median_us"],
            "copy_only_GBps": copy_bytes / (copy_only["median_us"] * 1e-6) / 1e9,
            "gemm_only_TFLOPs": cfg.flops() / (gemm_only["median_us"] * 1e-6) / 1e12,
            "fused_flushed_TFLOPs": cfg.flops() / (fused["median_us"] * 1e-6) / 1e12,
            "trace": trace_summary(ag, flush),
        }

    extra = {}
    if not args.no_extra and overlap is not None:
        # Flag batching on the same workload: one flag per 256-column K-batch
        # (the headline setting), per 4 or 16 K-tiles, or per whole panel.
        batching = {"1": round(fused["median_us"], 1)}
        for tpf in (4, 16, 0):
            log(f"[bench] flag batching: tiles_per_flag={tpf}")
            agb = AgBench(cfg, tiles_per_flag=tpf)
            agb.run()
            batching[str(tpf)] = round(timed_reps(lambda: agb.run(ovl.MODE_FUSED), args.reps, flush)["median_us"], 1)
            agb.check()
            del agb
        # Split-unit arrivals (signal ADD): each 256 x 256 flag unit moved by W
        # producer workgroups that add to its counter; the last publishes.
        split_units = {"1": round(fused["median_us"], 1)}
        for W in (2, 4):
            log(f"[bench] unit producers: {W}")
            agw = AgBench(cfg, tiles_per_flag=1, unit_producers=W)
            agw.run()
            split_units[str(W)] = round(timed_reps(lambda: agw.run(ovl.MODE_FUSED), args.reps, flush)["median_us"], 1)
            agw.check()
            del agw
        extra = side_workloads(args.reps, flush)
        extra["ag_flag_batching_fused_us"] = {"by_tiles_per_flag": batching,
                                              "note": "0 = one flag per 256-row panel (all of K)"}
        extra["ag_unit_producers_fused_us"] = {
            "by_producers_per_unit": split_units,
            "note": "one flag per 256x256 unit; W > 1: W workgroups copy a unit's rows, each adds an arrival, "
                    "the arrival completing a multiple of W sets the flag"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "AG-GEMM R=8 emulated ranks, A shard 1024x4096 bf16 N(0,1) per rank "
                               "(M=8192), B 4096x3584 bf16 N(0,0.02), tile 256x256, seeded random producer "
                               "order, epochs increasing on one flag buffer",
                   "m": cfg.m, "n": cfg.n, "k": cfg.k, "ranks": cfg.ranks, "tile": [cfg.tile_m, cfg.tile_n],
                   "tiles_per_flag": 1},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (TRAFFIC_BYTES if kernel_sources_sha() == TRAFFIC_SOURCES_SHA else None),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-scaled)",
                     "algorithmic_flops_per_launch": cfg.flops(),
                     "kernel": "ag_gemm_kernel<256, 256, 2, 0> (fused)", "avg_launch_us": round(kern_us, 2)},
        "overlap": overlap,
        # the same back-to-back launches against the bf16 peak scaled to the shader clock they
        # ran at (sampled in a traced launch right behind 10 back-to-back ones; the published
        # peak assumes 2.4 GHz), and the flushed launch at its own clock
        "roofline_at_measured_clock": ({
            "sclk_GHz": round(b2b_trace["sclk_GHz"], 3),
            "peak": round(PEAK_BF16_TFLOPS * b2b_trace["sclk_GHz"] / 2.4, 1),
            "frac": round(achieved / (PEAK_BF16_TFLOPS * b2b_trace["sclk_GHz"] / 2.4), 4),
            "flushed_sclk_GHz": round(overlap["trace"]["sclk_GHz"], 3),
            "flushed_frac": round(cfg.flops() / (overlap["fused_us"]["median_us"] * 1e-6) / 1e12
                                  / (PEAK_BF16_TFLOPS * overlap["trace"]["sclk_GHz"] / 2.4), 4)}
            if overlap else None),
        "side": extra,
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


def side_workloads(reps, flush):
    import torch
    import synth
    from communication_overlap_amd import ovl
    res = {}

    # The small R=2 AllGather -> GEMM (128x256x256, 32x32 flag tiles): a
    # latency-bound correctness workload; its time is reported, with no target.
    cfg = synth.CONFIGS["ag_r2_128x256x256"]
    log(f"[bench] side {cfg.name}")
    sm = AgBench(cfg, tiles_per_flag=1)
    sm.run()
    t = timed_reps(lambda: sm.run(), reps, flush)
    gemm = timed_reps(lambda: sm.run(ovl.MODE_GEMM_ONLY), reps, flush)
    sm.check()
    res[cfg.name] = {"fused_us": t, "gemm_only_us": gemm, "flag_units": sm.plan.num_units,
                     "TFLOPs": cfg.flops() / (t["median_us"] * 1e-6) / 1e12}
    del sm

    # Skinny decode-like AllGather -> GEMM (HBM bound: B is 117 MB).
    cfg = synth.CONFIGS["ag_r8_skinny_128x7168x8192"]
    log(f"[bench] side {cfg.name}")
    sk = AgBench(cfg, tiles_per_flag=4)
    sk.run()
    t = timed_reps(lambda: sk.run(), reps, flush)
    gemm = timed_reps(lambda: sk.run(ovl.MODE_GEMM_ONLY), reps, flush)
    copy = timed_reps(lambda: sk.run(ovl.MODE_COPY_ONLY), reps, flush)
    sk.check()
    bytes_min = cfg.k * cfg.n * 2 + 2 * cfg.m * cfg.k * 2 + cfg.m * cfg.n * 4
    res[cfg.name] = {"fused_us": t, "gemm_only_us": gemm, "copy_only_us": copy,
                     "GBps": bytes_min / (t["median_us"] * 1e-6) / 1e9,
                     "pct_of_hbm_peak": 100 * bytes_min / (t["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "TFLOPs": cfg.flops() / (t["median_us"] * 1e-6) / 1e12}
    del sk

    # GEMM -> ReduceScatter.
    cfg = synth.CONFIGS["rs_r8_8192x4096x1792"]
    log(f"[bench] side {cfg.name}")
    a, b, parts = synth.rs_inputs(cfg)
    desc = ovl.gemm_rs_desc(cfg.ranks, 0, cfg.m, cfg.n, cfg.k)
    fb = ovl.gemm_rs_flags_bytes(desc)
    bm = cfg.block_m
    d_a, d_b = dev(a), dev(b)
    peer_out = [None] + [torch.zeros(bm, cfg.n, device="cuda") for _ in range(1, cfg.ranks)]
    peer_in = [None] + [dev(parts[p]) for p in range(1, cfg.ranks)]
    out = torch.zeros(bm, cfg.n, device="cuda")
    out_flags = torch.zeros(fb, dtype=torch.uint8, device="cuda")
    in_flags = torch.zeros(fb, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(ovl.gemm_rs_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    ovl.ovl_flags_reset(out_flags, fb, ws, ws.numel())
    ep = [0]

    def rs_ready():
        """The peers' partials are pre-resident: their flags are set to the
        coming run's epoch (outside the timed region, after the flush)."""
        flush()
        in_flags.view(torch.int64).fill_(ep[0] + 1)

    def rs(mode=0):
        ep[0] += 1
        ovl.gemm_rs_run(desc, d_a, d_b, peer_out, peer_in, out, out_flags, in_flags, ws, ep[0], mode=mode)

    rs_ready()
    rs()
    t = timed_reps(rs, reps, rs_ready)
    g = timed_reps(lambda: rs(ovl.MODE_GEMM_ONLY), reps, rs_ready)
    ovl.ovl_check(ws)
    res[cfg.name] = {"fused_us": t, "gemm_only_us": g,
                     "TFLOPs": cfg.flops() / (t["median_us"] * 1e-6) / 1e12,
                     "pct_of_bf16_peak": 100 * cfg.flops() / (t["median_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}

    # All-to-all dispatch -> grouped expert GEMM (rank 0 receives the most rows).
    cfg = synth.CONFIGS["a2a_r8_t4096_h4096_e64"]
    log(f"[bench] side {cfg.name}")
    x, topk, w = synth.dispatch_inputs(cfg)
    R, cap, E = cfg.ranks, cfg.cap, cfg.experts_per_rank
    desc = ovl.a2a_desc(R, cfg.rank, cfg.tokens, cfg.hidden, cfg.n, cfg.topk, cfg.num_experts, E, 8)
    fb = ovl.a2a_flags_bytes(desc)
    d_x = [dev(v) for v in x]
    d_topk = [dev(t) for t in topk]
    d_w = dev(w)
    recv_x = torch.zeros(R, cap, cfg.hidden, dtype=torch.int16, device="cuda")
    recv_src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    recv_count = torch.zeros(R, E, dtype=torch.int32, device="cuda")
    y = torch.zeros(R, cap, cfg.n, dtype=torch.float32, device="cuda")
    flags = torch.zeros(fb, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(ovl.a2a_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    ovl.ovl_flags_reset(flags, fb, ws, ws.numel())
    ep = [0]

    def a2a(mode=0):
        ep[0] += 1
        ovl.a2a_dispatch_grouped_gemm_run(desc, d_x, d_topk, d_w, recv_x, recv_src, recv_count, y, flags, ws,
                                          ep[0], mode=mode)

    a2a()
    t = timed_reps(a2a, reps, flush)
    disp = timed_reps(lambda: a2a(ovl.MODE_COPY_ONLY), reps, flush)
    g = timed_reps(lambda: a2a(ovl.MODE_GEMM_ONLY), reps, flush)
    ovl.ovl_check(ws)
    rows = int(recv_count.sum().item())
    lo = cfg.rank * E
    uniq = sum(int(((tk >= lo) & (tk < lo + E)).any(axis=1).sum()) for tk in topk)
    d_bytes = uniq * cfg.hidden * 2 + rows * (cfg.hidden * 2 + 4)  # token reads; row + source writes
    flops = 2.0 * rows * cfg.hidden * cfg.n
    res[cfg.name] = {"fused_us": t, "dispatch_only_us": disp, "gemm_only_us": g,
                     "routed_rows": rows, "unique_tokens": uniq,
                     "dispatch_bytes": d_bytes, "grouped_gemm_flops": flops,
                     "dispatch_GBps": d_bytes / (disp["median_us"] * 1e-6) / 1e9,
                     "dispatch_pct_of_hbm_peak": 100 * d_bytes / (disp["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "gemm_only_TFLOPs": flops / (g["median_us"] * 1e-6) / 1e12,
                     "fused_TFLOPs": flops / (t["median_us"] * 1e-6) / 1e12,
                     "fused_pct_of_bf16_peak": 100 * flops / (t["median_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                     "fused_over_dispatch_plus_gemm": t["median_us"] / (disp["median_us"] + g["median_us"]),
                     "fused_over_gemm_only": t["median_us"] / g["median_us"]}
    # The same dispatch in FP8: tokens quantized per row at each source (E4M3
    # codes + a float32 scale), weights as transposed E4M3 rows with a scale
    # per output column; the quantization is done once, outside the timing.
    log("[bench] side a2a fp8")
    x8, xs8 = [], []
    for s in range(R):
        q8 = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.uint8, device="cuda")
        sc8 = torch.empty(cfg.tokens, dtype=torch.float32, device="cuda")
        ovl.fp8_quantize_rows(d_x[s], q8, sc8, cfg.tokens, cfg.hidden)
        x8.append(q8)
        xs8.append(sc8)
    wt = d_w.view(E, cfg.hidden, cfg.n).transpose(1, 2).contiguous().view(E * cfg.n, cfg.hidden)
    w8 = torch.empty(E * cfg.n, cfg.hidden, dtype=torch.uint8, device="cuda")
    ws8 = torch.empty(E * cfg.n, dtype=torch.float32, device="cuda")
    ovl.fp8_quantize_rows(wt, w8, ws8, E * cfg.n, cfg.hidden)
    del wt
    recv_x8 = torch.zeros(R, cap, cfg.hidden, dtype=torch.uint8, device="cuda")
    recv_s8 = torch.zeros(R, cap, dtype=torch.float32, device="cuda")
    y8 = torch.zeros(R, cap, cfg.n, dtype=torch.float32, device="cuda")

    def a2a8(mode=0):
        ep[0] += 1
        ovl.a2a_dispatch_grouped_gemm_fp8_run(desc, x8, xs8, d_topk, w8, ws8, recv_x8, recv_s8, recv_src,
                                              recv_count, y8, flags, ws, ep[0], mode=mode)

    a2a8()
    t8 = timed_reps(a2a8, reps, flush)
    disp8 = timed_reps(lambda: a2a8(ovl.MODE_COPY_ONLY), reps, flush)
    g8 = timed_reps(lambda: a2a8(ovl.MODE_GEMM_ONLY), reps, flush)
    ovl.ovl_check(ws)
    d8_bytes = uniq * (cfg.hidden + 4) + rows * (cfg.hidden + 4 + 4)  # codes + scale read; row, scale, source written
    res["a2a_fp8_r8_t4096_h4096_e64"] = {
        "fused_us": t8, "dispatch_only_us": disp8, "gemm_only_us": g8, "dispatch_bytes": d8_bytes,
        "dispatch_GBps": d8_bytes / (disp8["median_us"] * 1e-6) / 1e9,
        "gemm_only_TFLOPs": flops / (g8["median_us"] * 1e-6) / 1e12,
        "gemm_only_pct_of_fp8_peak": 100 * flops / (g8["median_us"] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS,
        "fused_TFLOPs": flops / (t8["median_us"] * 1e-6) / 1e12,
        "fused_over_dispatch_plus_gemm": t8["median_us"] / (disp8["median_us"] + g8["median_us"]),
        "fused_over_gemm_only": t8["median_us"] / g8["median_us"]}
    del x8, recv_x8, y8, w8

    # MoE combine at the same rank: reverse puts of y to the 7 peers, then the
    # gate-weighted sum of this rank's tokens (peers' returned rows pre-resident).
    log("[bench] side a2a combine")
    gates, ret_in = synth.combine_inputs(cfg)
    d_gates = dev(gates)
    d_ret_in = [None if q == cfg.rank else dev(ret_in[q]) for q in range(R)]
    del ret_in
    ret_out = [None if q == cfg.rank else torch.zeros(cap, cfg.n, dtype=torch.float32, device="cuda")
               for q in range(R)]
    out = torch.zeros(cfg.tokens, cfg.n, dtype=torch.float32, device="cuda")
    cfb = ovl.a2a_combine_flags_bytes(desc)
    c_out_flags = torch.zeros(cfb, dtype=torch.uint8, device="cuda")
    c_in_flags = torch.zeros(cfb, dtype=torch.uint8, device="cuda")
    c_ws = torch.zeros(ovl.a2a_combine_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    ovl.ovl_flags_reset(c_out_flags, cfb, c_ws, c_ws.numel())
    cep = [0]

    def comb_ready():
        """The peers' returned rows are pre-resident: their flags hold the
        coming run's epoch (outside the timed region, after the flush)."""
        flush()
        c_in_flags.view(torch.int64).fill_(cep[0] + 1)

    def comb(mode=0):
        cep[0] += 1
        ovl.a2a_combine_run(desc, y, recv_count, ret_out, d_ret_in, d_topk[cfg.rank], d_gates, out, c_out_flags,
                            c_in_flags, c_ws, cep[0], mode=mode)

    comb_ready()
    comb()
    t = timed_reps(comb, reps, comb_ready)
    put = timed_reps(lambda: comb(ovl.MODE_COPY_ONLY), reps, comb_ready)
    sm = timed_reps(lambda: comb(ovl.MODE_GEMM_ONLY), reps, comb_ready)
    ovl.ovl_check(c_ws)
    rc = recv_count.cpu().numpy()
    rows_back = int(sum(rc[s].sum() for s in range(R) if s != cfg.rank))
    put_bytes = 2 * rows_back * cfg.n * 4
    sum_bytes = cfg.tokens * (cfg.topk + 1) * cfg.n * 4
    res["a2a_combine_r8_t4096_n1408"] = {
        "fused_us": t, "reverse_put_only_us": put, "sum_only_us": sm, "rows_sent_back": rows_back,
        "bytes": put_bytes + sum_bytes,
        "GBps": (put_bytes + sum_bytes) / (t["median_us"] * 1e-6) / 1e9,
        "pct_of_hbm_peak": 100 * (put_bytes + sum_bytes) / (t["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        "fused_over_put_plus_sum": t["median_us"] / (put["median_us"] + sm["median_us"])}
    del recv_x, y, ret_out, d_ret_in, out

    # Ring all-reduce: 8 emulated ranks x 8M fp32 (32 MiB each), 16K-element
    # tiles, every rank's steps in one launch (FUSED) or one launch per ring
    # step (BARRIER: no tile-level overlap between steps).
    cfg = synth.CONFIGS["ring_r8_n8m"]
    log(f"[bench] side {cfg.name}")
    R = cfg.ranks
    r_in = [dev(v) for v in synth.ring_inputs(cfg)]
    r_out = [torch.zeros(cfg.n, dtype=torch.float32, device="cuda") for _ in range(R)]
    rdesc = ovl.ring_desc(R, cfg.n, cfg.tile)
    rfb = ovl.ring_allreduce_flags_bytes(rdesc)
    r_flags = torch.zeros(rfb, dtype=torch.uint8, device="cuda")
    r_ws = torch.zeros(ovl.ring_allreduce_workspace_bytes(rdesc), dtype=torch.uint8, device="cuda")
    ovl.ovl_flags_reset(r_flags, rfb, r_ws, r_ws.numel())
    rep_ = [0]

    def ring(mode=0):
        rep_[0] += 1
        ovl.ring_allreduce_run(rdesc, r_in, r_out, r_flags, r_ws, rep_[0], mode=mode)

    ring()
    t = timed_reps(ring, reps, flush)
    b = timed_reps(lambda: ring(ovl.MODE_BARRIER), reps, flush)
    ovl.ovl_check(r_ws)
    # per rank and tile position: send (2 tile-bytes), R-2 add-and-send (3),
    # complete-and-send (4), R-2 forwards (2): (5R - 4) x n x 4 bytes in all
    r_bytes = (5 * R - 4) * cfg.n * 4
    res[cfg.name] = {"fused_us": t, "barrier_us": b, "bytes": r_bytes,
                     "GBps": r_bytes / (t["median_us"] * 1e-6) / 1e9,
                     "pct_of_hbm_peak": 100 * r_bytes / (t["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "fused_over_barrier": t["median_us"] / b["median_us"]}
    del r_in, r_out

    # Plain copy, for the HBM reference point.
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = timed_reps(lambda: ovl.ovl_copy(dst, src, src.numel()), reps, flush)
    res["plain_copy_256MiB"] = {"us": t, "GBps": 2 * src.numel() / (t["median_us"] * 1e-6) / 1e9}
    return res


if __name__ == "__main__":
    main()
