#!/usr/bin/env python3
"""Benchmark of the NVFP4 routed-expert MoE layer on one MI355X.

A step is one moe_layer_forward call over one synthetic batch: grouping, gather +
quantize, w13 grouped GEMM, SwiGLU + re-quantize, w2 grouped GEMM, scatter-add — every
step of the path, inputs and packed weights already resident in HBM.  The step is timed
both as eager launches and as one HIP-graph replay of the same launches (the pages'
graph-launched layer); the faster of the two medians is the reported value (both are in
the line), and the run checks that a replay gives the eager output bit for bit.  Each timed block follows an untimed warm-up of
at least --warmup steps and at least --settle-ms of continuous work (default 500 ms;
measured on MI355X, the layer runs up to 10% slower during the first few hundred ms of
work after the GPU was idle).

Metric (the pages' own byte model, table "Bytes decide it before the kernel runs" of the
[MF]): weight-stream GB/s = active experts x 14,155,776 B / layer time.

Prints ONE JSON line.  The workloads in --also (default: ragged2303 and the skewed zipf512
decode batch) are timed the same way in the same run.  Also times the dominant kernel (the
w13 grouped GEMM) with HIP
events on its own stream over a loop of launches on the layer's real inputs, and the CPU
oracle on a bounded sample of the same workload (cpu_baseline).

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1"; [MF] the page "Fusing the MoE layer's two grouped GEMMs is
worth 4%, and a CUDA graph already collects it" (gabewillen.github.io/rocket).
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer ms + weight-stream HBM GB/s (% of peak), 288 experts, 570/2303 rows"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
W13_BYTES_PER_EXPERT = 2 * 2048 * 4096 * 9 // 16   # 9,437,184
W2_BYTES_PER_EXPERT = 2048 * 4096 * 9 // 16      # 4,718,592
LAYER_BYTES_PER_EXPERT = 3 * 2048 * 4096 * 9 // 16  # 14,155,776


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle-ms", type=float, default=500.0,
                   help="the untimed warm-up before each timed block runs at least --warmup "
                        "steps and at least this long (the GPU reaches steady clocks only "
                        "after a few hundred ms of continuous work)")
    p.add_argument("--workload", default="ragged570",
                   choices=["ragged570", "ragged2303", "zipf512", "decode1"])
    p.add_argument("--no-decode-sweep", action="store_true",
                   help="skip the decode-batch M sweep (M = 1 .. 32 token streams, top-8)")
    p.add_argument("--no-w4a16", action="store_true",
                   help="skip the W4A16 leg (bf16 activations against the same weights)")
    p.add_argument("--flush-mb", type=int, default=512,
                   help="device copy run before every timed decode-sweep call so that no "
                        "expert weight is served from the 256 MB MALL or the L2s")
    p.add_argument("--also", default="ragged2303,zipf512",
                   help="comma-separated workloads timed in the same run after the main one "
                        "('' for none)")
    p.add_argument("--flags", type=int, default=None, help="GEMM path (0 auto, 1 GEMV, 2 MFMA)")
    p.add_argument("--gemv-max-rows", type=int, default=None)
    p.add_argument("--kernel-iters", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-read-probe", action="store_true",
                   help="skip the measured read roofline (moe_hbm_read_probe over 4.0 GiB)")
    p.add_argument("--no-graph", action="store_true",
                   help="time eager launches only (default: also a HIP-graph replay of the "
                        "layer, which is the reported value)")
    p.add_argument("--cpu-experts", type=int, default=144,
                   help="experts in the oracle's bounded sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy 3 times (reference for the HBM "
                        "byte counters) and exit")
    return p.parse_args()


def calibrate_copy():
    """A plain device-to-device copy of known size, so that profiler byte counters
    (FETCH_SIZE, WRITE_SIZE) can be scaled: each copy reads and writes 1 GiB."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": 3}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_layer_ragged570_hbm_bytes.txt")


def measured_traffic(workload):
    """HBM bytes per w13 grouped-GEMM launch from the committed profiler-counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size), or None when
    the summary is for another workload or the GEMM sources changed since it was taken."""
    from nvfp4_block_scaled_gather_amd import build as _b
    try:
        fields = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines()
                      if ":" in l and not l.startswith((" ", "#", "|")))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("workload") != workload:
        return None
    if fields.get("kernel_sources_sha256") != _b.kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def warm(step, warmup, settle_ms):
    """Untimed warm-up: at least `warmup` steps and at least `settle_ms` of continuous work."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_layer(dl, steps, warmup, settle_ms=0.0):
    import torch
    warm(dl.forward, warmup, settle_ms)
    per = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    for _ in range(steps):
        start.record()
        dl.forward()
        stop.record()
        stop.synchronize()
        per.append(start.elapsed_time(stop))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return float(np.median(per)), float(np.min(per)), float(np.max(per)), wall


def time_graph(dl, steps, warmup, settle_ms=0.0):
    """The same layer step as time_layer, launched as one HIP-graph replay (the pages'
    graph-launched variant): every kernel of the layer runs on every replay."""
    import torch
    graph = dl.capture_graph()
    warm(graph.replay, warmup, settle_ms)
    per = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    for _ in range(steps):
        start.record()
        graph.replay()
        stop.record()
        stop.synchronize()
        per.append(start.elapsed_time(stop))
    return float(np.median(per)), float(np.min(per)), float(np.max(per)), graph


def time_gemms(dl, iters, settle_ms=0.0):
    """Average duration of one w13 and one w2 grouped-GEMM launch (grouped_gemm_nvfp4) on
    the layer's own data: the quantized activation rows for w13, and the quantized SwiGLU
    output of those rows for w2 (the plain fp32 output, without the layer's scatter-ready
    epilogue).  HIP events on the launch stream, back-to-back launches."""
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    wl = dl.wl
    R, E, H, I, T, S = wl.R, wl.E, wl.H, wl.I, wl.T, wl.S
    dev = torch.device("cuda")
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    xg, off = e((R, H), torch.int16), e((E + 1,), torch.int32)
    rs, rd, rw = e((R,), torch.int32), e((R,), torch.int32), e((R,), torch.float32)
    to, tr, err = e((T + 1,), torch.int32), e((R,), torch.int32), e((1,), torch.int32)
    stream = torch.cuda.Stream()
    flags, gmax = dl.desc.flags, dl.desc.gemv_max_rows

    def timed(launch):
        # untimed: at least 10 launches and settle_ms of them, to steady clocks
        warm(launch, 10, settle_ms)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(iters):
            launch()
        stop.record(stream)
        stop.synchronize()
        return start.elapsed_time(stop) / iters

    with torch.cuda.stream(stream):
        B.moe_gather_rows(dl.x, S, H, dl.a_expert, dl.a_src, dl.a_dst, dl.a_w, R, E, T, xg, off,
                          rs, rd, rw, to, tr, err)
        xq, xs, xgs = e((R, H // 2), torch.uint8), e((R, H // 16), torch.uint8), e((R,), torch.float32)
        B.nvfp4_quantize_rows(xg, R, H, xq, xs, xgs)
        acc = e((R, 2 * I), torch.float32)
        w13_ms = timed(lambda: B.grouped_gemm_nvfp4(xq, xs, off, E, R, dl.w13, 2 * I, H, acc,
                                                    flags, gmax))
        h = e((R, I), torch.int16)
        B.swiglu_grouped(acc, R, I, off, E, dl.g_gate, dl.g_up, xgs, h)
        hq, hs, hgs = e((R, I // 2), torch.uint8), e((R, I // 16), torch.uint8), e((R,), torch.float32)
        B.nvfp4_quantize_rows(h, R, I, hq, hs, hgs)
        y = e((R, H), torch.float32)
        w2_ms = timed(lambda: B.grouped_gemm_nvfp4(hq, hs, off, E, R, dl.w2, H, I, y, flags, gmax))
    torch.cuda.synchronize()
    return w13_ms, w2_ms


# Read-probe buffer: 14,564 GEMM work items of 288 KiB (8 tiles of 36 KiB), 4.0 GiB
READ_PROBE_BYTES = 14564 * 294912
READ_PROBE_VARIANTS = {0: "contiguous per wave, 8 KiB in flight, 32 waves/CU",
                       1: "contiguous per wave, 16 KiB in flight, 32 waves/CU",
                       2: "contiguous per wave, 16 KiB in flight, 16 waves/CU",
                       3: "the w13 GEMM's items: 4 waves x 2 tiles of 36 KiB, 4 KiB of each "
                          "in flight",
                       4: "contiguous per wave, 32 KiB in flight, 32 waves/CU"}


def read_roofline(iters, settle_ms=0.0):
    """The measured HBM read roofline: moe_hbm_read_probe over a 4.0 GiB buffer of random
    bytes, each load pattern timed with HIP events on its launch stream over `iters`
    back-to-back launches after a warm-up; GB/s = bytes read / average launch time."""
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    buf = torch.randint(0, 256, (READ_PROBE_BYTES,), dtype=torch.uint8, device="cuda", generator=g)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    res = {}
    with torch.cuda.stream(stream):
        for v in range(B.moe_hbm_read_probe_variants()):
            launch = lambda: B.moe_hbm_read_probe(buf, READ_PROBE_BYTES, v, 0x9E3779B9, sink)
            warm(launch, 5, settle_ms)
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(iters):
                launch()
            stop.record(stream)
            stop.synchronize()
            ms = start.elapsed_time(stop) / iters
            res[v] = {"pattern": READ_PROBE_VARIANTS.get(v, str(v)), "ms": ms,
                      "GBps": READ_PROBE_BYTES / (ms * 1e-3) / 1e9}
            log(json.dumps({"read_probe": v, **res[v]}))
    del buf
    torch.cuda.synchronize()
    best = max(res, key=lambda v: res[v]["GBps"])
    return {"GBps": res[best]["GBps"], "best_variant": best, "bytes": READ_PROBE_BYTES,
            "variants": res}


def cpu_baseline(wl, n_experts):
    """The CPU oracle on a bounded sample: the rows of the first n_experts active experts
    (their whole layer: quantize, both GEMMs, SwiGLU, scatter), reported in the metric's
    unit (weight-stream GB/s over the sample) plus the layer time it extrapolates to."""
    from oracle import moe as omoe
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    active = wl.active_experts()
    keep = set(active[:n_experts])
    sel = np.array([j for j in range(wl.R) if int(wl.a_expert[j]) in keep], dtype=np.int64)
    # input generation (the seeded weights) stays outside the timed region
    w13 = {e: wl.w13(e) for e in keep}
    w2 = {e: wl.w2(e) for e in keep}
    t0 = time.perf_counter()
    omoe.layer_forward(wl.x, wl.a_expert[sel], wl.a_src[sel], wl.a_dst[sel], wl.a_w[sel], wl.T,
                       w13.__getitem__, w2.__getitem__, wl.g_gate, wl.g_up, wl.g_down,
                       wl.E, wl.H, wl.I)
    dt = time.perf_counter() - t0
    nbytes = len(keep) * LAYER_BYTES_PER_EXPERT
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": "%s: rows of the first %d of %d active experts (%d of %d expert-rows), whole "
                  "layer in the numpy float64 oracle, weight generation excluded; %.2f s, extrapolates to %.0f ms per layer; "
                  "host %d logical CPUs (%s); numpy dequantization is single-threaded, BLAS "
                  "matrix-vector products use %d threads"
                  % (wl.name, len(keep), len(active), len(sel), wl.R, dt,
                     dt * 1e3 * len(active) / len(keep), os.cpu_count() or 0, cpu_model,
                     blas_threads),
    }


def run_workload(name, args, weights=None):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload(name)
    kw = {}
    if args.flags is not None:
        kw["flags"] = args.flags
    if args.gemv_max_rows is not None:
        kw["gemv_max_rows"] = args.gemv_max_rows
    if weights is None:
        log("packing %d experts (w13 + w2, %.3f GB)" % (wl.E, wl.E * LAYER_BYTES_PER_EXPERT / 1e9))
        t0 = time.perf_counter()
        weights = (L.pack_expert_weights(wl.w13, wl.E, 2 * wl.I, wl.H),
                   L.pack_expert_weights(wl.w2, wl.E, wl.H, wl.I))
        log("packed in %.1f s" % (time.perf_counter() - t0))
    dl = L.DeviceLayer(wl, weights=weights, **kw)
    e_med, e_lo, e_hi, wall = time_layer(dl, args.steps, args.warmup, args.settle_ms)
    err = dl.device_error()
    if err:
        raise RuntimeError("device error word %d" % err)
    eager_out = dl.forward().clone()
    torch.cuda.synchronize()
    launch = "eager"
    med, lo, hi = e_med, e_lo, e_hi
    g_med = g_lo = g_hi = None
    if not args.no_graph:
        g_med, g_lo, g_hi, graph = time_graph(dl, args.steps, args.warmup, args.settle_ms)
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(dl.out, eager_out):  # a replay must give the eager bits
            raise RuntimeError("graph replay output differs from the eager layer output")
        if g_med <= e_med:  # the faster launch mode is the reported one
            med, lo, hi = g_med, g_lo, g_hi
            launch = "hip-graph replay"
    n_act = len(wl.active_experts())
    wbytes = n_act * LAYER_BYTES_PER_EXPERT
    w13_ms, w2_ms = time_gemms(dl, args.kernel_iters, args.settle_ms)
    res = {
        "workload": name, "expert_rows": wl.R, "tokens": wl.T, "active_experts": n_act,
        "launch": launch,
        "layer_ms_median": med, "layer_ms_min": lo, "layer_ms_max": hi,
        "layer_ms_eager_median": e_med, "layer_ms_eager_min": e_lo, "layer_ms_eager_max": e_hi,
        "layer_ms_eager_wall": wall,
        "layer_ms_graph_median": g_med, "layer_ms_graph_min": g_lo, "layer_ms_graph_max": g_hi,
        "weight_bytes": wbytes, "weight_GBps": wbytes / (med * 1e-3) / 1e9,
        "frac_of_hbm_peak": wbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "frac_of_hbm_peak_eager": wbytes / (e_med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "w13_gemm_ms": w13_ms,
        "w13_GBps": n_act * W13_BYTES_PER_EXPERT / (w13_ms * 1e-3) / 1e9,
        "w2_gemm_ms": w2_ms,
        "w2_GBps": n_act * W2_BYTES_PER_EXPERT / (w2_ms * 1e-3) / 1e9,
        "gemm_path": {"flags": dl.desc.flags, "gemv_max_rows": dl.desc.gemv_max_rows},
    }
    log(json.dumps(res))
    return wl, dl, res, weights


def decode_sweep(args, weights):
    """The decode-batch M sweep ([GG] "Numbers", extended to M = 16 and 32): M token streams
    with top-8 routing each, one layer call per step, on the full resident expert set.
    Honest cache: before every timed call an untimed copy of --flush-mb MB (read and write)
    replaces the MALL and L2 contents, so the active experts' weights come from HBM (their
    113 MB at M=1 would otherwise fit in the 256 MB MALL).  Each call is a HIP-graph replay
    (checked equal to the eager output) and, separately, eager calls, timed with HIP events;
    the faster median is reported.  Bytes per token are the weight bytes streamed per step
    over M."""
    import torch
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    nbytes = args.flush_mb << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out = []
    for M in W.DECODE_SWEEP:
        wl = W.make_workload("decode%d" % M)
        dl = L.DeviceLayer(wl, weights=weights)
        eager = dl.forward().clone()
        graph = dl.capture_graph()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(dl.out, eager):
            raise RuntimeError("decode%d: graph replay differs from the eager output" % M)

        def timed(run):
            def step():
                dst.copy_(src)
                run()

            warm(step, args.warmup, args.settle_ms)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                dst.copy_(src)
                a.record()
                run()
                b.record()
            torch.cuda.synchronize()
            return sorted(a.elapsed_time(b) for a, b in ev)

        tg = timed(graph.replay)
        te = timed(dl.forward)
        g_med, e_med = float(np.median(tg)), float(np.median(te))
        med, t, launch = (g_med, tg, "hip-graph replay") if g_med <= e_med else (e_med, te, "eager")
        n_act = len(wl.active_experts())
        wbytes = n_act * LAYER_BYTES_PER_EXPERT
        out.append({"M": M, "expert_rows": wl.R, "active_experts": n_act,
                    "layer_us": med * 1e3, "layer_us_min": t[0] * 1e3, "launch": launch,
                    "layer_us_graph": g_med * 1e3, "layer_us_eager": e_med * 1e3,
                    "weight_bytes": wbytes, "weight_GBps": wbytes / (med * 1e-3) / 1e9,
                    "frac_of_hbm_peak": wbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "weight_bytes_per_token": wbytes / M, "tokens_per_s": M / (med * 1e-3)})
        log(json.dumps(out[-1]))
        del graph, dl
    return {"launch": "the faster of hip-graph replay and eager launches (both medians are "
                      "given), %d MB cache flush before each call" % args.flush_mb,
            "points": out}


def w4a16_leg(args, weights):
    """The W4A16 mode (moe_layer_forward_w4a16: bf16 activations against the same resident
    NVFP4 weights, the pages' GEMV arithmetic) on ragged570 and ragged2303, timed like the
    main leg (eager calls and graph replays after the settle, the faster reported), and on
    decode M = 1, 8, 32 like the M sweep (cache flush before each call; the faster of graph
    replay and eager launches).  Also the largest difference between the W4A16 and
    W4A4 layer outputs on ragged570, relative to the W4A16 row RMS (informational: two
    different arithmetics, [GG] "Numbers")."""
    import torch
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    res = {}
    for name in ("ragged570", "ragged2303"):
        wl = W.make_workload(name)
        dl = L.DeviceLayer(wl, weights=weights, arithmetic="w4a16")
        out16 = dl.forward().clone()
        e_med, e_lo, e_hi, _ = time_layer(dl, args.steps, args.warmup, args.settle_ms)
        g_med, g_lo, g_hi, graph = time_graph(dl, args.steps, args.warmup, args.settle_ms)
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(dl.out, out16):
            raise RuntimeError("W4A16 %s: graph replay differs from the eager output" % name)
        med, lo, hi, launch = ((g_med, g_lo, g_hi, "hip-graph replay") if g_med <= e_med
                               else (e_med, e_lo, e_hi, "eager"))
        n_act = len(wl.active_experts())
        wbytes = n_act * LAYER_BYTES_PER_EXPERT
        r = {"launch": launch, "layer_ms_median": med, "layer_ms_min": lo, "layer_ms_max": hi,
             "layer_ms_eager_median": e_med, "layer_ms_graph_median": g_med,
             "weight_GBps": wbytes / (med * 1e-3) / 1e9,
             "frac_of_hbm_peak": wbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        if name == "ragged570":
            d4 = L.DeviceLayer(wl, weights=weights)
            o4 = d4.forward().view(torch.bfloat16).float()
            o16 = out16.view(torch.bfloat16).float()
            rms = o16.pow(2).mean(dim=1, keepdim=True).sqrt()
            r["max_diff_vs_w4a4_over_row_rms"] = float(((o4 - o16).abs() / rms).max())
            r["rms_diff_vs_w4a4_over_rms"] = float((o4 - o16).pow(2).mean().sqrt()
                                                   / o16.pow(2).mean().sqrt())
            del d4
        res[name] = r
        log(json.dumps({"w4a16": name, **r}))
        del graph, dl
    nbytes = args.flush_mb << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    pts = []
    for M in (1, 8, 32):
        wl = W.make_workload("decode%d" % M)
        dl = L.DeviceLayer(wl, weights=weights, arithmetic="w4a16")
        graph = dl.capture_graph()

        def timed(run):
            def step():
                dst.copy_(src)
                run()

            warm(step, args.warmup, args.settle_ms)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                dst.copy_(src)
                a.record()
                run()
                b.record()
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in ev]))

        g_med, e_med = timed(graph.replay), timed(dl.forward)
        med, launch = (g_med, "hip-graph replay") if g_med <= e_med else (e_med, "eager")
        n_act = len(wl.active_experts())
        wbytes = n_act * LAYER_BYTES_PER_EXPERT
        pts.append({"M": M, "layer_us": med * 1e3, "launch": launch,
                    "layer_us_graph": g_med * 1e3, "layer_us_eager": e_med * 1e3,
                    "weight_GBps": wbytes / (med * 1e-3) / 1e9,
                    "frac_of_hbm_peak": wbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS})
        log(json.dumps({"w4a16_decode": pts[-1]}))
        del graph, dl
    res["decode"] = pts
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode (it would "
              "shard by expert, each GPU running this layer on its share); got --gpus %d"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    from nvfp4_block_scaled_gather_amd import binding as B
    B.load()
    wl, dl, res, weights = run_workload(args.workload, args)
    also = {}
    for name in (n for n in args.also.split(",") if n and n != args.workload):
        if wl.E != 288:
            break
        _, dl2, res2, _ = run_workload(name, args, weights)
        also[name] = res2
        del dl2
    sweep = None
    if not args.no_decode_sweep and wl.E == 288:
        log("decode M sweep")
        sweep = decode_sweep(args, weights)
    w4a16 = None
    if not args.no_w4a16 and wl.E == 288:
        log("W4A16 leg")
        w4a16 = w4a16_leg(args, weights)

    # dominant kernel: the w13 grouped GEMM (one grouped_gemm_nvfp4 call)
    R, H, I = wl.R, wl.H, wl.I
    alg_bytes = (res["active_experts"] * W13_BYTES_PER_EXPERT     # weights, read once
                 + R * H * 9 // 16                                  # NVFP4 activations
                 + R * 2 * I * 4)                                   # fp32 outputs
    achieved = alg_bytes / (res["w13_gemm_ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload),
                "kernel": "grouped_gemm_nvfp4 (w13, N=4096, K=4096) on %s" % args.workload,
                "bytes_per_launch": alg_bytes}
    if not args.no_read_probe:
        log("measured read roofline")
        rp = read_roofline(args.kernel_iters, args.settle_ms)
        roofline["read_peak"] = rp
        roofline["frac_of_read_peak"] = achieved / rp["GBps"]
        roofline["read_peak_frac_of_spec"] = rp["GBps"] / HBM_PEAK_GBPS
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.cpu_experts)
    ms = res["layer_ms_median"]
    line = {
        "metric": METRIC, "value": res["weight_GBps"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "nvfp4",
        "data": "synthetic",
        "config": {"workload": "%s: 288 experts, H=4096, I=2048, %d expert-rows, %d tokens"
                               % (args.workload, R, wl.T),
                   "experts": wl.E, "hidden": H, "intermediate": I, "expert_rows": R,
                   "active_experts": res["active_experts"], "weight_bytes": res["weight_bytes"],
                   "parallelism": "single GPU"},
        "launch": res["launch"],
        "layer_ms": ms, "layer_ms_min": res["layer_ms_min"], "layer_ms_max": res["layer_ms_max"],
        "frac_of_hbm_peak": res["frac_of_hbm_peak"],
        "layer_ms_eager": res["layer_ms_eager_median"],
        "layer_ms_graph": res["layer_ms_graph_median"],
        "frac_of_hbm_peak_eager": res["frac_of_hbm_peak_eager"],
        "w13_gemm_ms": res["w13_gemm_ms"], "w13_weight_GBps": res["w13_GBps"],
        "w2_gemm_ms": res["w2_gemm_ms"], "w2_weight_GBps": res["w2_GBps"],
        "roofline": roofline, "cpu_baseline": cpu, "also": also, "decode_sweep": sweep,
        "w4a16": w4a16,
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
