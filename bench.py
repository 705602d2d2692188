"""Benchmark of the W4A16 MoE expert layer on one MI355X.

One step = one pass of the whole layer over one batch: alignment of the
top-k routing, W13 grouped GEMM with fused dequantisation and SwiGLU, W2
grouped GEMM storing each routed row's routing-weighted output, and the
top-k combine into BF16 (for the indexed layout: the entry point with
internal alignment). Inputs are seeded synthetic tensors already resident in
HBM when timing starts.

Default workload: Kimi-K2.x-shaped decode, indexed layout (384 experts,
hidden 7168, intermediate 2048, 448 tokens, top-8). --workload picks any of
the eight (synth.WORKLOADS).

Prints one JSON line. The K timed steps are bracketed by stream events only.
Per-kernel durations come from K further steps during which the library
records HIP events around each launch on the launch stream (those events add
a few µs between launches, so they stay out of the timed steps). The
roofline's traffic is the rocprofv3 counter measurement recorded under
profiles/ for the same kernel and workload (null when none matches the
current sources).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs/call; decode weight GB/s & prefill TFLOP/s as % of roofline"
# HBM traffic of the dominant kernel as measured with rocprofv3 TCC counters
# (profiles/); reported only while the sources it was measured on are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
TRAFFIC_SOURCES = ["moe_gemm_small_m.hip", "moe_gemm_large_m.hip", "moe_device.h", "moe_layout.h", "moe_tile.h",
                   "moe_launch.h", "moe_api.cpp"]
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense BF16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="keep warming up past --warmup calls until this much wall time has passed: the "
                         "GPU's clocks take ~50-100 ms of load to settle after idle")
    ap.add_argument("--workload", type=int, default=1,
                    help="index into synth.WORKLOADS (1: the Kimi decode layer, the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="indexed workloads: time the unfused steps (align, gate_up GEMM with a BF16 "
                         "output, SwiGLU, down GEMM with a BF16 output; no combine) instead of the layer")
    ap.add_argument("--dispatch", type=int, default=0, choices=(0, 1, 2, 3),
                    help="indexed small-M token-tile dispatch: 0 semi-static grid over experts "
                         "(default), 1 persistent static ranges, 2 persistent atomic job queue, "
                         "3 semi-static grid over routing blocks")
    ap.add_argument("--cpu-experts", type=int, default=48, help="experts in the oracle's timed sample")
    ap.add_argument("--cold-calls", type=int, default=0, metavar="N",
                    help="after the timed steps, time N more calls one by one, each after a 1 GiB write "
                         "that evicts the L2s and the MALL, and report their p10/p50/p90")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (steps times), the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(mib, steps):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes": n, "ms_per_copy": ms, "GBps_read_plus_write": 2 * n / ms / 1e6}))


def sources_sha256():
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "w4a16_int4_grouped_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """Bytes read + written per launch by `kernel` on `workload`, from the
    counter record, or None when there is none or the sources changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    sha = sources_sha256()
    for r in recs:
        if r["workload"] == workload and r["kernel"] == kernel and r["sources_sha256"] == sha:
            return r["fetch_bytes"] + r["write_bytes"]
    return None


def cold_calls(step, stream, n):
    """Per-call µs of n calls, each timed alone with HIP events on the call's
    stream after a 1 GiB write that evicts the L2s and the 256 MB MALL."""
    import numpy as np
    import torch
    scratch = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    with torch.cuda.stream(stream):
        for i in range(n):
            scratch.fill_(i)
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
            "p90": float(np.percentile(us, 90)), "calls": n, "flush_bytes": 1 << 30}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, torch, np):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(wl, w, x, ids, tw, n_experts):
    """The oracle as it stands, on a bounded sample: experts 0..n-1 with all
    the rows routed to them (dequantisation, both GEMMs, SwiGLU and their
    share of the combine), scaled by E / n to a whole call."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    experts = list(range(min(n_experts, wl.E)))
    t0 = time.perf_counter()
    for e in experts:
        rows = np.argwhere(ids == e)
        if rows.size == 0:
            continue
        w13 = O.dequant(w[0][e], w[1][e])
        w2 = O.dequant(w[2][e], w[3][e])
        _, _, y = O.expert_ffn(x[rows[:, 0]], w13, w2)
        _ = tw[rows[:, 0], rows[:, 1]][:, None].astype(np.float64) * y
    dt = time.perf_counter() - t0
    per_call_us = dt * 1e6 * wl.E / len(experts)
    return {"value": per_call_us, "unit": "us/call", "cores": int(threads), "kind": "oracle",
            "sample": f"experts 0..{len(experts) - 1} of {wl.E} with all their routed rows "
                      f"({dt:.1f} s), scaled x{wl.E / len(experts):.0f} to one call"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import w4a16_int4_grouped_amd as M

    wl = synth.WORKLOADS[args.workload]
    if args.unfused and wl.layout != "indexed":
        print(f"--unfused runs the indexed layout's steps; workload {args.workload} is {wl.layout}",
              file=sys.stderr)
        sys.exit(2)
    log(f"workload {wl.name}: generating inputs")
    t = time.time()
    w = synth.stacked_weights(wl)
    log(f"  generated weights in {time.time() - t:.1f} s; uploading and preparing")
    dw = [to_dev(a, torch, np) for a in w]
    h = M.PreparedWeights(*dw, mode=wl.layout)
    del dw
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    x = ids = tw = None

    if wl.layout == "indexed":
        x = synth.activations(wl.iseed, wl.T, wl.H)
        ids, tw = synth.routing(wl)
        x_d, ids_d, tw_d = to_dev(x, torch, np), to_dev(ids, torch, np), to_dev(tw, torch, np)
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        ovr = {"dispatch": args.dispatch} if args.dispatch else None
        Eg = wl.extra.get("global_experts", 0)
        if Eg:   # expert-parallel share: experts 0 .. E-1 of the Eg global ones
            ovr = dict(ovr or {}, global_experts=Eg)
            emap = np.full(Eg, -1, dtype=np.int32)
            emap[:wl.E] = np.arange(wl.E)
            map_d = to_dev(emap, torch, np)
            ids = np.where((ids >= 0) & (ids < wl.E), ids, -1)   # the share's rows, for the counts
        ws = torch.empty(h.workspace_bytes(wl.T, wl.topk, wl.T, ovr=ovr), dtype=torch.uint8, device="cuda")
        log(f"  schedule: {h.describe(wl.T, wl.topk, ovr=ovr)}")
        rows = int(((ids >= 0) & (ids < wl.E)).sum())
        touched = int(np.unique(ids[(ids >= 0) & (ids < wl.E)]).size)

        def step():
            h.indexed(x_d, ids_d, tw_d, out=out, ws=ws, stream=stream, ovr=ovr)

        if Eg:
            routing_ep = torch.empty(h.routing_layout(wl.T, wl.topk, ovr).total_ints, dtype=torch.int32,
                                     device="cuda")

            def step():
                h.align_ep(ids_d, map_d, Eg, ovr=ovr, routing=routing_ep, stream=stream)
                h.indexed(x_d, ids_d, tw_d, routing=routing_ep, out=out, ws=ws, stream=stream, ovr=ovr)

        if args.unfused:
            lay = h.routing_layout(wl.T, wl.topk, ovr)
            routing_buf = torch.empty(lay.total_ints, dtype=torch.int32, device="cuda")
            hbuf = torch.empty((lay.cap, 2 * wl.I), dtype=torch.bfloat16, device="cuda")
            abuf = torch.empty((lay.cap, wl.I), dtype=torch.bfloat16, device="cuda")
            ybuf = torch.empty((lay.cap, wl.H), dtype=torch.bfloat16, device="cuda")

            def step():
                h.align(ids_d, ovr=ovr, routing=routing_buf, stream=stream)
                h.gate_up(x_d, wl.topk, routing_buf, out=hbuf, ovr=ovr, stream=stream)
                M.swiglu(hbuf, out=abuf, stream=stream)
                h.down(abuf, wl.T, wl.topk, routing_buf, out=ybuf, ovr=ovr, stream=stream)
    elif wl.layout == "contiguous" and wl.extra.get("rows_per_expert"):
        # grouped rows already aligned per expert (an EP share after its dispatch); no combine
        rpe = wl.extra["rows_per_expert"]
        total = wl.E * rpe
        a_d = to_dev(synth.activations(wl.iseed, total, wl.H), torch, np)
        m_d = to_dev(np.repeat(np.arange(wl.E, dtype=np.int32), rpe), torch, np)
        out = torch.empty((total, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(total, 0, 0), dtype=torch.uint8, device="cuda")
        log(f"  M_pad={total}; schedule: {h.describe(total)}")
        rows = total
        touched = wl.E

        def step():
            h.contiguous(a_d, m_d, out=out, ws=ws, stream=stream)
    elif wl.layout == "contiguous":
        # the contiguous input comes from the library's own align (block 128) + permute
        x = synth.activations(wl.iseed, wl.T, wl.H)
        ids, tw = synth.routing(wl)
        x_d, ids_d, tw_d = to_dev(x, torch, np), to_dev(ids, torch, np), to_dev(tw, torch, np)
        hi = M.PreparedWeights(*[to_dev(a, torch, np) for a in synth.stacked_weights(
            synth.scaled(wl, I=32))], mode="indexed")   # align + permute only need E and H
        ovr = {"block_m": 128}
        routing = hi.align(ids_d, ovr=ovr)
        a_d, m_d, src_d = hi.permute(x_d, wl.topk, routing, ovr=ovr)
        total = int(routing[7].item())
        a_d, m_d, src_d = a_d[:total].contiguous(), m_d[:total].contiguous(), src_d[:total].contiguous()
        del hi, routing
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(total, wl.topk, wl.T), dtype=torch.uint8, device="cuda")
        log(f"  M_pad={total}; schedule: {h.describe(total)}")
        rows = wl.T * wl.topk
        touched = int(np.unique(ids).size)

        def step():
            h.contiguous(a_d, m_d, src_d, tw_d, wl.T, wl.topk, out=out, ws=ws, stream=stream)
    else:
        a3, mm = synth.masked_inputs(wl)
        a3_d, mm_d = to_dev(a3, torch, np), to_dev(mm, torch, np)
        out = torch.empty((wl.E * wl.max_m, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(wl.max_m), dtype=torch.uint8, device="cuda")
        log(f"  schedule: {h.describe(wl.max_m, expected_m=wl.expected_m)}")
        rows = int(mm.sum())
        touched = int((mm > 0).sum())

        def step():
            h.masked(a3_d, mm_d, wl.expected_m, out=out, ws=ws, stream=stream)

    # warmup: at least --warmup calls and --warmup-ms of wall time, in groups
    # of 8 calls with a synchronisation after each, so that the wall time
    # follows the GPU; the host API overhead (wall time to enqueue one call,
    # no synchronisation) is the median over these calls
    host_us = []
    t_warm = time.perf_counter()
    while len(host_us) < args.warmup or (time.perf_counter() - t_warm) * 1e3 < args.warmup_ms:
        for _ in range(8 if len(host_us) >= args.warmup else min(8, args.warmup - len(host_us))):
            t0 = time.perf_counter()
            step()
            host_us.append((time.perf_counter() - t0) * 1e6)
        torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t_warm) * 1e3
    # the timed steps: stream events around all K calls and nothing in between
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel durations: K more calls with the library's HIP events around
    # each launch on its stream (the events add a few µs between launches,
    # so they stay out of the timed steps)
    M.profile_reset()
    M.profile_enable(True)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(args.steps):
        step()
    p1.record(stream)
    torch.cuda.synchronize()
    M.profile_enable(False)
    kernels = M.profile_read()
    log(f"  profiled steps: {p0.elapsed_time(p1) / args.steps * 1e3:.1f} us/call (timed: {ms * 1e3:.1f})")
    log("  kernels (avg us): " + ", ".join(f"{k}={v[1] / v[0] * 1e3:.1f}" for k, v in sorted(kernels.items())))

    # dominant kernel: the W13 grouped GEMM. Few rows per expert: bound by HBM
    # on its packed weight bytes (every touched expert's W13 streamed once).
    # Many rows per expert: bound by MFMA on valid-row flops (4*H*I per row).
    dom = next((k for k in kernels if k.startswith("gemm_w13")), "gemm_w13")
    n, tot_ms = kernels.get(dom, (0, 0.0))
    dom_us = tot_ms / max(n, 1) * 1e3
    rows_per_expert = rows / max(touched, 1)
    layer_packed = touched * 1.5 * wl.H * wl.I
    layer_flops = rows * 6.0 * wl.H * wl.I
    if rows_per_expert < 80:
        work = touched * wl.H * wl.I            # packed W13 bytes: 2I rows x H/2 bytes
        achieved = work / (dom_us * 1e-6) / 1e9 if dom_us > 0 else 0.0
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None, "avg_us": dom_us, "bytes_per_launch": work}
    else:
        work = rows * 4.0 * wl.H * wl.I         # valid-row W13 flops
        achieved = work / (dom_us * 1e-6) / 1e12 if dom_us > 0 else 0.0
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None, "avg_us": dom_us,
                "flops_per_launch": work}
    roof["traffic"] = measured_traffic(wl.name, dom)
    result = {
        "metric": METRIC,
        "value": ms * 1e3,
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layout": wl.layout, "experts": wl.E, "hidden": wl.H,
                   "intermediate": wl.I, "tokens": wl.T, "topk": wl.topk, "rows": rows,
                   "experts_touched": touched, "weights": "uint4 g32 bf16-scale",
                   "dispatch": ["semi-static", "persistent-static", "persistent-queue",
                                "semi-static-blocks"][args.dispatch],
                   "steps": "unfused: align, gate_up, swiglu, down (BF16 hand-offs, no combine)"
                   if args.unfused else "fused layer",
                   "layer_packed_GBps": layer_packed / (ms * 1e-3) / 1e9,
                   "layer_packed_frac_hbm": layer_packed / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "layer_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
                   "layer_frac_mfma": layer_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "roofline": roof,
        "kernels_avg_us": {k: v[1] / v[0] * 1e3 for k, v in kernels.items()},
    }
    result["warmup_calls"] = len(host_us)   # --warmup, extended to --warmup-ms of wall time
    result["warmup_ms"] = warm_ms
    if host_us:
        result["host_us_per_call"] = float(np.median(host_us))
    if args.cold_calls > 0:
        result["per_call_flushed_us"] = cold_calls(step, stream, args.cold_calls)
    if not args.no_cpu_baseline and wl.layout == "indexed":
        log("  timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(wl, w, x, ids, tw, args.cpu_experts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
