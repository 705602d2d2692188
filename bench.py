"""Benchmark of the W4A16 MoE expert layer on one MI355X.

One step = one pass of the whole layer over one batch: alignment of the
top-k routing, W13 grouped GEMM with fused dequantisation and SwiGLU, W2
grouped GEMM storing each routed row's routing-weighted output, and the
top-k combine into BF16 (for the indexed layout: the entry point with
internal alignment). Inputs are seeded synthetic tensors already resident in
HBM when timing starts.

Default run: the five configurations of the metric, one after the other on
the same GPU. The headline value is the Kimi-K2.x-shaped decode (indexed
layout: 384 experts, hidden 7168, intermediate 2048, 448 tokens, top-8), the
configuration the metric is quoted on; the tiny layer, the Zipf prefill
(contiguous), the masked decode batch and the TP8 shard are reported beside it
under "per_config", each with its own µs/call, per-call percentiles, roofline
fraction, BF16 output floor, a sampled parity check and a CPU-oracle baseline.
--workload N runs only synth.WORKLOADS[N] (any of the eight).

Timing. The K timed steps are bracketed by stream events only. Per-call
percentiles come from K further calls, each between two events. Per-kernel
durations come from K more steps during which the library records HIP events
around each launch on the launch stream (those events add a few µs between
launches, so they stay out of the timed steps). The roofline's traffic is the
rocprofv3 counter measurement recorded under profiles/ for the same kernel and
workload (null when none matches the current sources).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
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
HEADLINE = 1                   # the Kimi decode layer
PER_CONFIG = {0: "tiny", 1: "decode", 2: "prefill", 3: "masked", 4: "tp8_shard"}
# the metric's targets: decode configurations at >= 60 % of HBM on packed
# weight bytes, prefill configurations at >= 40 % of BF16 MFMA on valid rows
TARGET_FRAC = {"hbm": 0.60, "mfma": 0.40}
CPU_SAMPLE_EXPERTS = 48        # bound of the oracle's sample (dequantised experts)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="keep warming up past --warmup calls until this much wall time has passed: the "
                         "GPU's clocks take ~50-100 ms of load to settle after idle")
    ap.add_argument("--workload", type=int, default=None,
                    help="run only synth.WORKLOADS[N] (default: the five configurations, decode as headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle legs (cpu_baseline, floor and sampled parity)")
    ap.add_argument("--unfused", action="store_true",
                    help="indexed workloads: time the unfused steps (align, gate_up GEMM with a BF16 "
                         "output, SwiGLU, down GEMM with a BF16 output; no combine) instead of the layer")
    ap.add_argument("--dispatch", type=int, default=0, choices=(0, 1, 2, 3),
                    help="indexed small-M token-tile dispatch: 0 semi-static grid over experts "
                         "(default), 1 persistent static ranges, 2 persistent atomic job queue, "
                         "3 semi-static grid over routing blocks")
    ap.add_argument("--cold-calls", type=int, default=0, metavar="N",
                    help="after the timed steps, time N more calls one by one, each after a 1 GiB write "
                         "that evicts the L2s and the MALL, and report their p10/p50/p90")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one call of each workload in a HIP graph (on a stream of its own) "
                         "and time K replays: the layer without host launch overhead")
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


def inputs_sha256(arrays):
    """SHA-256 manifest of the input bytes: each array hashed (large ones per
    leading index, on a thread pool), then the list of digests hashed."""
    import numpy as np
    parts = []
    for a in arrays:
        a = np.ascontiguousarray(a)
        parts.extend([a[i] for i in range(a.shape[0])] if a.ndim >= 3 else [a])
    with cf.ThreadPoolExecutor(8) as ex:
        digests = list(ex.map(lambda p: hashlib.sha256(memoryview(p).cast("B")).digest(), parts))
    return hashlib.sha256(b"".join(digests)).hexdigest()


def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, torch, np):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def percentiles(v):
    import numpy as np
    v = np.asarray(v, dtype=np.float64)
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90)), "calls": int(v.size)}


# --------------------------------------------------------------------------
# One workload on the GPU
# --------------------------------------------------------------------------

class Case:
    """A prepared workload: step() runs one call; rows / touched count the
    valid rows and the experts holding rows; `sample` tells the CPU leg what
    to recompute and `fetch` reads the matching GPU output rows."""


def setup_case(wl, dev_w, args, torch, np, M):
    """Inputs on the device and the step closure for workload `wl`, whose
    canonical weights are already on the device (dev_w)."""
    import synth
    c = Case()
    c.wl = wl
    c.h = M.PreparedWeights(*dev_w, mode=wl.layout)
    h = c.h
    # a graph is captured on a stream of the caller's own (not the null stream);
    # without --graph the calls run on torch's current stream
    stream = torch.cuda.Stream() if args.graph else torch.cuda.current_stream()
    c.stream = stream
    c.inputs = []
    if wl.layout == "indexed":
        x = synth.activations(wl.iseed, wl.T, wl.H)
        ids, tw = synth.routing(wl)
        c.inputs = [x, ids, tw]
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
        c.describe = h.describe(wl.T, wl.topk, ovr=ovr)
        c.rows = int(((ids >= 0) & (ids < wl.E)).sum())
        c.touched = int(np.unique(ids[(ids >= 0) & (ids < wl.E)]).size)
        c.out = out
        c.x, c.ids, c.tw = x, ids, tw

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
            c.out = None
    elif wl.layout == "contiguous" and wl.extra.get("rows_per_expert"):
        # grouped rows already aligned per expert (an EP share after its dispatch); no combine
        rpe = wl.extra["rows_per_expert"]
        total = wl.E * rpe
        a = synth.activations(wl.iseed, total, wl.H)
        c.inputs = [a]
        a_d = to_dev(a, torch, np)
        m_d = to_dev(np.repeat(np.arange(wl.E, dtype=np.int32), rpe), torch, np)
        out = torch.empty((total, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(total, 0, 0), dtype=torch.uint8, device="cuda")
        c.describe = f"M_pad={total}; " + h.describe(total)
        c.rows, c.touched, c.out = total, wl.E, None

        def step():
            h.contiguous(a_d, m_d, out=out, ws=ws, stream=stream)
    elif wl.layout == "contiguous":
        # the contiguous input comes from the library's own align (block 128) + permute
        x = synth.activations(wl.iseed, wl.T, wl.H)
        ids, tw = synth.routing(wl)
        c.inputs = [x, ids, tw]
        x_d, ids_d, tw_d = to_dev(x, torch, np), to_dev(ids, torch, np), to_dev(tw, torch, np)
        hi = M.PreparedWeights(*[to_dev(v, torch, np) for v in synth.stacked_weights(
            synth.scaled(wl, I=32))], mode="indexed")   # align + permute only need E and H
        ovr = {"block_m": 128}
        routing = hi.align(ids_d, ovr=ovr)
        perm = hi.permute(x_d, wl.topk, routing, ovr=ovr)
        total = int(routing[7].item())
        a_d, m_d, src_d = (v[:total].contiguous() for v in perm)

        def route_step():
            # the routing step that makes this input, timed on its own: it
            # writes its own buffers, not the GEMMs' copies above
            hi.align(ids_d, ovr=ovr, routing=routing, stream=stream)
            hi.permute(x_d, wl.topk, routing, ovr=ovr, stream=stream, out=perm)
        c.route_step = route_step
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(total, wl.topk, wl.T), dtype=torch.uint8, device="cuda")
        c.describe = f"M_pad={total}; " + h.describe(total)
        c.rows = wl.T * wl.topk
        c.touched = int(np.unique(ids).size)
        c.out = out
        c.x, c.ids, c.tw = x, ids, tw

        def step():
            h.contiguous(a_d, m_d, src_d, tw_d, wl.T, wl.topk, out=out, ws=ws, stream=stream)
    else:
        a3, mm = synth.masked_inputs(wl)
        c.inputs = [a3, mm]
        a3_d, mm_d = to_dev(a3, torch, np), to_dev(mm, torch, np)
        out = torch.empty((wl.E * wl.max_m, wl.H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(h.workspace_bytes(wl.max_m), dtype=torch.uint8, device="cuda")
        c.describe = h.describe(wl.max_m, expected_m=wl.expected_m)
        c.rows = int(mm.sum())
        c.touched = int((mm > 0).sum())
        c.out = out
        c.a3, c.mm = a3, mm

        def step():
            h.masked(a3_d, mm_d, wl.expected_m, out=out, ws=ws, stream=stream)
    c.step = step
    if args.graph:
        torch.cuda.synchronize()   # inputs written on torch's stream before the calls on c.stream
    return c


def time_case(c, args, torch, np, M):
    """Warmup, K timed steps, K per-call timings and K profiled steps."""
    step, stream = c.step, c.stream
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
    # per-call spread: K more calls, each between two events of its own
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = percentiles([a.elapsed_time(b) * 1e3 for a, b in ev])
    # per-kernel durations: K more calls with the library's HIP events around
    # each launch on its stream
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
    log(f"  {c.wl.name}: {ms * 1e3:.1f} us/call timed, per call p50 {per_call['p50']:.1f}, "
        f"profiled {p0.elapsed_time(p1) / args.steps * 1e3:.1f}")
    log("  kernels (avg us): " + ", ".join(f"{k}={v[1] / v[0] * 1e3:.1f}" for k, v in sorted(kernels.items())))
    return dict(ms=ms, per_call=per_call, kernels=kernels, host_us=host_us, warm_ms=warm_ms)


def roofline(wl, kernels, rows, touched):
    """Roofline of the dominant kernel, the W13 grouped GEMM. Few rows per
    expert: bound by HBM on its packed weight bytes (every touched expert's
    W13 streamed once, H*2I/2 bytes). Many rows per expert: bound by MFMA on
    valid-row flops (2*H*2I per row)."""
    dom = next((k for k in kernels if k.startswith("gemm_w13")), "gemm_w13")
    n, tot_ms = kernels.get(dom, (0, 0.0))
    dom_us = tot_ms / max(n, 1) * 1e3
    if rows / max(touched, 1) < 80:
        work = touched * wl.H * wl.I
        achieved = work / (dom_us * 1e-6) / 1e9 if dom_us > 0 else 0.0
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None, "avg_us": dom_us, "bytes_per_launch": work}
    else:
        work = rows * 4.0 * wl.H * wl.I
        achieved = work / (dom_us * 1e-6) / 1e12 if dom_us > 0 else 0.0
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None, "avg_us": dom_us,
                "flops_per_launch": work}
    roof["traffic"] = measured_traffic(wl.name, dom)
    return roof


def layer_figures(wl, ms, rows, touched):
    """Whole-layer rates: packed weight bytes of the touched experts (both
    GEMMs, 1.5*H*I bytes an expert) and valid-row flops (6*H*I a row)."""
    packed = touched * 1.5 * wl.H * wl.I
    flops = rows * 6.0 * wl.H * wl.I
    gbs = packed / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    bound = "hbm" if rows / max(touched, 1) < 80 else "mfma"
    frac = gbs / HBM_PEAK_GBS if bound == "hbm" else tfs / BF16_PEAK_TFLOPS
    return {"layer_packed_GBps": gbs, "layer_packed_frac_hbm": gbs / HBM_PEAK_GBS, "layer_TFLOPs": tfs,
            "layer_frac_mfma": tfs / BF16_PEAK_TFLOPS, "layer_bound": bound, "layer_frac": frac,
            "target_frac": TARGET_FRAC[bound], "meets_target": frac >= TARGET_FRAC[bound]}


# --------------------------------------------------------------------------
# The CPU oracle leg: a bounded sample of the same workload
# --------------------------------------------------------------------------

def token_sample(ids, max_experts):
    """Leading tokens whose routed experts number at most max_experts (at
    least one token)."""
    import numpy as np
    seen, n = set(), 0
    for r in ids:
        s = seen | set(int(v) for v in r if v >= 0)
        if n and len(s) > max_experts:
            break
        seen, n = s, n + 1
    return np.arange(n), len(seen)


def cpu_sample(c):
    """What the CPU leg recomputes for workload c.wl, chosen from its inputs
    alone: the whole call when it is small (the tiny layer, the TP8 shard),
    else the leading tokens whose rows touch at most CPU_SAMPLE_EXPERTS
    experts (indexed, contiguous), or the first CPU_SAMPLE_EXPERTS experts
    holding rows (masked). Returns (kind, ids, output rows to read)."""
    import numpy as np
    wl = c.wl
    if wl.layout == "masked":
        experts = [e for e in range(wl.E) if c.mm[e] > 0][:CPU_SAMPLE_EXPERTS]
        rows = np.concatenate([np.arange(e * wl.max_m, e * wl.max_m + c.mm[e]) for e in experts])
        return "experts", np.array(experts), rows
    if wl.E * wl.H * wl.I <= 384 * 7168 * 256:
        tok = np.arange(wl.T)
    else:
        tok, _ = token_sample(c.ids, CPU_SAMPLE_EXPERTS)
    return "tokens", tok, tok


def cpu_leg(data, w, kind, sel, got):
    """Time the oracle as it stands on a bounded sample of one workload and
    compare the GPU's output rows `got` with it. `data` holds the workload and
    its host inputs. Returns (cpu_baseline, parity). The sample and its
    scaling to one call are stated in the record; BLAS runs on the process's
    CPUs (cores = len(sched_getaffinity))."""
    import numpy as np
    from oracle import moe_oracle as O
    wl = data["wl"]
    touched = data["touched"]
    cores = cpu_cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(cores)
    except Exception:
        limiter = None
    try:
        if kind == "experts":
            experts = [int(e) for e in sel]
            a3, mm = data["a3"], data["mm"]
            t0 = time.perf_counter()
            ref = O.moe_masked(a3[experts], mm[experts], lambda i: tuple(v[experts[i]] for v in w))
            dt = time.perf_counter() - t0
            ref_rows = np.concatenate([ref[i * wl.max_m:i * wl.max_m + mm[e]] for i, e in enumerate(experts)])
            scale = touched / len(experts)
            sample = (f"experts {experts[0]}..{experts[-1]} ({len(experts)} of the {touched} holding rows) "
                      f"with all their valid rows ({dt:.1f} s), scaled x{scale:.2f} to one call")
            what = f"{ref_rows.shape[0]} rows of {len(experts)} experts"
        else:
            tok = sel
            ids = data["ids"]
            n_exp = int(np.unique(ids[tok][(ids[tok] >= 0) & (ids[tok] < wl.E)]).size)
            runs = 5 if wl.E * wl.H * wl.I < 1 << 24 else 1
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                ref_rows = O.moe_indexed(data["x"], ids, data["tw"], lambda e: tuple(v[e] for v in w), E=wl.E,
                                         tokens=tok)
                times.append(time.perf_counter() - t0)
            dt = float(np.median(times))
            scale = touched / max(n_exp, 1)
            if tok.size == wl.T:
                scale = 1.0
                sample = f"the whole call ({dt:.1f} s{', median of 5' if runs > 1 else ''})"
            else:
                sample = (f"tokens 0..{tok[-1]} of {wl.T} with all their top-{wl.topk} rows, {n_exp} experts "
                          f"dequantised ({dt:.1f} s), scaled x{scale:.2f} by the {touched} experts one "
                          f"call touches")
            what = f"{tok.size} tokens"
        m = O.compare(got, ref_rows)
    finally:
        if limiter is not None:
            limiter.unregister()
    base = {"value": dt * 1e6 * scale, "unit": "us/call", "cores": cores, "kind": "oracle", "sample": sample}
    par = {"rel_fro": m["rel_fro"], "max_abs_over_rms": m["max_abs_over_rms"], "bf16_floor": m["bf16_floor"],
           "n": m["n"], "over": what,
           "pass": bool(m["rel_fro"] <= 5e-3 and m["max_abs_over_rms"] <= max(3e-2, m["bf16_floor"] + 5e-3))}
    return base, par


# --------------------------------------------------------------------------

def run_one(idx, w, dev_w, args, torch, np, M, with_cpu):
    """Prepare, time and (optionally) check one workload; returns its record."""
    import synth
    wl = synth.WORKLOADS[idx]
    c = setup_case(wl, dev_w, args, torch, np, M)
    log(f"  schedule: {c.describe}")
    t = time_case(c, args, torch, np, M)
    rec = {"workload": wl.name, "layout": wl.layout, "us_per_call": t["ms"] * 1e3,
           "per_call_us": t["per_call"], "roofline": roofline(wl, t["kernels"], c.rows, c.touched),
           "kernels_avg_us": {k: v[1] / v[0] * 1e3 for k, v in t["kernels"].items()},
           "rows": c.rows, "experts_touched": c.touched, "schedule": c.describe}
    rec.update(layer_figures(wl, t["ms"], c.rows, c.touched))
    rec["warmup_calls"] = len(t["host_us"])
    rec["warmup_ms"] = t["warm_ms"]
    rec["host_us_per_call"] = float(np.median(t["host_us"])) if t["host_us"] else None
    if args.cold_calls > 0:
        rec["per_call_flushed_us"] = cold_calls(c.step, c.stream, args.cold_calls)
    if getattr(c, "route_step", None) is not None:
        rec["routing_step"] = time_route(c, args, torch, M)
    if args.graph:
        rec["graph_replay"] = time_graph(c, args, torch)
    rec["inputs_sha256"] = inputs_sha256(list(w) + c.inputs)
    if with_cpu and c.out is not None:
        # the GPU rows of the sample are read now; the oracle runs after every
        # workload has been timed, on the host inputs kept here
        kind, sel, rows = cpu_sample(c)
        bits = c.out[torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()].contiguous()
        got = (bits.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16) \
            .view(np.float32).astype(np.float64)
        data = {"wl": wl, "touched": c.touched}
        for k in ("x", "ids", "tw", "a3", "mm"):
            if hasattr(c, k):
                data[k] = getattr(c, k)
        rec["_cpu"] = (data, kind, sel, got)
    del c
    return rec


def time_graph(c, args, torch):
    """One call captured in a HIP graph on the workload's stream (inputs,
    output and workspace are the step's fixed buffers), then K replays
    between two events on that stream. Returns µs per replayed call."""
    c.step()   # warm (already warm after the timed steps)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=c.stream):
        c.step()
    torch.cuda.synchronize()
    with torch.cuda.stream(c.stream):
        for _ in range(max(args.warmup, 3)):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(c.stream)
    with torch.cuda.stream(c.stream):
        for _ in range(args.steps):
            g.replay()
    e1.record(c.stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    log(f"  {c.wl.name} graph replay: {us:.1f} us/call")
    return {"us_per_call": us, "replays": args.steps}


def time_route(c, args, torch, M):
    """The align + permute that produce the contiguous input, timed apart from
    the layer call (which takes that input ready-made): warmup, then K calls
    between two stream events, and the per-kernel durations of K more."""
    for _ in range(max(args.warmup, 3)):
        c.route_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(c.stream)
    for _ in range(args.steps):
        c.route_step()
    e1.record(c.stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    M.profile_reset()
    M.profile_enable(True)
    for _ in range(args.steps):
        c.route_step()
    torch.cuda.synchronize()
    M.profile_enable(False)
    kernels = {k: v[1] / v[0] * 1e3 for k, v in M.profile_read().items()}
    log(f"  {c.wl.name} routing step (align + permute): {us:.1f} us/call; " +
        ", ".join(f"{k}={v:.1f}" for k, v in sorted(kernels.items())))
    return {"what": "align (128-row blocks) + permute of the T x topk rows, outside us_per_call",
            "us_per_call": us, "kernels_avg_us": kernels}


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
    return dict(percentiles(us), flush_bytes=1 << 30)


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

    single = args.workload is not None
    head = args.workload if single else HEADLINE
    if args.unfused and synth.WORKLOADS[head].layout != "indexed":
        print(f"--unfused runs the indexed layout's steps; workload {head} is {synth.WORKLOADS[head].layout}",
              file=sys.stderr)
        sys.exit(2)
    order = [head] if single else [HEADLINE, 2, 3, 4, 0]
    with_cpu = not args.no_cpu_baseline
    weights = {}          # (wseed, E, H, I) -> (host arrays, device arrays)
    recs = {}
    for idx in order:
        wl = synth.WORKLOADS[idx]
        key = (wl.wseed, wl.E, wl.H, wl.I)
        if key not in weights:
            for k in list(weights):       # one weight set on the device at a time
                del weights[k]
            torch.cuda.empty_cache()
            log(f"workload {wl.name}: generating weights")
            t = time.time()
            w = synth.stacked_weights(wl)
            log(f"  generated in {time.time() - t:.1f} s; uploading")
            weights[key] = (w, [to_dev(a, torch, np) for a in w])
        w, dev_w = weights[key]
        log(f"workload {wl.name}")
        recs[idx] = run_one(idx, w, dev_w, args, torch, np, M, with_cpu)
        recs[idx]["_w"] = w
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    if with_cpu:
        for idx in order:
            r = recs[idx]
            if "_cpu" not in r:
                continue
            data, kind, sel, got = r.pop("_cpu")
            log(f"CPU oracle leg: {r['workload']}")
            r["cpu_baseline"], r["parity"] = cpu_leg(data, r["_w"], kind, sel, got)
            log(f"  {r['cpu_baseline']['value'] / 1e6:.1f} s/call; parity {r['parity']}")
    for r in recs.values():
        r.pop("_w", None)
        r.pop("_cpu", None)

    h = recs[head]
    wl = synth.WORKLOADS[head]
    result = {
        "metric": METRIC,
        "value": h["us_per_call"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["us_per_call"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layout": wl.layout, "experts": wl.E, "hidden": wl.H,
                   "intermediate": wl.I, "tokens": wl.T, "topk": wl.topk, "rows": h["rows"],
                   "experts_touched": h["experts_touched"], "weights": "uint4 g32 bf16-scale",
                   "dispatch": ["semi-static", "persistent-static", "persistent-queue",
                                "semi-static-blocks"][args.dispatch],
                   "steps": "unfused: align, gate_up, swiglu, down (BF16 hand-offs, no combine)"
                   if args.unfused else "fused layer",
                   "inputs_sha256": h["inputs_sha256"]},
        "roofline": h["roofline"],
        "per_call_us": h["per_call_us"],
        "kernels_avg_us": h["kernels_avg_us"],
        "warmup_calls": h["warmup_calls"],
        "warmup_ms": h["warmup_ms"],
        "host_us_per_call": h["host_us_per_call"],
    }
    for k in ("layer_packed_GBps", "layer_packed_frac_hbm", "layer_TFLOPs", "layer_frac_mfma"):
        result["config"][k] = h[k]
    if "per_call_flushed_us" in h:
        result["per_call_flushed_us"] = h["per_call_flushed_us"]
    if "graph_replay" in h:
        result["graph_replay"] = h["graph_replay"]
    if "cpu_baseline" in h:
        result["cpu_baseline"] = h["cpu_baseline"]
    if "parity" in h:
        result["parity"] = h["parity"]
    if not single:
        result["per_config"] = {PER_CONFIG[i]: recs[i] for i in order}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
