#!/usr/bin/env python3
"""Benchmark of the groupwise W4 dequantize-GEMM on one MI355X; prints ONE JSON line.

Default workload (the decode / MTP-verify configuration): W4 weights N=12288 x K=5120, one
fp16 scale and zero per 64 columns, codes uniform 0..15, zero-points uniform 6..9, scales
uniform [0.005, 0.02], X ~ N(0, 1) fp16.  A step is one call at each verify width
T = 1, 2 and 4 (three launches, each through the public ``w4_linear`` and the route table).

Cold weights: every weight set here fits in MI355X's 256 MB Infinity Cache, so each launch
reads the next of C >= 1 GiB / W-stream device copies of the packed weights (the cold regime
of the ninfer-3080 performance notes, "Route boundaries are measured here").  Activations stay
resident, as when produced by the previous op.

Every call of the library is capturable (no allocation, no host synchronisation), so the
launches are replayed from HIP graphs, the way a decode loop replays one graph per verify
width; Python launch overhead never sits between two kernels.  The timed region is one replay
of a graph holding exactly `--steps` steps, bracketed by synchronize; value = effective
weight-stream GB/s over it (packed codes + fp16 scales + fp16 zeros per launch, times
launches, divided by the timed wall time).  The per-launch duration of each width comes from
HIP events on the launch stream around replays of a graph of back-to-back launches of that
width (one per cold copy); the widest launch of the step (most work per launch) is the roofline
kernel: its algorithmic bytes (or flops) over that duration give roofline.achieved, and
roofline.traffic is its HBM bytes per launch from the committed counter record
(profiles/traffic_<workload>.json, written by --traffic-summary from rocprofv3 FETCH_SIZE /
WRITE_SIZE runs scaled by the same counters of a plain copy kernel), or null when the kernel
sources changed since the counters were taken.

cpu_baseline is the only place bench.py uses the fp64 oracle: it checks this run's GPU outputs
(256 sampled output columns per width, first launch of each width) against the oracle, and
times the oracle on the host cores over repeats of the same step (about 10-30 s); the timing is
a reference point, not a target.  --no-cpu-baseline skips both (parity is then null).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published

WORKLOADS = {
    # name: (synth config, widths per step, op)
    "decode": ("decode", (1, 2, 4), "linear"),
    "batched": ("batched", (8, 16, 32, 64), "linear"),
    "swiglu": ("swiglu", (1, 4, 16, 64), "swiglu"),
    "prefill": ("prefill", (1024, 4096), "add"),
    # 256 x 512: latency, not bandwidth (the weights fit in L2); reported in us, its GB/s figure
    # is not representative of the weight stream
    "tiny": ("tiny", (1,), "linear"),
    # route-boundary sweep shapes (--route-sweep), not part of the default run
    "q5_k5120": ("q5_k5120", (1, 64), "linear"),
    "q5_down": ("q5_down", (1, 64), "linear"),
    "q4_k17408": ("q4_k17408", (1, 64), "linear"),
    "q5_k8192": ("q5_k8192", (1, 64), "linear"),
    "q5_k12288": ("q5_k12288", (1, 64), "linear"),
    "q4_k8192": ("q4_k8192", (1, 64), "linear"),
    "swiglu_4096": ("swiglu_4096", (1, 64), "swiglu"),
    "swiglu_q5_8192": ("swiglu_q5_8192", (1, 64), "swiglu"),
}
ALL_ORDER = ("decode", "tiny", "batched", "swiglu", "prefill")
METRIC = "W4 GEMM effective weight GB/s (T<=64) and MFMA TFLOP/s (T>=1024), % roofline"


# Sources each measured kernel is built from (its own file, the headers it includes and the
# route table that picks its instance): a traffic record is valid while these are unchanged.
KERNEL_SOURCES = {
    "stream_kernel": ["stream.hip", "device.h", "layout.h", "kernels.h", "api.hip"],
    "narrow_kernel": ["narrow.hip", "tile32.h", "device.h", "layout.h", "kernels.h", "api.hip"],
    "wide_kernel": ["wide.hip", "tile32.h", "device.h", "layout.h", "kernels.h", "api.hip"],
    "regring_kernel": ["regring.hip", "tile32.h", "device.h", "layout.h", "kernels.h", "api.hip"],
    "regring32_kernel": ["regring.hip", "tile32.h", "device.h", "layout.h", "kernels.h", "api.hip"],
}


def kernel_source_sha(files) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4_groupwise_gemm_amd", "csrc")
    for name in sorted(files):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, T: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it still
    describes the current sources of the measured kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    files = rec.get("kernel_sources")
    if not files or rec.get("kernel_src_sha") != kernel_source_sha(files):
        return None
    v = rec.get("bytes_per_launch", {}).get(str(T))
    return None if v is None else float(v)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                    help="one configuration, or all of them in one run (decode is the headline)")
    ap.add_argument("--cold-bytes", type=float, default=1.0, help="GiB of rotated weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--route", type=int, default=-1, help="force one route (bench of a schedule)")
    ap.add_argument("--probe", choices=["copy", "read", "bcast", "lds"], default=None,
                    help="run only a kernel of libw4probe.so: plain copy / read (counter reference, "
                         "HBM read rate), bcast (every workgroup reads the same --probe-mb buffer "
                         "from L2; sweeps grids, registers and direct-to-LDS), lds (LDS read rate "
                         "per compute unit; sweeps waves per workgroup and grids)")
    ap.add_argument("--probe-mb", type=float, default=256.0)
    ap.add_argument("--probe-cold", action="store_true",
                    help="read probe over rotated copies (--cold-bytes GiB), graph-replayed "
                         "back to back like the GEMM launches: the cold-read ceiling at that size")
    ap.add_argument("--probe-grid", type=int, default=2048, help="workgroups of the probe kernels")
    ap.add_argument("--probe-unroll", type=int, default=1, choices=[1, 2, 4, 8],
                    help="independent 16-byte loads in flight per lane in the read probe")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="with --probe read --probe-cold: sweep unroll 1/2/4/8 x grid 256..16384 and "
                         "report the fastest (the cold-read ceiling at --probe-mb)")
    ap.add_argument("--widths", default=None,
                    help="comma list of T overriding the workload's widths (counter runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch eagerly instead of replaying HIP graphs (counter runs)")
    ap.add_argument("--traffic-summary", default=None, metavar="DIR",
                    help="no GPU work: turn the FETCH_SIZE / WRITE_SIZE counter runs under DIR "
                         "(subdirs fetch, write, copy_fetch, copy_write) into the traffic record")
    ap.add_argument("--kernel-match", default=None,
                    help="substring of the measured kernel's name (with --traffic-summary)")
    ap.add_argument("--route-sweep", action="store_true",
                    help="time every route whose T domain holds each width (graph replays of "
                         "back-to-back launches over the cold copies); prints one JSON line")
    ap.add_argument("--copy-mb", type=float, default=256.0,
                    help="--probe-mb of the copy runs (with --traffic-summary)")
    args = ap.parse_args()

    if args.traffic_summary:
        return traffic_summary(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (each GPU runs the "
              "same kernels on its own shard); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import w4_groupwise_gemm_amd as w4

    if args.probe:
        return run_probe(args)

    if args.workload != "all":
        line = run_workload(args, args.workload, torch, w4, cpu_timing=not args.no_cpu_baseline)
        if isinstance(line, int):  # route sweep
            return line
        print(json.dumps(line))
        return 1 if line["parity_ok"] is False else 0

    # Every configuration in one run: decode (the headline, at T = 1, 2, 4) first, then the others,
    # each with its own cold copies (freed before the next), parity sample and roofline.  The
    # oracle's timing runs once, on the decode step.
    if args.widths or args.route >= 0 or args.route_sweep:
        print("--widths, --route and --route-sweep take one --workload", file=sys.stderr)
        return 2
    lines = {}
    for name in ALL_ORDER:
        lines[name] = run_workload(args, name, torch, w4,
                                   cpu_timing=(name == "decode" and not args.no_cpu_baseline))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    line = dict(lines["decode"])
    line["per_config"] = {n: {k: v for k, v in l.items() if k not in
                              ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
                               "data", "cpu_baseline")}
                          for n, l in lines.items()}
    oks = [l["parity_ok"] for l in lines.values()]
    line["parity_ok"] = None if any(v is None for v in oks) else all(oks)
    line["metric"] = METRIC
    print(json.dumps(line))
    return 1 if line["parity_ok"] is False else 0


def run_workload(args, wname, torch, w4, cpu_timing):
    """Time one workload (all its widths) and check its outputs; returns the JSON record (or the
    exit status of a route sweep)."""
    from synth import make_workload

    cfg_name, widths, opname = WORKLOADS[wname]
    all_widths = widths
    if args.widths and args.workload != "all":
        widths = tuple(int(v) for v in args.widths.split(","))
        # X is drawn once at the largest width (so a token's row is the same at every width)
        all_widths = tuple(sorted(set(all_widths) | set(widths)))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg_name}", file=sys.stderr, flush=True)
    wl = make_workload(cfg_name, Ts=all_widths)
    bits = wl.weights[0].bits
    K = wl.weights[0].K
    if opname == "swiglu":
        g, u = wl.weights
        packed = w4.repack_pair((g.lo, g.hi, g.scales, g.zeros), (u.lo, u.hi, u.scales, u.zeros), bits)
        N, pair, op = g.N, True, w4.OP_SWIGLU
        rows = 2 * N
    else:
        if len(wl.weights) > 1:  # parents sharing one activation: one N-concatenated matrix
            lo = np.concatenate([ws.lo for ws in wl.weights])
            sc = np.concatenate([ws.scales for ws in wl.weights])
            ze = np.concatenate([ws.zeros for ws in wl.weights])
            hi = None if bits == 4 else np.concatenate([ws.hi for ws in wl.weights])
        else:
            ws = wl.weights[0]
            lo, hi, sc, ze = ws.lo, ws.hi, ws.scales, ws.zeros
        packed = w4.repack(lo, hi, sc, ze, bits)
        N, pair = lo.shape[0], False
        op = w4.OP_ADD if opname == "add" else w4.OP_LINEAR
        rows = N
    wstream = sum(int(a.nbytes) for a in packed)  # codes + scales + zeros as laid out
    wstream_alg = rows * K * bits // 8 + rows * (K // 64) * 4
    # (at most 512 copies: the tiny workload's 74 KB would otherwise ask for ~14,000; its
    # launches are latency bound and its copies stay within the Infinity Cache anyway)
    copies = min(512, max(2, int(np.ceil(args.cold_bytes * (1 << 30) / wstream))))
    print(f"[bench] {copies} cold copies of {wstream / 1e6:.2f} MB", file=sys.stderr, flush=True)
    pws = [w4.to_device(packed, N, K, bits, pair, device=dev) for _ in range(copies)]
    x_all = torch.from_numpy(wl.x).to(dev)
    xs = {T: x_all[:T].contiguous() for T in widths}
    res = {T: torch.from_numpy(wl.r[:T]).to(dev) for T in widths} if wl.r is not None else {}
    outs = {T: torch.empty((T, N), dtype=torch.float16, device=dev) for T in widths}

    def call(T, pw):
        if args.route >= 0:
            return w4.linear_route(args.route, op, xs[T], pw, residual=res.get(T), out=outs[T])
        if op == w4.OP_SWIGLU:
            return w4.linear_swiglu(xs[T], pw, out=outs[T])
        if op == w4.OP_ADD:
            return w4.linear_add(xs[T], pw, res[T], out=outs[T])
        return w4.linear(xs[T], pw, out=outs[T])

    if args.route_sweep:
        return route_sweep(args, w4, torch, widths, op, pws, xs, res, outs, copies, wstream_alg,
                           N, K, rows, bits)
    print(f"[bench] {wname}: timing T in {list(widths)}", file=sys.stderr, flush=True)

    # ---- outputs of the first launch at each width, kept for the parity check of the
    # cpu_baseline leg (sampled output columns against the fp64 oracle, same run)
    rng = np.random.default_rng(0)
    gpu_out = {}
    for T in widths:
        call(T, pws[0])
        torch.cuda.synchronize()
        cols = np.sort(rng.choice(N, 256, replace=False))
        gpu_out[T] = (cols, outs[T].cpu().numpy().astype(np.float64)[:, cols])

    # ---- timing through HIP graphs: every call is capturable (no allocation, no host sync),
    # so the launches are replayed from graphs and the GPU never waits on Python.
    class Eager:
        """Same interface as a captured graph, launching eagerly (counter runs)."""

        def __init__(self, seq):
            self.seq = list(seq)

        def replay(self):
            for T, c in self.seq:
                call(T, pws[c])

    def capture(seq):
        if args.no_graph:
            return Eager(seq)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for T, c in seq:
                call(T, pws[c])
        return g

    stream = torch.cuda.current_stream()
    # every launch of a step reads a weight copy that no launch has touched since the other
    # copies went through (a copy is never reused inside a step: no Infinity Cache hits)
    def rotation(nsteps):
        return [(T, (s * len(widths) + i) % copies) for s in range(nsteps) for i, T in enumerate(widths)]

    g_warm = capture(rotation(max(1, args.warmup)))
    g_steps = capture(rotation(args.steps))
    g_width = {T: capture([(T, c) for c in range(copies)]) for T in widths}
    # the same number of launches, all on copy 0: the "hot" figure, weights served partly by the
    # 256 MB Infinity Cache (context only; every headline figure above is cold)
    g_hot = {T: capture([(T, 0) for _ in range(copies)]) for T in widths}
    g_warm.replay()
    for g in g_width.values():
        g.replay()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps, one graph replay, bracketed by synchronize
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch duration of each width: HIP events around replays of `copies` back-to-back
    # launches of that width (one per cold copy), on the launch stream; 20 replays, mean with a
    # bootstrap 95% interval
    reps = 20

    def replay_us(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / copies  # us per launch

    boot = np.random.default_rng(12345)
    per_T = {}
    for T in widths:
        d = np.array([replay_us(g_width[T]) for _ in range(reps)])
        means = boot.choice(d, size=(2000, d.size), replace=True).mean(axis=1)
        ci = [float(np.percentile(means, 2.5)), float(np.percentile(means, 97.5))]
        hot = float(np.median([replay_us(g_hot[T]) for _ in range(5)]))
        alg_bytes = wstream_alg + T * K * 2 + T * N * 2 * (2 if op == w4.OP_ADD else 1)
        flops = 2.0 * T * rows * K
        rid = args.route if args.route >= 0 else w4.route_for(op, bits, T, N, K)
        per_T[str(T)] = {
            "route": w4.route_name(rid), "us_mean": float(d.mean()), "us_ci95": ci,
            "us_min": float(d.min()), "us_max": float(d.max()), "launches_timed": reps * copies,
            "us_hot_mall": hot,
            "weight_GBs": wstream_alg / (d.mean() * 1e3), "alg_GBs": alg_bytes / (d.mean() * 1e3),
            "TFLOPs": flops / (d.mean() * 1e6), "alg_bytes": alg_bytes,
        }

    # roofline of the widest launch of the step (the most work per launch)
    dom = max(widths)
    pd = per_T[str(dom)]
    prefill = min(widths) >= 1024
    if prefill:
        achieved, peak, unit, bound = pd["TFLOPs"], MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = pd["alg_GBs"], HBM_PEAK_GBS, "GB/s", "hbm"
    traffic = traffic_from_profiles(wname, dom)
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic,
                "kernel": f"T={dom} {pd['route']}", "alg_bytes_per_launch": pd["alg_bytes"],
                "us_per_launch": pd["us_mean"]}

    ms_per_step = wall * 1e3 / args.steps
    if prefill:
        metric = "W5 LinearAdd MFMA TFLOP/s (T>=1024)"
        value = sum(2.0 * T * rows * K for T in widths) / (ms_per_step * 1e9)
        unit_v = "TFLOP/s"
    else:
        metric = "W4 GEMM effective weight GB/s (T<=64)"
        value = len(widths) * wstream_alg / (ms_per_step * 1e6)
        unit_v = "GB/s"

    context = context_figures(args, w4, torch, wl, widths, bits, K, N, op, pair, per_T, dev, wname,
                              pws, copies)

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(wl, widths, op, bits, lo if not pair else None,
                                   hi if not pair else None, sc if not pair else None,
                                   ze if not pair else None, wstream_alg, prefill, rows, K, gpu_out,
                                   timing=cpu_timing)
        print(f"[bench] {wname} parity {parity}", file=sys.stderr, flush=True)
        if context and "a8_route" in context:
            a8_accuracy(wl, context["a8_route"], bits, op)
    if context and "a8_route" in context:
        for d in context["a8_route"]["per_T"].values():
            d.pop("_sample", None)
    parity_ok = None if parity is None else all(p["ok"] for p in parity.values())

    line = {
        "metric": metric, "value": value, "unit": unit_v, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{wname}: {'SwiGLU pair ' if pair else ''}W{bits} N={N} "
                               f"K={K} group=64, T in {list(widths)}, cold ({copies} copies)",
                   "N": N, "K": K, "bits": bits, "T": list(widths), "op": opname,
                   "cold_copies": copies, "parallelism": "none (1 GPU)"},
        "parity_ok": parity_ok, "parity": parity, "per_T": per_T,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    if context:
        line["context"] = context
    del pws
    return line



def context_figures(args, w4, torch, wl, widths, bits, K, N, op, pair, per_T, dev, wname, pws,
                    copies):
    """Figures reported beside the measured path, never as its value.

    * Parents that share one activation (the batched workload): each parent as a call of its
      own and the sum of the two, beside the one N-concatenated call that per_T times; and the
      two mixed-width (4-bit + 5-bit) input projections through the grouped call, beside the
      same two matrices as two calls.
    * Prefill widths: a dense fp16 GEMM of the same shape through the vendor library (random
      fp16 weights held as [K][N] for x @ W and as [N][K] for linear(x, W)), over rotated cold
      weight copies: the ceiling a dequantising kernel is compared with.
    * Decode and prefill: the same calls with bf16 activations (w4_linear_bf16 /
      w4_linear_add_bf16: the per-token exponent pass plus the fp16 kernel), on the same cold
      copies, beside the fp16 call.
    * Decode: one verify-width decode step of three calls (the input projection of this
      workload, a SwiGLU pair [17408, 5120] and a LinearAdd down projection [5120, 17408]),
      launched eagerly from Python and replayed from a per-width graph set (VerifyGraphs).
    Both timed over >= --cold-bytes of rotated copies, HIP events on the launch stream, median
    of 5 (our calls replayed from a graph, the library's launched eagerly)."""
    if args.route >= 0 or args.no_graph or pair:
        return None
    stream = torch.cuda.current_stream()

    def timed(launch, copies, graph=True):
        # graph: our own calls (capturable); eager for the vendor library, whose launches stay
        # out of graphs here (a 80-280 us GEMM does not notice the launch gap)
        for c in range(min(copies, 4)):
            launch(c)
        torch.cuda.synchronize()
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(copies):
                    launch(c)
            run = g.replay
        else:
            def run():
                for c in range(copies):
                    launch(c)
        run()
        torch.cuda.synchronize()
        us = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / copies)
        return float(np.median(us))

    out = {}
    if len(wl.weights) > 1 and op == w4.OP_LINEAR:
        sep = {str(T): {} for T in widths}
        for ws in wl.weights:
            packed = w4.repack(ws.lo, ws.hi, ws.scales, ws.zeros, bits)
            nbytes = sum(int(a.nbytes) for a in packed)
            copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / nbytes)))
            pws = [w4.to_device(packed, ws.N, K, bits, False, device=dev) for _ in range(copies)]
            for T in widths:
                x = torch.from_numpy(np.ascontiguousarray(wl.x[:T])).to(dev)
                y = torch.empty((T, ws.N), dtype=torch.float16, device=dev)
                sep[str(T)][f"{ws.N}x{K}_us"] = timed(lambda c: w4.linear(x, pws[c], out=y), copies)
            del pws
        for T in widths:
            d = sep[str(T)]
            d["sum_us"] = float(sum(v for k, v in d.items() if k.endswith("_us")))
            d["concatenated_us"] = per_T[str(T)]["us_mean"]
        out["parents_as_separate_calls"] = sep
        out["mixed_bits_parents"] = mixed_bits_parents(w4, torch, args, timed, K, dev)
    if min(widths) >= 1024:
        wbytes = N * K * 2
        copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / wbytes)))
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        # the two operand layouts a caller could hold: W as [K][N] (x @ W) and as [N][K]
        # (linear(x, W) = x @ W^T, a plain 2-D fp16 product), both contiguous
        wkn = [torch.randn((K, N), generator=gen, device=dev, dtype=torch.float16) for _ in range(copies)]
        wnk = [torch.randn((N, K), generator=gen, device=dev, dtype=torch.float16) for _ in range(copies)]
        dense = {}
        for T in widths:
            x = torch.from_numpy(np.ascontiguousarray(wl.x[:T])).to(dev)
            us_kn = timed(lambda c: torch.matmul(x, wkn[c]), copies, graph=False)
            us_nk = timed(lambda c: torch.nn.functional.linear(x, wnk[c]), copies, graph=False)
            best = min(us_kn, us_nk)
            dense[str(T)] = {"us_w_kn": us_kn, "us_w_nk": us_nk, "us_best": best,
                             "TFLOPs_best": 2.0 * T * N * K / (best * 1e6)}
        del wkn, wnk
        out["dense_fp16_gemm_ceiling"] = {"what": "vendor-library fp16 GEMM (torch.matmul / linear) on random "
                                                  "fp16 weights of the same shape, cold copies", "per_T": dense}
        if op in (w4.OP_ADD, w4.OP_LINEAR) and bits in (4, 5):
            out["a8_route"] = a8_route(w4, torch, args, timed, wl, widths, bits, K, N, op, dev)
    if wname in ("decode", "prefill") and len(wl.weights) == 1:
        out["bf16_activations"] = bf16_context(w4, torch, timed, wl, widths, N, K, op, pws, copies,
                                               per_T, dev)
    if wname == "decode":
        out["verify_step_graphs"] = verify_step_context(w4, torch, pws[0], K, dev)
    return out or None


def bf16_context(w4, torch, timed, wl, widths, N, K, op, pws, copies, per_T, dev):
    """bf16 activations and outputs (and residual) through the public bf16 calls, over the
    workload's cold weight copies, graph-replayed: per width the whole call (exponent pass +
    kernel) beside the fp16 call of per_T."""
    res = {}
    for T in widths:
        x = torch.from_numpy(np.ascontiguousarray(wl.x[:T])).to(dev).to(torch.bfloat16)
        r = (torch.from_numpy(np.ascontiguousarray(wl.r[:T])).to(dev).to(torch.bfloat16)
             if op == w4.OP_ADD else None)
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, w4.bf16_workspace_bytes(T, K)), dtype=torch.uint8, device=dev)
        if op == w4.OP_ADD:
            us = timed(lambda c: w4.linear_add_bf16(x, pws[c], r, out=y, workspace=ws), copies)
        else:
            us = timed(lambda c: w4.linear_bf16(x, pws[c], out=y, workspace=ws), copies)
        res[str(T)] = {"us": us, "fp16_us": per_T[str(T)]["us_mean"],
                       "extra_us": us - per_T[str(T)]["us_mean"]}
    return {"what": "bf16 activations, outputs (and residual): per-token exponent pass + fp16 "
                    "kernel, cold copies, graph-replayed", "per_T": res}


def verify_step_context(w4, torch, pw_in, K, dev, widths=(1, 2, 4, 8), steps=20, layers=8):
    """A decode step at a verify width: `layers` layers of three calls each -- y = linear(x,
    W_in), h = swiglu(x, W_gu), o = linear_add(h, W_down, x_res) -- launched eagerly from Python
    and replayed from the width's recorded graph (one launch per step), mean over `steps` steps
    between synchronisations.  Two scales: the decode shapes (W_in this workload's matrix, W_gu a
    [17408, 5120] pair, W_down [5120, 17408]; each kernel 8-25 us, so Python stays ahead of the
    GPU) and small ones (W_in [2048, 1024], W_gu [2048, 1024], W_down [1024, 2048]; each kernel a
    few us, so the launches dominate).  4-bit random packed codes, integer zero-points and N(0, 1)
    activations (the kernels' cost does not depend on the values); the layers share one set of
    weights, hot in the Infinity Cache: this isolates the launch overhead the graph removes."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)

    def rand_pw(N, Kc, pair):
        rows = 2 * N if pair else N
        nb = w4.packed_bytes(rows, Kc, 4)
        nsz = w4.packed_sz_bytes(rows, Kc) // 2
        w = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=dev, generator=gen)
        s = torch.full((nsz,), 0.01, dtype=torch.float16, device=dev).view(torch.int16)
        z = torch.full((nsz,), 8.0, dtype=torch.float16, device=dev).view(torch.int16)
        return w4.PackedWeight(w, s, z, N, Kc, 4, pair)

    scales = {
        "decode_shapes": (pw_in, rand_pw(17408, K, True), rand_pw(5120, 17408, False)),
        "small_shapes": (rand_pw(2048, 1024, False), rand_pw(2048, 1024, True), rand_pw(1024, 2048, False)),
    }
    out = {"what": f"decode step of {layers} layers x 3 calls (input projection, SwiGLU pair, LinearAdd "
                   "down projection), eager Python launches vs. one graph-set replay per step, hot weights",
           "layers": layers}
    for name, (p_in, p_gu, p_dn) in scales.items():
        vg = w4.VerifyGraphs()
        st = vg.stream
        res = {}
        for T in widths:
            x = torch.randn((T, p_in.K), generator=gen, device=dev).to(torch.float16)
            xr = torch.randn((T, p_dn.N), generator=gen, device=dev).to(torch.float16)
            y = torch.empty((T, p_in.N), dtype=torch.float16, device=dev)
            h = torch.empty((T, p_gu.N), dtype=torch.float16, device=dev)
            o = torch.empty((T, p_dn.N), dtype=torch.float16, device=dev)

            def step(T_, x=x, xr=xr, y=y, h=h, o=o, p_in=p_in, p_gu=p_gu, p_dn=p_dn):
                for _ in range(layers):
                    w4.linear(x, p_in, out=y, stream=st)
                    w4.linear_swiglu(x, p_gu, out=h, stream=st)
                    w4.linear_add(h, p_dn, xr, out=o, stream=st)

            def per_step_us(fn):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(steps):
                    fn()
                e1.record(st)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / steps

            with torch.cuda.stream(st):
                eager = per_step_us(lambda: step(T))
            vg.run(T, step)
            torch.cuda.synchronize()
            graph = per_step_us(lambda: vg.run(T))
            res[str(T)] = {"eager_us": eager, "graph_us": graph, "graph_over_eager": graph / eager}
        vg.close()
        out[name] = res
    return out


def a8_route(w4, torch, args, timed, wl, widths, bits, K, N, op, dev):
    """The lossy A8 route on the same workload (int8 activations per 64 columns): per width the
    time of the whole call (quantisation + GEMM), of the quantisation alone and of the GEMM on
    pre-quantised activations, over rotated cold weight copies; effective rate 2 T N K / time.
    Its accuracy against the exact product is added by the oracle leg (a8_accuracy)."""
    ws0 = wl.weights[0]
    packed = w4.repack(ws0.lo, ws0.hi, ws0.scales, ws0.zeros, bits)
    nbytes = sum(int(a.nbytes) for a in packed)
    copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / nbytes)))
    pws = [w4.to_device(packed, N, K, bits, False, device=dev) for _ in range(copies)]
    res = {}
    for T in widths:
        x = torch.from_numpy(np.ascontiguousarray(wl.x[:T])).to(dev)
        r = torch.from_numpy(np.ascontiguousarray(wl.r[:T])).to(dev) if wl.r is not None else None
        y = torch.empty((T, N), dtype=torch.float16, device=dev)
        ws = torch.empty(w4.a8_workspace_bytes(T, K), dtype=torch.uint8, device=dev)

        def call(c, xx=x):
            if op == w4.OP_ADD:
                w4.linear_add_a8(xx, pws[c], r, out=y, workspace=ws, T=T)
            else:
                w4.linear_a8(xx, pws[c], out=y, workspace=ws, T=T)
        us_all = timed(lambda c: call(c), copies)
        us_q = timed(lambda c: w4.quantize_a8(x, workspace=ws), copies)
        w4.quantize_a8(x, workspace=ws)
        us_gemm = timed(lambda c: call(c, None), copies)
        call(0)
        torch.cuda.synchronize()
        cols = np.sort(np.random.default_rng(T).choice(N, 256, replace=False))
        res[str(T)] = {"us": us_all, "us_quantise": us_q, "us_gemm": us_gemm,
                       "TOPs": 2.0 * T * N * K / (us_all * 1e6),
                       "_sample": (cols, y.cpu().numpy().astype(np.float64)[:, cols])}
    del pws
    return {"what": "lossy A8 route: int8 activations with a scale per 64 columns, int8 matrix-core "
                    "steps, per-group rescale (w4_linear*_a8); cold weight copies", "per_T": res}


def a8_accuracy(wl, ctx, bits, op):
    """Oracle leg: relative L2 error of the A8 route's sampled outputs against the exact fp64
    product (the pages hold the route to 0.04)."""
    import oracle
    ws0 = wl.weights[0]
    for T, d in ctx["per_T"].items():
        cols, got = d.pop("_sample")
        T = int(T)
        ref = oracle.linear_rows(wl.x[:T], ws0.lo, ws0.hi, ws0.scales, ws0.zeros, bits, cols)
        if op == 2:
            ref = ref + wl.r[:T][:, cols].astype(np.float64)
        d["rel_l2_vs_exact"] = oracle.rel_l2(got, ref)
        d["within_0.04"] = bool(d["rel_l2_vs_exact"] <= 0.04)


def mixed_bits_parents(w4, torch, args, timed, K, dev):
    """The two mixed-width input projections of the hybrid model (GDN input: 4-bit 4096 rows +
    5-bit 12288 rows; attention input: 4-bit 7168 + 5-bit 7168; K = 5120) at widths across the
    one-launch grouped path: the grouped call against the two single-matrix calls launched
    back to back, over rotated cold copies.  Weights follow the batched workload's
    distribution for the 4-bit parent and the prefill workload's for the 5-bit one."""
    from synth import make_weights, make_activations
    from synth.inputs import CONFIGS
    rng = np.random.default_rng(77)
    x = torch.from_numpy(make_activations(rng, 64, K, 1.0, 8)[0]).to(dev)
    res = {}
    for name, specs in (("gdn_in", ((4096, 4), (12288, 5))), ("attn_in", ((7168, 4), (7168, 5)))):
        packed = []
        for i, (n, b) in enumerate(specs):
            cfg = CONFIGS["batched" if b == 4 else "prefill"]
            ws = make_weights(rng, f"{name}{i}", n, K, b, cfg["zero"], cfg["scale"])
            packed.append(w4.repack(ws.lo, ws.hi, ws.scales, ws.zeros, b))
        nbytes = sum(int(a.nbytes) for p in packed for a in p)
        copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / nbytes)))
        pws = [[w4.to_device(p, n, K, b, False, device=dev) for p, (n, b) in zip(packed, specs)]
               for _ in range(copies)]
        per_T = {}
        for T in (1, 4, 8, 16, 32, 64):
            xt = x[:T].contiguous()
            ys = [torch.empty((T, n), dtype=torch.float16, device=dev) for n, _ in specs]
            g_us = timed(lambda c: w4.linear_grouped(xt, pws[c], outs=ys), copies)

            def both(c):
                for pw, y in zip(pws[c], ys):
                    w4.linear(xt, pw, out=y)
            s_us = timed(both, copies)
            per_T[str(T)] = {"grouped_us": g_us, "two_calls_us": s_us, "saved_us": s_us - g_us}
        res[name] = {"parents": [f"W{b} {n}x{K}" for n, b in specs], "per_T": per_T}
        del pws
    return res


def route_sweep(args, w4, torch, widths, op, pws, xs, res, outs, copies, wstream_alg, N, K, rows,
                bits) -> int:
    """Per-launch time of every route at every width (the data the route boundaries are chosen
    from): graph replays of `copies` back-to-back launches, HIP events, median of 5."""
    stream = torch.cuda.current_stream()
    table = {}
    for T in widths:
        for rid in range(w4.route_count()):
            lo, hi = w4.route_domain(rid)
            if not lo <= T <= hi:
                continue
            name = w4.route_name(rid)

            def one(c, T=T, rid=rid):
                w4.linear_route(rid, op, xs[T], pws[c], residual=res.get(T), out=outs[T])

            one(0)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(copies):
                    one(c)
            g.replay()
            torch.cuda.synchronize()
            samples = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                samples.append(e0.elapsed_time(e1) * 1e3 / copies)
            us = float(np.median(samples))
            table.setdefault(str(T), {})[name] = us
            print(f"[sweep] {args.workload} T={T:5d} {name:18s} {us:9.2f} us  "
                  f"{wstream_alg / us / 1e3:7.0f} GB/s  {2.0 * T * rows * K / us / 1e6:7.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
    best = {T: min(r, key=r.get) for T, r in table.items()}
    picks = {T: w4.route_name(w4.route_for(op, bits, int(T), N, K)) for T in table}
    # the same table as markdown (stderr): one row per width, the fastest route and the public
    # calls' choice, marked with its excess over the fastest when that is above 3 %
    names = [w4.route_name(i) for i in range(w4.route_count())
             if any(w4.route_name(i) in r for r in table.values())]
    md = [f"## {args.workload}: N={N}, K={K}, {bits}-bit, {('linear', 'SwiGLU pair', 'LinearAdd')[op]}, us per launch", "",
          "| T | " + " | ".join(names) + " | fastest | public call picks |",
          "|---" * (len(names) + 3) + "|"]
    for T, r in table.items():
        extra = r[picks[T]] / r[best[T]] - 1.0
        note = f" (+{100 * extra:.0f} %)" if extra > 0.03 else ""
        md.append(f"| {T} | " + " | ".join(f"{r[n]:.2f}" if n in r else "" for n in names) +
                  f" | {best[T]} | {picks[T]}{note} |")
    print("\n".join(md), file=sys.stderr, flush=True)
    print(json.dumps({"route_sweep": args.workload, "N": N, "K": K, "bits": bits,
                      "cold_copies": copies, "us": table, "fastest": best, "picks": picks}))
    return 0


def run_probe(args) -> int:
    """Plain copy (or read) kernel over a buffer of known size: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters, and the achievable HBM read rate.  With --probe-cold the
    read kernel walks rotated copies (each launch reads a buffer that no launch has touched
    since the others went through), timed like the GEMM launches: HIP events around graph
    replays of back-to-back launches."""
    import ctypes
    import torch
    P = ctypes.CDLL(os.path.join(ROOT, "w4_groupwise_gemm_amd", "libw4probe.so"))
    P.w4probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    P.w4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    P.w4probe_read_u.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    P.w4probe_bcast.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p]
    P.w4probe_lds.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = int(args.probe_mb * 1e6) // 4096 * 4096
    dev = torch.device("cuda:0")
    grid = args.probe_grid
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    if args.probe in ("bcast", "lds"):
        sink = torch.empty(16, dtype=torch.uint8, device=dev)
        buf = torch.randint(0, 255, (max(nbytes, 16),), dtype=torch.uint8, device=dev)

        def timed(launch, n):
            for _ in range(3):
                if launch() != 0:
                    raise RuntimeError("probe launch failed")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        table = {}
        if args.probe == "bcast":
            for dma in (0, 1):
                for g_wg in (256, 512, 768, 1024):
                    us = timed(lambda: P.w4probe_bcast(buf.data_ptr(), nbytes, sink.data_ptr(), g_wg, dma, sh), 200)
                    moved = g_wg * nbytes
                    table[f"{'lds' if dma else 'vgpr'}_g{g_wg}"] = {
                        "us": us, "TBs": moved / us / 1e6, "B_per_clk_per_CU": moved / 256 / (us * 1e-6 * 2.4e9)}
                    print(f"[probe] bcast {nbytes / 1e3:.0f} KB x {g_wg} workgroups, "
                          f"{'direct-to-LDS' if dma else 'registers'}: {us:.2f} us "
                          f"{moved / us / 1e6:.1f} TB/s", file=sys.stderr, flush=True)
        else:
            iters = 2000
            for threads in (256, 512, 1024):
                for g_wg in (256, 512, 1024):
                    us = timed(lambda: P.w4probe_lds(iters, sink.data_ptr(), g_wg, threads, sh), 10)
                    moved = g_wg * threads * iters * 8 * 16
                    table[f"t{threads}_g{g_wg}"] = {
                        "us": us, "B_per_clk_per_CU": moved / 256 / (us * 1e-6 * 2.4e9)}
                    print(f"[probe] lds {threads // 64} waves x {g_wg} workgroups: {us:.1f} us "
                          f"{moved / 256 / (us * 1e-6 * 2.4e9):.1f} B/clk per compute unit",
                          file=sys.stderr, flush=True)
        print(json.dumps({"probe": args.probe, "bytes": nbytes if args.probe == "bcast" else None,
                          "clock_GHz_assumed": 2.4, "compute_units": 256, "table": table}))
        return 0
    if args.probe_cold:
        if args.probe != "read":
            raise SystemExit("--probe-cold applies to --probe read")
        copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / nbytes)))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        sink = torch.empty(16, dtype=torch.uint8, device=dev)

        def measure(g_wg, unroll):
            def launch_all():
                cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # the capture stream
                for b in bufs:
                    if P.w4probe_read_u(b.data_ptr(), nbytes, sink.data_ptr(), g_wg, unroll, cs) != 0:
                        raise RuntimeError("probe launch failed")

            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launch_all()
            stream = torch.cuda.current_stream()
            for _ in range(max(1, args.warmup)):
                g.replay()
            torch.cuda.synchronize()
            samples = []
            for _ in range(max(1, args.steps)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                samples.append(e0.elapsed_time(e1) * 1e3 / copies)
            return float(np.median(samples))

        if args.probe_sweep:
            table = {}
            for unroll in (1, 2, 4, 8):
                for g_wg in (256, 512, 1024, 2048, 4096, 8192, 16384):
                    us = measure(g_wg, unroll)
                    table[f"u{unroll}_g{g_wg}"] = us
                    print(f"[probe] {nbytes / 1e6:.1f} MB unroll={unroll} grid={g_wg}: {us:.2f} us "
                          f"{nbytes / us / 1e3:.0f} GB/s", file=sys.stderr, flush=True)
            best = min(table, key=table.get)
            print(json.dumps({"probe": "read_cold_sweep", "bytes_read": nbytes, "copies": copies,
                              "us": table, "best": best, "best_us": table[best],
                              "best_GBs": nbytes / table[best] / 1e3}))
            return 0
        us = measure(grid, args.probe_unroll)
        print(json.dumps({"probe": "read_cold", "bytes_read": nbytes, "copies": copies, "grid": grid,
                          "unroll": args.probe_unroll, "us_median": us, "GBs": nbytes / us / 1e3}))
        return 0
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes if args.probe == "copy" else 16, dtype=torch.uint8, device=dev)
    times = []
    for i in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if args.probe == "copy":
            rc = P.w4probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid, sh)
        else:
            rc = P.w4probe_read(src.data_ptr(), nbytes, dst.data_ptr(), grid, sh)
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
        if i >= args.warmup:
            times.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in times]) * 1e3)
    moved = nbytes * (2 if args.probe == "copy" else 1)
    print(json.dumps({"probe": args.probe, "bytes_read": nbytes,
                      "bytes_written": nbytes if args.probe == "copy" else 0,
                      "us_median": us, "GBs": moved / us / 1e3}))
    return 0


def _counter_per_dispatch(run_dir: str, counter: str, match: str):
    """Mean over dispatches of `counter` (rows of one dispatch summed) for kernels whose name
    contains `match`, from rocprofv3 --pmc csv output under run_dir."""
    import csv
    import glob
    per = {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    name = None
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter or match not in r["Kernel_Name"]:
                    continue
                name = r["Kernel_Name"]
                key = (f, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for a kernel matching {match!r} under {run_dir}")
    return sum(per.values()) / len(per), len(per), name


def traffic_summary(args) -> int:
    """Counter runs -> profiles/traffic_<workload>.json: HBM bytes per launch of the measured
    kernel, FETCH_SIZE and WRITE_SIZE each scaled by what that counter reads for the plain copy
    kernel of libw4probe.so over a buffer of known size."""
    if not args.kernel_match or not args.widths:
        print("--traffic-summary needs --kernel-match and --widths", file=sys.stderr)
        return 2
    d = args.traffic_summary
    fetch, nf, kname = _counter_per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE", args.kernel_match)
    write, nw, _ = _counter_per_dispatch(os.path.join(d, "write"), "WRITE_SIZE", args.kernel_match)
    cf, ncf, _ = _counter_per_dispatch(os.path.join(d, "copy_fetch"), "FETCH_SIZE", "copy_kernel")
    cw, ncw, _ = _counter_per_dispatch(os.path.join(d, "copy_write"), "WRITE_SIZE", "copy_kernel")
    copy_bytes = int(args.copy_mb * 1e6) // 4096 * 4096
    fscale, wscale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    rd, wr = fetch * 1024.0 * fscale, write * 1024.0 * wscale
    T = args.widths
    family = next((k for k in KERNEL_SOURCES if k in kname), None)
    if family is None:
        print(f"no source list for kernel {kname}", file=sys.stderr)
        return 2
    rec = {
        "workload": args.workload, "T": T, "kernel": kname,
        "kernel_sources": KERNEL_SOURCES[family],
        "kernel_src_sha": kernel_source_sha(KERNEL_SOURCES[family]),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "dispatches": {"fetch": nf, "write": nw, "copy_fetch": ncf, "copy_write": ncw},
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": fscale, "write_scale": wscale,
        "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
        "bytes_per_launch": {str(t): rd + wr for t in T.split(",")},
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def cpu_baseline(wl, widths, op, bits, lo, hi, sc, ze, wstream_alg, prefill, rows, K, gpu_out,
                 timing=True):
    """The fp64 oracle on the host cores: (1) the parity check of this run's GPU outputs on 256
    sampled output columns per width; (2) the oracle timed on a bounded sample of the same step.
    Returns (baseline record, parity record)."""
    import oracle
    parity = {}
    for T in widths:
        cols, got = gpu_out[T]
        if op == 1:
            g, u = wl.weights
            gref = oracle.linear_rows(wl.x[:T], g.lo, g.hi, g.scales, g.zeros, bits, cols)
            uref = oracle.linear_rows(wl.x[:T], u.lo, u.hi, u.scales, u.zeros, bits, cols)
            ref = oracle.silu(gref) * uref
        else:
            ref = oracle.linear_rows(wl.x[:T], lo, hi, sc, ze, bits, cols)
            if op == 2:
                ref = ref + wl.r[:T][:, cols].astype(np.float64)
        rel = oracle.rel_l2(got, ref)
        elem = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
        parity[str(T)] = {"rel_l2": rel, "max_elem": elem, "ok": bool(rel <= 2e-3 and elem <= 1e-2),
                          "sampled_columns": int(len(cols))}
    if not timing:
        return None, parity
    try:
        import threadpoolctl
        threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    host = {"cpu_model": cpu_model, "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": threads}

    # the two phases of the oracle timed apart, for one call at the widest T (the first matrix
    # of the op): unpack + dequantise, then the fp64 product
    Tw = min(max(widths), 64)
    xw = wl.x[:Tw].astype(np.float64)
    m0 = wl.weights[0] if op == 1 else None
    mlo, mhi, msc, mze = (m0.lo, m0.hi, m0.scales, m0.zeros) if op == 1 else (lo, hi, sc, ze)
    t_dq = t_mm = 0.0
    for n0 in range(0, mlo.shape[0], 2048):
        n1 = min(mlo.shape[0], n0 + 2048)
        t0 = time.perf_counter()
        q = oracle.unpack_codes(mlo[n0:n1], None if mhi is None else mhi[n0:n1], K, bits)
        wdq = oracle.dequantize(q, msc[n0:n1], mze[n0:n1])
        t1 = time.perf_counter()
        _ = xw @ wdq.T
        t2 = time.perf_counter()
        t_dq += t1 - t0
        t_mm += t2 - t1
    host["phases_one_call"] = {"T": Tw, "dequant_s": t_dq, "matmul_s": t_mm}
    if prefill:
        # one token chunk of 64 over the full weight: scaled by FLOPs
        T = 64
        t0 = time.perf_counter()
        y = oracle.linear(wl.x[:T], lo, hi, sc, ze, bits)
        if op == 2:
            y = y + wl.r[:T].astype(np.float64)
        dt = time.perf_counter() - t0
        return ({"value": 2.0 * T * rows * K / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                 "kind": "oracle", "sample": f"T={T} tokens over the full {rows}x{K} weight, "
                                              f"{dt:.1f} s", **host}, parity)
    reps, total, t_start = 0, 0.0, time.perf_counter()
    while True:
        for T in widths:
            if op == 1:
                g, u = wl.weights
                oracle.swiglu(wl.x[:T], (g.lo, g.hi, g.scales, g.zeros),
                              (u.lo, u.hi, u.scales, u.zeros), bits=bits)
            else:
                oracle.linear(wl.x[:T], lo, hi, sc, ze, bits)
        reps += 1
        total = time.perf_counter() - t_start
        if total >= 10.0 or reps >= 20:
            break
    return ({"value": reps * len(widths) * wstream_alg / total / 1e9, "unit": "GB/s",
             "cores": threads, "kind": "oracle",
             "sample": f"{reps} full steps (T in {list(widths)}), {total:.1f} s", **host}, parity)


if __name__ == "__main__":
    sys.exit(main())
