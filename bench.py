#!/usr/bin/env python3
"""Benchmark of the ternary group-scaled GEMV/GEMM library on one MI355X.

Headline: the 8B-class decode GEMV set at M = 1 in the 2-bit-slot layout: 36 layers, each with
q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, gate 12288x4096, up 12288x4096 and down
4096x12288 (N x K), every matrix its own buffer (1.845 GB of packed weights, far more than the
256 MB last-level cache). One step = one pass over all 252 matrices in layer order, where
matrices that read the same input share a launch (q/k/v, gate/up): 144 launches, captured once
in a HIP graph and replayed. Inputs are seeded synthetic data already resident in HBM.

The default run prints one JSON line (rank 0): `value` is the headline's achieved algorithmic
GB/s (packed codes + fp16 scales + fp16 activations read + fp32 outputs written, over the wall
time of a step: HIP events around the replays, on the stream they run on). `roofline` reports the
GEMV kernel against the 8 TB/s HBM peak: algorithmic bytes per launch over the average launch
duration (the timed region divided by the launches in it; the launches run back to back), and
against the read bandwidth a plain streaming kernel reaches on the same device (`stream_read`,
`frac_vs_measured`). Its `traffic` is the HBM bytes per launch that rocprofv3 counters measured for
the same kernel, read from profiles/ only while the kernel sources still match the ones profiled.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload.

The same line carries the other measured configurations under `configs`, each with its own
roofline and CPU baseline: the single 256 x 1024 GEMV (latency), the base-3 8B set, the 27B-class
prefill GEMM at M in {16, 128, 2048} for both shapes, and the 27B-class rotated base-3 set at
M in {1, 8} with the rotation fused and as two passes.

`--workload` runs one workload alone (8b, gemv256, base3, gemm, rotated, binary, rmsnorm, flips,
stream) and prints its lines.
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

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "ternary GEMV achieved HBM GB/s (% of peak) + weight-tokens/s, 8B-class set, M=1"

LAYER_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288)]
# launches of one layer, in order; matrices in a group read the same activation vector
GROUPS_8B = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    choices=["all", "8b", "base3", "binary", "rotated", "gemm", "flips", "rmsnorm", "gemv256",
                             "stream"])
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the set (default: 36 for the 8B-class sets, 64 for the rotated 27B-class set)")
    ap.add_argument("--mode", default="layer", choices=["chain", "layer", "fused-layer", "set"],
                    help="launch grouping for the 8B set: the step chain in layer order (each step reads the "
                         "previous step's output; 16 steps per launch, 9 launches; slot-2 only), same-input "
                         "groups (144 launches), one launch per layer (36), or the whole set in as few launches "
                         "as possible (independent matrices: the multi-matrix upper bound)")
    ap.add_argument("--gemm-layout", default="slot2", choices=["slot2", "binary"],
                    help="code layout of the GEMM workload")
    ap.add_argument("--gemm-rot-block", type=int, default=0, choices=[0, 128, 1024],
                    help="GEMM workload with rotated weights: each product first rotates its fp16 activations "
                         "into a bf16 buffer with this block (0: plain basis)")
    ap.add_argument("--rot-block", type=int, default=128, choices=[128, 1024],
                    help="rotation block of the rotated 27B-class set (128: one block per scale group)")
    ap.add_argument("--one-mode", action="store_true", help="time only --mode (the others are reported by default)")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the eager pass before graph capture (with --warmup 0 every launch of the GEMV "
                         "kernels is then a timed replay: the command for a kernel trace of the timed region)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--stream-gib", type=int, default=0,
                    help="read a buffer of this many GiB once with the streaming-read probe first, then copy "
                         "256 MiB device to device (kernels of known traffic that calibrate the FETCH_SIZE and "
                         "WRITE_SIZE counters in a profile of this command)")
    return ap.parse_args()


def cpu_info():
    """Host CPU model (from /proc/cpuinfo) and the threads the oracle's OpenMP loops use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return model, threads


def roofline(bound, achieved, peak, unit, kernel, traffic=None, **extra):
    line = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}
    line.update(extra)
    return line


def stream_read_ceiling(torch, tgs, gib=4, launches=8):
    """Read bandwidth of the streaming-read probe over a cold buffer of `gib` GiB (16x the
    last-level cache): the best of `launches` back-to-back reads, each timed with HIP events."""
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = tgs.stream_read(buf)  # first touch
    torch.cuda.synchronize()
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(launches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        tgs.stream_read(buf, sink)
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    del buf, sink
    torch.cuda.empty_cache()
    best = min(times)
    log(f"[bench] streaming read of {gib} GiB: best {nbytes / best / 1e6:.0f} GB/s, median "
        f"{nbytes / sorted(times)[len(times) // 2] / 1e6:.0f} GB/s")
    return {"value": round(nbytes / best / 1e6, 1), "unit": "GB/s", "bytes": nbytes, "launches": launches,
            "median_gbs": round(nbytes / sorted(times)[len(times) // 2] / 1e6, 1), "kernel": "stream_read_kernel",
            "note": "plain cold read of the buffer, 16-byte non-temporal loads over the whole GPU"}


# ----------------------------------------------------------------------------- inputs

def build_matrix(torch, tgs, synth, layout, seed, tag, n, k, p_zero, rotated=False):
    """The device matrix, plus its trits and fp16 scales (the oracle packs the trits itself)."""
    t = synth.trits(seed, synth.stream_id(tag, "codes"), (n, k), p_zero)
    s = synth.scales_f16(seed, synth.stream_id(tag, "scales"), (n, k // 128))
    codes, scales = tgs.pack_ternary(layout, t, s)
    w = tgs.PackedMatrix(layout, torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda(), k,
                         rotated=rotated)
    return w, t, s


def x_f16_dev(torch, synth, seed, tag, m, k):
    x = synth.x_f16(seed, synth.stream_id(tag, "x"), (m, k))
    return torch.from_numpy(x.view(np.int16).copy()).cuda().view(torch.float16), x


# ----------------------------------------------------------------------------- timing helpers

def time_graph(torch, fn, steps, warmup, eager=True):
    """Capture fn() once into a graph; replay warmup + steps times; ms per replay (event timing)."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    if eager:
        with torch.cuda.stream(stream):
            fn()  # eager run before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(steps):
            graph.replay()
        stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, graph


_CSRC = "ternary_group_scaled_amd/csrc/"
_COMMON_SOURCES = [_CSRC + "tgs_internal.h", _CSRC + "tgs_host.cpp", _CSRC + "lane_ops.h", _CSRC + "rms_norm.h"]
# the sources each kernel's code and launch configuration come from (gemv.hip holds the GEMV plan)
KERNEL_SOURCES = {
    "gemv_s2_mfma_kernel": [_CSRC + "gemv_s2_mfma.hip", _CSRC + "s2_mfma.h", _CSRC + "gemv.hip"] + _COMMON_SOURCES,
    "gemv_chain_kernel": [_CSRC + "gemv_chain.hip", _CSRC + "s2_mfma.h"] + _COMMON_SOURCES,
    "gemv_b3_mfma_kernel": [_CSRC + "gemv_mfma.hip", _CSRC + "gemv.hip"] + _COMMON_SOURCES,
    "gemv_wave_kernel": [_CSRC + "gemv.hip"] + _COMMON_SOURCES,
    "gemm": [_CSRC + "gemm.hip"] + _COMMON_SOURCES,
}


def kernel_source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(profile_name, kernel):
    """HBM bytes per launch from a committed counter summary (profiles/<name>), or None when the
    summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != kernel_source_sha(kernel):
        return None
    try:
        out = {"fetch": float(fields["fetch_bytes_per_launch"]), "write": float(fields["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None
    try:  # the profiler's average launch duration, when the summary records it
        out["trace_avg_launch_us"] = float(fields["trace_avg_launch_us"].split()[0])
    except (KeyError, ValueError, IndexError):
        pass
    return out


# ----------------------------------------------------------------------------- 8B decode set

LAYOUT_NAME = {1: "slot2", 2: "base3", 3: "binary"}


def bench_8b(args, torch, tgs, synth, layout=1, p_zero=0.4, tag="8b", workload_name=None, metric=METRIC,
             ceiling=None):
    layers = args.layers or 36
    log(f"[bench] building {layers} layers x {len(LAYER_8B)} matrices ({LAYOUT_NAME[layout]})")
    t0 = time.time()
    mats, host = [], []
    for L in range(layers):
        d = {}
        for name, n, k in LAYER_8B:
            w, trits, scales = build_matrix(torch, tgs, synth, layout, 0, f"{tag}/L{L}/{name}", n, k, p_zero)
            d[name] = w
            if L == 0:
                host.append((name, trits, scales, n, k))
        mats.append(d)
    inputs, outputs = [], []
    for L in range(layers):
        xs = {}
        for grp in GROUPS_8B:
            k = mats[L][grp[0]].k
            xs[grp] = x_f16_dev(torch, synth, 0, f"{tag}/L{L}/{grp[0]}", 1, k)
        inputs.append(xs)
        outputs.append({name: torch.empty((1, n), dtype=torch.float32, device="cuda") for name, n, _ in LAYER_8B})
    torch.cuda.synchronize()
    log(f"[bench] built in {time.time() - t0:.1f}s")

    w_bytes = sum(mats[L][name].nbytes for L in range(layers) for name, _, _ in LAYER_8B)
    x_bytes = sum(inputs[L][g][0].numel() * 2 for L in range(layers) for g in GROUPS_8B)
    y_bytes = sum(outputs[L][name].numel() * 4 for L in range(layers) for name, _, _ in LAYER_8B)
    total_bytes = w_bytes + x_bytes + y_bytes

    # launch lists for one pass, per launch mode
    def group_launch(L, grp):
        ws = [mats[L][nm] for nm in grp]
        xs = [inputs[L][grp][0]] * len(grp)
        ys = [outputs[L][nm] for nm in grp]
        return lambda: tgs.ternary_gemv_batched(ws, xs, ys)

    # kernel launches of one batched call: the library launches once per distinct kernel shape among
    # its matrices (for slot-2 and binary, once per distinct K; every base-3 matrix of a call shares one)
    def kernels_of(ws):
        return 1 if layout == 2 else len({w.k for w in ws})

    def batched_launches(chunk):
        per = [(mats[L][nm], inputs[L][g][0], outputs[L][nm]) for L in range(layers) for g in GROUPS_8B for nm in g]
        out, kernels = [], 0
        for i in range(0, len(per), chunk):
            part = per[i:i + chunk]
            kernels += kernels_of([a for a, _, _ in part])
            out.append((lambda p: lambda: tgs.ternary_gemv_batched([a for a, _, _ in p], [b for _, b, _ in p],
                                                                   [c for _, _, c in p]))(part))
        return out, kernels

    fused, fused_kernels = batched_launches(len(LAYER_8B))
    whole, whole_kernels = batched_launches(tgs.MAX_BATCH)
    modes = {"layer": [group_launch(L, g) for L in range(layers) for g in GROUPS_8B],
             "fused-layer": fused, "set": whole}
    kernels = {"layer": layers * len(GROUPS_8B), "fused-layer": fused_kernels, "set": whole_kernels}
    all_modes = ["layer", "fused-layer", "set"]
    chain = None
    if layout == 1:
        chain = chain_steps_8b(torch, tgs, synth, mats, inputs, outputs, layers)
        wsp = tgs.chain_workspace()
        modes["chain"] = [(lambda part: lambda: tgs.ternary_gemv_chain(part, wsp))(chain[i:i + tgs.CHAIN_MAX_STEPS])
                          for i in range(0, len(chain), tgs.CHAIN_MAX_STEPS)]
        kernels["chain"] = len(modes["chain"])
        all_modes = ["chain"] + all_modes
    mode = args.mode if args.mode in modes else "layer"
    timings = {}
    timed_modes = [mode] + [m for m in all_modes if m != mode and not args.one_mode]
    for timed in timed_modes:  # (not `mode`: that stays the headline's launch mode)
        launches = modes[timed]

        def one_pass(launches=launches):
            for fn in launches:
                fn()

        log(f"[bench] timing {args.steps} graph replays of {len(launches)} launches ({timed})")
        ms_m, _graph = time_graph(torch, one_pass, args.steps, args.warmup, eager=not args.no_eager)
        del _graph
        timings[timed] = (ms_m, kernels[timed], len(launches))
        log(f"[bench]   {timed}: step {ms_m * 1e3:.1f} us -> {total_bytes / ms_m / 1e6:.0f} GB/s, "
            f"{ms_m * 1e3 / kernels[timed]:.2f} us per kernel launch ({kernels[timed]} launches, {len(launches)} calls)")
    ms, n_launches, n_calls = timings[mode]
    gbs = total_bytes / (ms * 1e-3) / 1e9
    per_launch_bytes = total_bytes / n_launches
    per_launch_s = ms * 1e-3 / n_launches
    kernel_gbs = per_launch_bytes / per_launch_s / 1e9
    kernel = {1: "gemv_s2_mfma_kernel", 2: "gemv_b3_mfma_kernel", 3: "gemv_wave_kernel"}[layout]
    if mode == "chain":
        kernel = "gemv_chain_kernel"
    profile = f"{kernel}.8b_{LAYOUT_NAME[layout]}_m1_{mode}.pmc.txt"
    traffic = measured_traffic(profile, kernel)
    extra = {"avg_launch_us": round(per_launch_s * 1e6, 3), "bytes_per_launch_avg": int(per_launch_bytes),
             "traffic_profile": profile if traffic is not None else None,
             "duration": "timed region / launches (HIP events on the replay stream; back-to-back launches)"}
    if traffic is not None and "trace_avg_launch_us" in traffic:
        # the kernel-side figure: the same kernel sources under rocprofv3 --kernel-trace (each dispatch
        # signals the profiler, so traced launches run somewhat longer than untraced ones)
        extra["trace_avg_launch_us"] = traffic["trace_avg_launch_us"]
        extra["trace_gbs"] = round(per_launch_bytes / (traffic["trace_avg_launch_us"] * 1e-6) / 1e9, 1)
    if ceiling:
        extra["measured_read_ceiling_gbs"] = ceiling["value"]
        extra["frac_vs_measured"] = round(kernel_gbs / ceiling["value"], 4)

    result = {
        "metric": metric, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": workload_name or "8B-class decode GEMV set, 2-bit-slot layout, M=1",
                   "layers": layers, "matrices": layers * len(LAYER_8B), "launches_per_step": n_launches,
                   "calls_per_step": n_calls,
                   "launch_mode": mode, "p_zero": p_zero, "algorithmic_bytes_per_step": int(total_bytes),
                   "weight_bytes_per_step": int(w_bytes)},
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms, 1),
        "launch_modes": {m: {"launches": t[1], "calls": t[2], "ms_per_step": round(t[0], 5),
                             "gbs": round(total_bytes / t[0] / 1e6, 1)} for m, t in timings.items()},
        "roofline": roofline("hbm", kernel_gbs, HBM_PEAK_GBS, "GB/s", kernel,
                             None if traffic is None else int(traffic["fetch"] + traffic["write"]), **extra),
    }
    if not args.no_cpu_baseline:
        for fn in modes["layer"][:len(GROUPS_8B)]:  # layer 0 on its own inputs, for the oracle comparison
            fn()
        result["cpu_baseline"] = cpu_baseline_8b(torch, host, inputs[0], outputs[0], layout, args.cpu_seconds, ms,
                                                 total_bytes / layers, layers)
        if "chain" in timings:  # the chain's layer-0 steps against the oracle, on the chain's own outputs
            result["cpu_baseline"]["chain_parity_max_err_over_bound"] = chain_parity_check(
                tgs, torch, chain, wsp, host_chain_of(host, chain))
    return result


def chain_steps_8b(torch, tgs, synth, mats, inputs, outputs, layers):
    """The 144 steps of a pass in layer order, each reading the output of the step before it: q/k/v
    the RMS-normalised layer input (layer 0: the external fp16 input; later layers: the output of
    the previous layer's down projection), o the output of q, gate/up the RMS-normalised output of o,
    down the output of gate. Norm weights bf16 1 + N(0, 0.25^2), eps 1e-6."""
    def gamma(tag):
        g = synth.bf16_bits(1.0 + 0.25 * synth.normal(0, synth.stream_id("chain8b", tag), (4096,)))
        return torch.from_numpy(g.view(np.int16).copy()).cuda()

    g_in, g_post = gamma("input_norm"), gamma("post_norm")
    flat = lambda L, nm: outputs[L][nm].view(-1)
    steps = []
    for L in range(layers):
        x_in = inputs[0][("q", "k", "v")][0].view(-1) if L == 0 else flat(L - 1, "down")
        steps.append({"ws": [mats[L][nm] for nm in ("q", "k", "v")], "x": x_in,
                      "ys": [flat(L, nm) for nm in ("q", "k", "v")], "gamma": g_in, "eps": 1e-6})
        steps.append({"ws": [mats[L]["o"]], "x": flat(L, "q"), "ys": [flat(L, "o")]})
        steps.append({"ws": [mats[L]["gate"], mats[L]["up"]], "x": flat(L, "o"),
                      "ys": [flat(L, "gate"), flat(L, "up")], "gamma": g_post, "eps": 1e-6})
        steps.append({"ws": [mats[L]["down"]], "x": flat(L, "gate"), "ys": [flat(L, "down")]})
    return steps


def host_chain_of(host, chain):
    """Layer 0's oracle inputs for the chain check: for each of its 4 steps, (codes, scales, k) of
    each matrix, packed by the oracle from the trits."""
    import oracle
    by_name = {name: (oracle.pack(1, trits), scales, k) for name, trits, scales, n, k in host}
    names = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    return [[by_name[nm] for nm in grp] for grp in names]


def chain_parity_check(tgs, torch, chain, wsp, host_steps, rows_per_matrix=64):
    """Run the chain once more and check layer 0's four steps against the oracle on sampled rows of
    every matrix, each from the fp16 rounding of the input the GPU actually read (for o, gate/up and
    down: the GPU's output of the step before)."""
    import oracle
    for i in range(0, len(chain), tgs.CHAIN_MAX_STEPS):
        tgs.ternary_gemv_chain(chain[i:i + tgs.CHAIN_MAX_STEPS], wsp)
    torch.cuda.synchronize()
    if int(wsp[-1].item()) != 0:
        raise SystemExit("chain: a wait between steps gave up (error word set)")
    worst = 0.0
    for i, grp in enumerate(host_steps):
        st = chain[i]
        x16 = st["x"].float().cpu().numpy().reshape(1, -1).astype(np.float16)
        gbits = st["gamma"].cpu().numpy().view(np.uint16) if "gamma" in st else None
        for (codes, scales, k), w, y in zip(grp, st["ws"], st["ys"]):
            rows = np.unique(np.linspace(0, w.n - 1, rows_per_matrix).astype(np.int64))
            y_ref, bound = oracle.matmul(1, codes, scales, k, x16.view(np.uint16), oracle.X_F16, rows=rows,
                                         gamma=gbits, eps=st.get("eps", 0.0))
            ratio = float((np.abs(y.cpu().numpy()[rows].astype(np.float64) - y_ref[0]) / bound[0]).max())
            if not ratio <= 1.0:
                raise SystemExit(f"chain step {i}: parity check failed (max err/bound {ratio:.3g})")
            worst = max(worst, ratio)
    log(f"[bench] chain: layer-0 steps against the oracle ok on sampled rows (max err/bound {worst:.3g})")
    return round(worst, 6)


def cpu_baseline_8b(torch, host, xs, ys, layout, seconds, gpu_ms, layer_bytes, layers):
    """The fp64 oracle on the host cores over layer 0's 7 matrices, with the inputs the GPU pass
    used, repeated for ~`seconds`. Its first pass is also compared with the GPU's layer-0 outputs
    (every row, within the tolerance bound). The oracle packs layer 0's trits itself (untimed)."""
    import oracle
    model, threads = cpu_info()
    host = [(name, oracle.pack(layout, trits), scales, n, k) for name, trits, scales, n, k in host]
    torch.cuda.synchronize()
    y_gpu = {name: ys[name].cpu().numpy().astype(np.float64) for name, _, _, _, _ in host}
    x_of = {name: xs[[g for g in GROUPS_8B if name in g][0]][1] for name, _, _, _, _ in host}
    worst = 0.0
    t0 = time.time()
    passes = 0
    while True:
        for name, codes, scales, n, k in host:
            y_ref, bound = oracle.matmul(layout, codes, scales, k, x_of[name].view(np.uint16), oracle.X_F16)
            if passes == 0:
                ratio = float((np.abs(y_gpu[name] - y_ref) / bound).max())
                if not ratio <= 1.0:  # NaN fails too
                    raise SystemExit(f"parity check failed for layer 0 {name}: max err/bound {ratio:.3g}")
                worst = max(worst, ratio)
        passes += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / passes
    log(f"[bench] layer-0 parity against the oracle ok (max err/bound {worst:.3g})")
    layer_gbs = layer_bytes / dt / 1e9
    return {"value": round(layer_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu": model,
            "sample": f"layer 0 of the set (7 matrices, {int(layer_bytes)} algorithmic bytes), {passes} passes in "
                      f"{time.time() - t0:.1f}s; full-set equivalent {1.0 / (dt * layers):.3f} steps/s",
            "gpu_speedup": round((dt * layers) / (gpu_ms * 1e-3), 1)}


# ----------------------------------------------------------------------------- single GEMV (latency)

def bench_gemv256(args, torch, tgs, synth):
    """The single ternary GEMV of 256 outputs x 1024 inputs, M = 1, codes P(0) = 0.4, scales
    |N(0, 0.02)| + 1e-4, fp16 N(0, 1) activations, seed 0, 2-bit-slot layout: the pack/unpack round
    trip, and the time of one call in a stream of back-to-back calls (72,704 bytes fit the cache, so
    this is a latency figure). The CPU-baseline leg also checks the packing and every output against
    the oracle."""
    n, k = 256, 1024
    t = synth.trits(0, synth.stream_id("gemv256x1024", "codes"), (n, k), 0.4)
    s = synth.scales_f16(0, synth.stream_id("gemv256x1024", "scales"), (n, k // 128))
    codes, scales = tgs.pack_ternary(1, t, s)
    back, _ = tgs.unpack_ternary(1, codes, scales, k)
    if not (back == t).all():
        raise SystemExit("256x1024 GEMV: pack/unpack round trip failed")
    w = tgs.PackedMatrix(1, torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda(), k)
    x16 = synth.x_f16(0, synth.stream_id("gemv256x1024", "x"), (1, k))
    x = torch.from_numpy(x16.view(np.int16).copy()).cuda().view(torch.float16)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    calls = 200

    def run():
        for _ in range(calls):
            tgs.ternary_gemv(w, x, y=y)

    ms, _ = time_graph(torch, run, max(3, args.steps // 4), 1, eager=not args.no_eager)
    us = ms * 1e3 / calls
    nbytes = codes.nbytes + scales.nbytes + 2 * k + 4 * n
    log(f"[bench] single 256x1024 GEMV: {us:.2f} us per call")
    line = {"metric": "single ternary GEMV latency, 256x1024, 2-bit-slot, M=1", "value": round(us, 3), "unit": "us",
            "higher_is_better": False, "calls_per_replay": calls, "round_trip": "pack/unpack bit-exact",
            "config": {"workload": "single GEMV, N=256 x K=1024, groups of 128 along K, M=1, codes P(0)=0.4, "
                                   "seed 0", "algorithmic_bytes": int(nbytes)},
            "roofline": roofline("hbm", nbytes / us / 1e3, HBM_PEAK_GBS, "GB/s", "gemv_s2_mfma_kernel",
                                 note="72,704 bytes fit the cache: one launch's latency bounds the call, not HBM")}
    if not args.no_cpu_baseline:
        import oracle
        ref_codes = oracle.pack(1, t)
        if not (codes == ref_codes).all():
            raise SystemExit("256x1024 GEMV: packing differs from the oracle's")
        y_ref, bound = oracle.matmul(1, ref_codes, s, k, x16.view(np.uint16), oracle.X_F16)
        ratio = float((np.abs(y.cpu().numpy().astype(np.float64) - y_ref) / bound).max())
        if not ratio <= 1.0:
            raise SystemExit(f"256x1024 GEMV: parity check failed (max err/bound {ratio:.3g})")
        log(f"[bench] 256x1024 GEMV: packing and every output match the oracle (max err/bound {ratio:.3g})")
        line["cpu_baseline"] = cpu_baseline_gemv256(ref_codes, s, x16, k, us)
        line["cpu_baseline"]["parity_max_err_over_bound"] = ratio
    return line


_CONFIG1_ORACLE_SCRIPT = """
import sys, time
import numpy as np
sys.path.insert(0, {root!r})
import oracle, synth
n, k = 256, 1024
t = synth.trits(0, synth.stream_id("gemv256x1024", "codes"), (n, k), 0.4)
s = synth.scales_f16(0, synth.stream_id("gemv256x1024", "scales"), (n, k // 128))
x = synth.x_f16(0, synth.stream_id("gemv256x1024", "x"), (1, k)).view(np.uint16)
codes = oracle.pack(1, t)
oracle.matmul(1, codes, s, k, x, oracle.X_F16)
t0, calls = time.time(), 0
while time.time() - t0 < {seconds}:
    oracle.matmul(1, codes, s, k, x, oracle.X_F16)
    calls += 1
print((time.time() - t0) / calls * 1e6)
"""


def cpu_baseline_gemv256(codes, s, x16, k, gpu_us, seconds=2.0):
    """The oracle on the whole config-1 GEMV, on all host threads and (in a child process with
    OMP_NUM_THREADS=1) on one."""
    import subprocess

    import oracle
    model, threads = cpu_info()
    xb = x16.view(np.uint16)
    oracle.matmul(1, codes, s, k, xb, oracle.X_F16)
    t0, calls = time.time(), 0
    while time.time() - t0 < seconds:
        oracle.matmul(1, codes, s, k, xb, oracle.X_F16)
        calls += 1
    us = (time.time() - t0) / calls * 1e6
    single = None
    try:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        out = subprocess.run([sys.executable, "-c", _CONFIG1_ORACLE_SCRIPT.format(root=ROOT, seconds=seconds)],
                             env=env, capture_output=True, text=True, timeout=120)
        single = round(float(out.stdout.strip().splitlines()[-1]), 2)
    except (subprocess.SubprocessError, ValueError, IndexError):
        single = None
    return {"value": round(us, 2), "unit": "us", "cores": threads, "kind": "oracle", "cpu": model,
            "single_thread_us": single,
            "sample": f"the whole config-1 GEMV, {calls} calls in {seconds:.0f}s on {threads} threads; one thread "
                      f"in a child process",
            "gpu_speedup": round(us / gpu_us, 1)}


# ----------------------------------------------------------------------------- other workloads

def bench_rotated(args, torch, tgs, synth):
    """27B-class rotated-basis GEMV, base-3: gate/up 17408x5120 and down 5120x17408 per layer, 64
    layers (3.69 GB), M in {1, 8}. Fused: the rotation runs inside the GEMV (two launches per layer,
    gate/up sharing their input and signs). Two passes: hadamard_rotate of each input once (fp16),
    then the plain-basis GEMV on descriptors of the same code buffers. The CPU-baseline leg
    checks layer 0's gate and down outputs against the oracle on sampled rows."""
    layers = args.layers or 64
    block = args.rot_block
    shapes = [("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]
    res = []
    for m in (1, 8):
        log(f"[bench] rotated base-3 set, {layers} layers, m={m}, rotation block {block}")
        mats, xs, ys, sg, host = [], [], [], {}, {}
        for k in (5120, 17408):
            sg[k] = torch.from_numpy(synth.signs(0, synth.stream_id("rot/signs", k), k)).cuda()
        for L in range(layers):
            for name, n, k in shapes:
                w, t, s = build_matrix(torch, tgs, synth, 2, 0, f"rot/L{L}/{name}", n, k, 0.5, rotated=block)
                mats.append(w)
                ys.append(torch.empty((m, n), dtype=torch.float32, device="cuda"))
                if L == 0 and name in ("gate", "down"):
                    host[name] = (t, s, n, k)
            xg, xg16 = x_f16_dev(torch, synth, 0, f"rot/L{L}/in{m}", m, 5120)
            xd, xd16 = x_f16_dev(torch, synth, 0, f"rot/L{L}/mid{m}", m, 17408)
            xs += [xg, xg, xd]
            if L == 0:
                host["gate"] += (xg16,)
                host["down"] += (xd16,)
        nb = sum(w.nbytes for w in mats) + sum(x.numel() * 2 for x in xs[::3]) + sum(
            x.numel() * 2 for x in xs[2::3]) + sum(y.numel() * 4 for y in ys)
        launches = []
        for L in range(layers):
            i = 3 * L
            launches.append((lambda a, b, c, s: lambda: tgs.ternary_gemv_batched(a, b, c, signs=s))(
                mats[i:i + 2], xs[i:i + 2], ys[i:i + 2], [sg[5120]] * 2))
            launches.append((lambda a, b, c, s: lambda: tgs.ternary_gemv_batched(a, b, c, signs=s))(
                mats[i + 2:i + 3], xs[i + 2:i + 3], ys[i + 2:i + 3], [sg[17408]]))

        def one_pass():
            for fn in launches:
                fn()

        ms, _ = time_graph(torch, one_pass, args.steps, args.warmup, eager=not args.no_eager)
        log(f"[bench] rotated m={m}: step {ms * 1e3:.1f} us -> {nb / ms / 1e6:.0f} GB/s")
        y_gate, y_down = ys[0].cpu().numpy(), ys[2].cpu().numpy()

        # the same products in two passes: hadamard_rotate of each input once (fp16 out), then the
        # plain-basis GEMV on descriptors of the same code buffers (the rotation is not repeated by
        # every workgroup that reads a group)
        plain = [tgs.PackedMatrix(2, w.codes, w.scales, w.k, rotated=0) for w in mats]
        xr = [torch.empty_like(x) for x in xs]
        two = []
        for L in range(layers):
            i = 3 * L
            two.append((lambda a, b, s, bl: lambda: tgs.hadamard_rotate(a, s, block=bl, y=b))(xs[i], xr[i], sg[5120],
                                                                                              block))
            two.append((lambda a, b, c: lambda: tgs.ternary_gemv_batched(a, b, c))(plain[i:i + 2], [xr[i]] * 2,
                                                                                  ys[i:i + 2]))
            two.append((lambda a, b, s, bl: lambda: tgs.hadamard_rotate(a, s, block=bl, y=b))(xs[i + 2], xr[i + 2],
                                                                                              sg[17408], block))
            two.append((lambda a, b, c: lambda: tgs.ternary_gemv_batched(a, b, c))(plain[i + 2:i + 3], [xr[i + 2]],
                                                                                  ys[i + 2:i + 3]))

        def two_pass():
            for fn in two:
                fn()

        ms2, _ = time_graph(torch, two_pass, args.steps, args.warmup, eager=not args.no_eager)
        log(f"[bench] rotated m={m}, two passes: step {ms2 * 1e3:.1f} us -> {nb / ms2 / 1e6:.0f} GB/s")
        gbs = nb / ms / 1e6
        line = {"metric": "rotated ternary GEMV achieved GB/s, 27B-class set", "value": round(gbs, 1),
                "unit": "GB/s", "m": m, "ms_per_step": round(ms, 4), "launches_per_step": len(launches),
                "tokens_per_s": round(m * 1e3 / ms, 1), "dtype": "f16",
                "two_pass": {"gbs": round(nb / ms2 / 1e6, 1), "ms_per_step": round(ms2, 4),
                             "launches_per_step": len(two)},
                "config": {"workload": f"27B-class rotated GEMV set, base-3, {layers} layers, M={m}, "
                                       f"rotation block {block}",
                           "bytes_per_step": int(nb)},
                "roofline": roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "gemv_b3_mfma_kernel",
                                     avg_launch_us=round(ms * 1e3 / len(launches), 2),
                                     note="fused path; the two-pass schedule is reported beside it")}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_rotated(host, {"gate": y_gate, "down": y_down}, sg, block, m,
                                                        gbs)
        res.append(line)
        del mats, xs, ys, plain, xr
        torch.cuda.empty_cache()
    return res


def cpu_baseline_rotated(host, y_gpu, sg, block, m, gpu_gbs, seconds=2.0):
    """The oracle on sampled rows of layer 0's gate (K = 5120) and down (K = 17408) projections with
    the rotation, repeated for about `seconds`; the GPU's outputs at those rows are checked against it."""
    import oracle
    model, threads = cpu_info()
    jobs = []
    for name in ("gate", "down"):
        t, s, n, k, x16 = host[name]
        rows = np.unique(np.linspace(0, n - 1, 256).astype(np.int64))
        codes = oracle.pack(2, t)
        signs = sg[k].cpu().numpy()
        y_ref, bound = oracle.matmul(2, codes, s, k, x16.view(np.uint16), oracle.X_F16, signs=signs, rows=rows,
                                     block=block)
        ratio = float((np.abs(y_gpu[name][:, rows].astype(np.float64) - y_ref) / bound).max())
        if not ratio <= 1.0:
            raise SystemExit(f"rotated {name} m={m}: parity check failed on sampled rows (max err/bound {ratio:.3g})")
        nbytes = rows.size * (oracle.row_bytes(2, k) + k // 64) + m * k * 2 + m * rows.size * 4
        jobs.append((codes, s, k, x16, signs, rows, nbytes))
    t0, passes = time.time(), 0
    while True:
        for codes, s, k, x16, signs, rows, _ in jobs:
            oracle.matmul(2, codes, s, k, x16.view(np.uint16), oracle.X_F16, signs=signs, rows=rows, block=block)
        passes += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / passes
    nbytes = sum(j[6] for j in jobs)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu": model,
            "sample": f"256 sampled rows each of layer 0's gate and down projections, M={m}, rotation included, "
                      f"{passes} passes in {time.time() - t0:.1f}s; the GPU's outputs at those rows within the bound",
            "gpu_speedup": round(gpu_gbs / (nbytes / dt / 1e9), 1)}


def bench_gemm(args, torch, tgs, synth):
    """27B-class prefill GEMM (slot-2, or binary codes): gate/up 17408x5120 and down 5120x17408, M in
    {16, 128, 2048}. 16 distinct weight copies per shape (379 MB, beyond the last-level cache) run
    back to back. With --gemm-rot-block the weights are in the rotated basis: every product first
    rotates its fp16 activations into a bf16 buffer (hadamard_rotate), then multiplies that buffer
    with a plain-basis descriptor of the same codes; the line reports both launches together and
    the rotation alone. The CPU-baseline leg checks each point against the oracle on sampled output
    rows."""
    res = []
    copies = 16
    rot = args.gemm_rot_block
    layout, p_zero = (3, 0.0) if args.gemm_layout == "binary" else (1, 0.4)
    for n, k in ((17408, 5120), (5120, 17408)):
        w0, t0, s0 = build_matrix(torch, tgs, synth, layout, 0, f"gemm/{n}x{k}/0", n, k, p_zero)
        ws = [w0] + [build_matrix(torch, tgs, synth, layout, 0, f"gemm/{n}x{k}/{i}", n, k, p_zero)[0]
                     for i in range(1, copies)]
        ref_codes = None
        for m in (16, 128, 2048):
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            if rot:
                x16 = synth.x_f16(0, synth.stream_id("gemm/x16", m, k), (m, k))
                xh = torch.from_numpy(x16.view(np.int16).copy()).cuda().view(torch.float16)
                sg = torch.from_numpy(synth.signs(0, synth.stream_id("gemm/signs", k), k)).cuda()
                x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
                rotate = lambda: tgs.hadamard_rotate(xh, sg, block=rot, y=x)
                launches = [(lambda w: lambda: (rotate(), tgs.ternary_gemm(w, x, y)))(w) for w in ws]
            else:
                xb = synth.x_bf16_bits(0, synth.stream_id("gemm/x", m, k), (m, k))
                x = torch.from_numpy(xb.view(np.int16).copy()).cuda().view(torch.bfloat16)
                launches = [(lambda w: lambda: tgs.ternary_gemm(w, x, y))(w) for w in ws]

            def one_pass():
                for fn in launches:
                    fn()

            ms, _ = time_graph(torch, one_pass, max(2, args.steps // 4), 1, eager=not args.no_eager)
            per = ms / copies
            flops = 2.0 * m * n * k
            nb = ws[0].nbytes + m * k * 2 + m * n * 4
            tflops = flops / per / 1e9
            gbs = nb / per / 1e6
            bound = "hbm" if m <= 16 else "mfma"
            if bound == "hbm":
                rl = roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "gemm_skinny_kernel", avg_launch_us=round(per * 1e3, 2),
                              note="about 114 flop per byte at M=16, below the bf16 ridge of about 312")
            else:
                rl = roofline("mfma", tflops, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s", "gemm_tile_kernel",
                              avg_launch_us=round(per * 1e3, 2), dtype_peak="bf16 dense MFMA")
            line = {"metric": "ternary GEMM TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
                    "pct_of_bf16_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
                    "gbs": round(gbs, 1), "us": round(per * 1e3, 2), "dtype": "bf16",
                    "config": {"workload": f"27B-class prefill GEMM {n}x{k}, M={m}, {LAYOUT_NAME[layout]}"
                                           + (f", rotated basis ({rot}-blocks, rotation + GEMM)" if rot else ""),
                               "weight_copies": copies, "flops_per_launch": int(flops), "bytes_per_launch": int(nb)},
                    "roofline": rl}
            if rot:
                def rotations():
                    for _ in range(copies):
                        rotate()

                rms, _ = time_graph(torch, rotations, max(2, args.steps // 4), 1, eager=not args.no_eager)
                line["rotate_us"] = round(rms / copies * 1e3, 2)
            elif not args.no_cpu_baseline:
                if ref_codes is None:
                    import oracle
                    ref_codes = oracle.pack(layout, t0)
                # the last replay wrote y with copy 15; recompute copy 0's product for the parity sample
                tgs.ternary_gemm(ws[0], x, y)
                torch.cuda.synchronize()
                line["cpu_baseline"] = cpu_baseline_gemm(layout, ref_codes, s0, k, xb, y.cpu().numpy(), m, n, tflops)
            res.append(line)
            log(f"[bench] gemm {n}x{k} m={m}{' rot ' + str(rot) if rot else ''}: {per * 1e3:.1f} us, "
                f"{tflops:.1f} TFLOP/s" + (f" (rotation {line['rotate_us']} us)" if rot else ""))
        del ws, t0
        torch.cuda.empty_cache()
    return res


def cpu_baseline_gemm(layout, codes, s, k, xb, y_gpu, m, n, gpu_tflops, seconds=1.0):
    """The oracle on a sample of output rows (first, last and evenly spaced ones), repeated for about
    `seconds`; the GPU's outputs at those rows are checked against it."""
    import oracle
    model, threads = cpu_info()
    count = max(2, min(n, int(4e8 / (m * k))))
    rows = np.unique(np.linspace(0, n - 1, count).astype(np.int64))
    y_ref, bound = oracle.matmul(layout, codes, s, k, xb.view(np.uint16), oracle.X_BF16, rows=rows)
    ratio = float((np.abs(y_gpu[:, rows].astype(np.float64) - y_ref) / bound).max())
    if not ratio <= 1.0:
        raise SystemExit(f"gemm {n}x{k} m={m}: parity check failed on sampled rows (max err/bound {ratio:.3g})")
    t0, calls = time.time(), 0
    while True:
        oracle.matmul(layout, codes, s, k, xb.view(np.uint16), oracle.X_BF16, rows=rows)
        calls += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / calls
    tflops = 2.0 * m * k * rows.size / dt / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu": model,
            "sample": f"{rows.size} of {n} output rows at M={m}, {calls} passes in {time.time() - t0:.1f}s; "
                      f"the GPU's outputs at those rows within the bound (max err/bound {ratio:.3g})",
            "gpu_speedup": round(gpu_tflops / tflops, 1)}


def bench_rmsnorm(args, torch, tgs, synth):
    """The RMSNorm prologue on the launches that read a normalised input in an 8B-class layer
    (q/k/v after the input norm, gate/up after the post-attention norm), 36 layers, M = 1, for
    slot-2 and base-3 codes: the same launches timed with and without the fused norm."""
    layers = args.layers or 36
    res = []
    for layout, p_zero, name in ((1, 0.4, "slot2"), (2, 0.5, "base3")):
        log(f"[bench] rmsnorm prologue, {name}, {layers} layers")
        groups = [("q", "k", "v"), ("gate", "up")]
        shapes = {nm: (n, k) for nm, n, k in LAYER_8B}
        plain, normed = [], []
        nbytes = 0
        keep = []
        for L in range(layers):
            for grp in groups:
                k = shapes[grp[0]][1]
                ws = [build_matrix(torch, tgs, synth, layout, 0, f"nrm/{name}/L{L}/{nm}", shapes[nm][0], k, p_zero)[0]
                      for nm in grp]
                x = (x_f16_dev(torch, synth, 0, f"nrm/L{L}/{grp[0]}", 1, k)[0].float() * 5.0).half()
                g = torch.from_numpy(synth.bf16_bits(1.0 + 0.25 * synth.normal(0, synth.stream_id("nrm/g", L, grp[0]),
                                                                               (k,))).view(np.int16)).cuda()
                ys = [torch.empty((1, shapes[nm][0]), dtype=torch.float32, device="cuda") for nm in grp]
                keep.append((ws, x, g, ys))
                nbytes += sum(w.nbytes for w in ws) + 2 * k + 2 * k + sum(y.numel() * 4 for y in ys)
                plain.append((lambda a, b, c: lambda: tgs.ternary_gemv_batched(a, b, c))(ws, [x] * len(ws), ys))
                normed.append((lambda a, b, gg, c: lambda: tgs.ternary_gemv_rmsnorm_batched(a, b, gg, 1e-6, c))(
                    ws, [x] * len(ws), [g] * len(ws), ys))
        times = {}
        for label, launches in (("plain", plain), ("rmsnorm", normed)):
            def one_pass(launches=launches):
                for fn in launches:
                    fn()
            ms, _ = time_graph(torch, one_pass, args.steps, args.warmup)
            times[label] = ms
            log(f"[bench] {name} {label}: step {ms * 1e3:.1f} us, {ms * 1e3 / len(launches):.2f} us per launch, "
                f"{nbytes / ms / 1e6:.0f} GB/s")
        res.append({"metric": "GEMV with fused RMSNorm prologue, achieved GB/s, 8B-class q/k/v + gate/up launches, M=1",
                    "value": round(nbytes / times["rmsnorm"] / 1e6, 1), "unit": "GB/s",
                    "ms_per_step": round(times["rmsnorm"], 5), "ms_per_step_without_norm": round(times["plain"], 5),
                    "norm_overhead_pct": round(100 * (times["rmsnorm"] / times["plain"] - 1), 1),
                    "launches_per_step": len(normed),
                    "config": {"workload": f"8B-class q/k/v and gate/up launches with the RMSNorm prologue, {name}, "
                                           f"{layers} layers, M=1", "bytes_per_step": int(nbytes)}})
        del keep, plain, normed
        torch.cuda.empty_cache()
    return res


def bench_flips(args, torch, tgs, synth):
    """Code flips between two checkpoints of the 8B-class set (every matrix of 36 layers), one line
    per layout: the second checkpoint is the first with 0.7% of its codes changed (the rate the
    fine-tuning page reports for its best run). Up to 32 pairs per launch."""
    res = []
    layers = args.layers or 36
    for layout, p_zero, lname in ((1, 0.4, "2-bit-slot"), (2, 0.5, "base-3")):
        t0 = time.time()
        pairs, host0, planted = [], [], 0
        for L in range(layers):
            for nm, n, k in LAYER_8B:
                tag = f"flips{layout}/L{L}/{nm}"
                t = synth.trits(0, synth.stream_id(tag, "codes"), (n, k), p_zero)
                # positions to change: nonzero draws of a second stream, P = 0.007; each moves to
                # the next trit value, so every drawn position is a flip
                sel = synth.trits(0, synth.stream_id(tag, "flips"), (n, k), 0.993) != 0
                u = np.where(sel, ((t.astype(np.int16) + 2) % 3 - 1).astype(np.int8), t)
                planted += int(sel.sum())
                s = synth.scales_f16(0, synth.stream_id(tag, "scales"), (n, k // 128))
                ca, sc = tgs.pack_ternary(layout, t, s)
                cb, _ = tgs.pack_ternary(layout, u, s)
                sd = torch.from_numpy(sc.view(np.int16)).cuda()
                a = tgs.PackedMatrix(layout, torch.from_numpy(ca).cuda(), sd, k)
                b = tgs.PackedMatrix(layout, torch.from_numpy(cb).cuda(), sd, k)
                pairs.append((a, b))
                if L == 0:
                    host0.append((nm, t, u, k))
        totals = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in pairs]
        rows = [torch.empty(a.n, dtype=torch.int32, device="cuda") for a, _ in pairs]
        torch.cuda.synchronize()
        log(f"[bench] flips ({lname}): built {len(pairs)} pairs in {time.time() - t0:.1f}s")
        launches = []
        for i in range(0, len(pairs), tgs.MAX_BATCH):
            sl = slice(i, i + tgs.MAX_BATCH)
            launches.append((lambda p, t, r: lambda: tgs.ternary_code_flips_batched(p, t, r))(pairs[sl], totals[sl],
                                                                                          rows[sl]))

        def one_pass():
            for fn in launches:
                fn()

        ms, _graph = time_graph(torch, one_pass, args.steps, args.warmup)
        del _graph
        counted = sum(int(t.item()) for t in totals)
        if counted != planted:
            raise SystemExit(f"code flips: counted {counted}, planted {planted}")
        code_bytes = sum(a.codes.numel() + b.codes.numel() for a, b in pairs)
        out_bytes = sum(r.numel() * 4 for r in rows)
        gbs = (code_bytes + out_bytes) / (ms * 1e-3) / 1e9
        log(f"[bench] flips ({lname}): step {ms * 1e3:.1f} us -> {gbs:.0f} GB/s, {counted} flips "
            f"({100.0 * counted / sum(a.n * a.k for a, _ in pairs):.3f}% of codes)")
        line = {"metric": "ternary code flips between two checkpoints, achieved HBM GB/s", "value": round(gbs, 1),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
                "higher_is_better": True, "dtype": "u8", "data": "synthetic",
                "config": {"workload": f"8B-class set, two checkpoints, {lname} layout, 0.7% of codes changed",
                           "layers": layers, "pairs": len(pairs), "launches_per_step": len(launches),
                           "bytes_per_step": int(code_bytes + out_bytes), "flips": counted},
                "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "roofline": roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "code_flip_kernel")}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_flips(torch, host0, rows[:len(host0)], layout, args.cpu_seconds,
                                                      ms, len(pairs))
        res.append(line)
        del pairs, totals, rows, launches
        torch.cuda.empty_cache()
    return res


def cpu_baseline_flips(torch, host0, rows0, layout, seconds, gpu_ms, n_pairs):
    """The oracle's code-flip count over layer 0's 7 pairs, repeated for ~`seconds`; its first pass
    is also compared with the GPU's per-row counts of those pairs. The oracle packs the two
    checkpoints' trits itself (untimed)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    host0 = [(nm, oracle.pack(layout, t), oracle.pack(layout, u), k) for nm, t, u, k in host0]
    gpu_rows = [r.cpu().numpy().astype(np.int64) for r in rows0]
    t0 = time.time()
    passes, nbytes = 0, sum(ca.nbytes + cb.nbytes for _, ca, cb, _ in host0)
    while True:
        for i, (nm, ca, cb, k) in enumerate(host0):
            _, ref_rows = oracle.code_flips(layout, ca, cb, k)
            if passes == 0 and not (ref_rows == gpu_rows[i]).all():
                raise SystemExit(f"code flips of layer 0 {nm} differ from the oracle")
        passes += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / passes
    log("[bench] layer-0 code flips equal the oracle's")
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of the set (7 pairs, {nbytes} code bytes), {passes} passes in {time.time() - t0:.1f}s",
            "gpu_speedup": round((dt * n_pairs / len(host0)) / (gpu_ms * 1e-3), 1)}


def nested(line):
    """A workload's line as an entry of the combined line (without the run-wide fields)."""
    return {k: v for k, v in line.items() if k not in ("n_gpus", "steps", "warmup", "scaling", "vs_baseline", "data")}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library's hot path is a single-GPU "
                                   "kernel set; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import synth
    import ternary_group_scaled_amd as tgs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.stream_gib:
        buf = torch.empty(args.stream_gib << 30, dtype=torch.uint8, device="cuda")
        tgs.stream_read(buf)
        # a 256 MiB device-to-device copy: known writes (and reads) for the WRITE_SIZE counter
        dst = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst.copy_(buf[:256 << 20])
        torch.cuda.synchronize()
        del buf, dst
    if args.workload == "all":
        t_start = time.time()
        ceiling = stream_read_ceiling(torch, tgs)
        head = bench_8b(args, torch, tgs, synth, ceiling=ceiling)
        torch.cuda.empty_cache()
        configs = {"gemv_256x1024": nested(bench_gemv256(args, torch, tgs, synth))}
        saved = args.cpu_seconds
        args.cpu_seconds = min(saved, 5.0)
        configs["base3_8b_set"] = nested(bench_8b(
            args, torch, tgs, synth, layout=2, p_zero=0.5, tag="8b3",
            workload_name="8B-class decode GEMV set, base-3 layout, M=1",
            metric="base-3 ternary GEMV achieved HBM GB/s (% of peak), 8B-class set, M=1", ceiling=ceiling))
        args.cpu_seconds = saved
        torch.cuda.empty_cache()
        configs["gemm_27b"] = [nested(x) for x in bench_gemm(args, torch, tgs, synth)]
        configs["rotated_base3_27b_set"] = [nested(x) for x in bench_rotated(args, torch, tgs, synth)]
        head["stream_read"] = ceiling
        head["configs"] = configs
        head["wall_s"] = round(time.time() - t_start, 1)
        out = [head]
    elif args.workload == "8b":
        out = [bench_8b(args, torch, tgs, synth)]
    elif args.workload == "gemv256":
        out = [bench_gemv256(args, torch, tgs, synth)]
    elif args.workload == "base3":
        out = [bench_8b(args, torch, tgs, synth, layout=2, p_zero=0.5, tag="8b3",
                        workload_name="8B-class decode GEMV set, base-3 layout, M=1",
                        metric="base-3 ternary GEMV achieved HBM GB/s (% of peak), 8B-class set, M=1")]
    elif args.workload == "binary":
        out = [bench_8b(args, torch, tgs, synth, layout=3, p_zero=0.0, tag="8bb",
                        workload_name="8B-class decode GEMV set, binary layout (t in {-1, +1}), M=1",
                        metric="binary GEMV achieved HBM GB/s (% of peak), 8B-class set, M=1")]
    elif args.workload == "rotated":
        out = bench_rotated(args, torch, tgs, synth)
    elif args.workload == "gemm":
        out = bench_gemm(args, torch, tgs, synth)
    elif args.workload == "flips":
        out = bench_flips(args, torch, tgs, synth)
    elif args.workload == "rmsnorm":
        out = bench_rmsnorm(args, torch, tgs, synth)
    else:
        out = [stream_read_ceiling(torch, tgs)]
    for line in out:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
