#!/usr/bin/env python3
"""Benchmark of the ternary group-scaled GEMV/GEMM library on one MI355X.

Default workload: the 8B-class decode GEMV set at M = 1 in the 2-bit-slot layout: 36 layers,
each with q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, gate 12288x4096, up 12288x4096 and
down 4096x12288 (N x K), every matrix its own buffer (1.845 GB of packed weights, far more than
the 256 MB last-level cache). One step = one pass over all 252 matrices in layer order, where
matrices that read the same input share a launch (q/k/v, gate/up): 144 launches, captured once
in a HIP graph and replayed. Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line (rank 0). `value` is achieved algorithmic GB/s for the whole pass:
packed codes + fp16 scales + fp16 activations read + fp32 outputs written, divided by the
wall time of a step (HIP events around the replays, on the stream they run on). `roofline`
reports the GEMV kernel against the 8 TB/s HBM peak: algorithmic bytes per launch over the
average launch duration (the timed region divided by the launches in it; the launches run back
to back). Its `traffic` is the HBM bytes per launch that rocprofv3 counters measured for the
same command, read from profiles/ only while the kernel sources still match the ones profiled.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload.

Other workloads (`--workload base3|gemm|rotated|flips|config1`) print lines of their own; they are
measurements for the design notes, not the headline.
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
    ap.add_argument("--workload", default="8b",
                    choices=["8b", "base3", "binary", "rotated", "gemm", "flips", "rmsnorm", "config1"])
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the set (default: 36 for the 8B-class sets, 64 for the rotated 27B-class set)")
    ap.add_argument("--mode", default="layer", choices=["layer", "fused-layer", "set"],
                    help="launch grouping for the 8B set: same-input groups (144 launches), one launch per "
                         "layer (36), or the whole set in as few launches as possible")
    ap.add_argument("--gemm-layout", default="slot2", choices=["slot2", "binary"],
                    help="code layout of the GEMM workload")
    ap.add_argument("--gemm-rot-block", type=int, default=0, choices=[0, 128, 1024],
                    help="GEMM workload with rotated weights: each product first rotates its fp16 activations "
                         "into a bf16 buffer with this block (0: plain basis)")
    ap.add_argument("--rot-block", type=int, default=128, choices=[128, 1024],
                    help="rotation block of the rotated 27B-class set (128: one block per scale group)")
    ap.add_argument("--one-mode", action="store_true", help="time only --mode (the others are reported by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a known-size kernel that calibrates "
                         "the FETCH_SIZE/WRITE_SIZE counters in a profile of this command)")
    return ap.parse_args()


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

def time_graph(torch, fn, steps, warmup):
    """Capture fn() once into a graph; replay warmup + steps times; ms per replay (event timing)."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
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


KERNEL_SOURCES = ["ternary_group_scaled_amd/csrc/gemv.hip", "ternary_group_scaled_amd/csrc/lane_ops.h",
                  "ternary_group_scaled_amd/csrc/rms_norm.h",
                  "ternary_group_scaled_amd/csrc/tgs_internal.h", "ternary_group_scaled_amd/csrc/tgs_host.cpp"]


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(profile_name):
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
    if fields.get("source_sha256") != kernel_source_sha():
        return None
    try:
        return {"fetch": float(fields["fetch_bytes_per_launch"]), "write": float(fields["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- 8B decode set

LAYOUT_NAME = {1: "slot2", 2: "base3", 3: "binary"}


def bench_8b(args, torch, tgs, synth, layout=1, p_zero=0.4, tag="8b", workload_name=None, metric=METRIC):
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

    def batched_launches(chunk):
        per = [(mats[L][nm], inputs[L][g][0], outputs[L][nm]) for L in range(layers) for g in GROUPS_8B for nm in g]
        out = []
        for i in range(0, len(per), chunk):
            part = per[i:i + chunk]
            out.append((lambda p: lambda: tgs.ternary_gemv_batched([a for a, _, _ in p], [b for _, b, _ in p],
                                                                   [c for _, _, c in p]))(part))
        return out

    modes = {"layer": [group_launch(L, g) for L in range(layers) for g in GROUPS_8B],
             "fused-layer": batched_launches(len(LAYER_8B)),
             "set": batched_launches(tgs.MAX_BATCH)}
    timings = {}
    timed_modes = [args.mode] + [m for m in ("layer", "fused-layer", "set") if m != args.mode and not args.one_mode]
    for mode in timed_modes:
        launches = modes[mode]

        def one_pass(launches=launches):
            for fn in launches:
                fn()

        log(f"[bench] timing {args.steps} graph replays of {len(launches)} launches ({mode})")
        ms_m, _graph = time_graph(torch, one_pass, args.steps, args.warmup)
        del _graph
        timings[mode] = (ms_m, len(launches))
        log(f"[bench]   {mode}: step {ms_m * 1e3:.1f} us -> {total_bytes / ms_m / 1e6:.0f} GB/s, "
            f"{ms_m * 1e3 / len(launches):.2f} us per launch")
    ms, n_launches = timings[args.mode]
    gbs = total_bytes / (ms * 1e-3) / 1e9
    per_launch_bytes = total_bytes / n_launches
    per_launch_s = ms * 1e-3 / n_launches
    kernel_gbs = per_launch_bytes / per_launch_s / 1e9
    kernel = "gemv_b3_mfma_kernel" if layout == 2 else "gemv_wave_kernel"
    profile = f"{kernel}.8b_{LAYOUT_NAME[layout]}_m1_{args.mode}.pmc.txt"
    traffic = measured_traffic(profile)

    result = {
        "metric": metric, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": workload_name or "8B-class decode GEMV set, 2-bit-slot layout, M=1",
                   "layers": layers, "matrices": layers * len(LAYER_8B), "launches_per_step": n_launches,
                   "launch_mode": args.mode, "p_zero": p_zero, "algorithmic_bytes_per_step": int(total_bytes),
                   "weight_bytes_per_step": int(w_bytes)},
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms, 1),
        "launch_modes": {m: {"launches": t[1], "ms_per_step": round(t[0], 5), "gbs": round(total_bytes / t[0] / 1e6, 1)}
                         for m, t in timings.items()},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic["fetch"] + traffic["write"]),
                     "kernel": kernel, "avg_launch_us": round(per_launch_s * 1e6, 3),
                     "bytes_per_launch_avg": int(per_launch_bytes),
                     "traffic_profile": profile if traffic is not None else None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_8b(torch, host, inputs[0], outputs[0], layout, args.cpu_seconds, ms,
                                                 total_bytes / layers, layers)
    return result


def cpu_baseline_8b(torch, host, xs, ys, layout, seconds, gpu_ms, layer_bytes, layers):
    """The fp64 oracle on the host cores over layer 0's 7 matrices, with the inputs the GPU pass
    used, repeated for ~`seconds`. Its first pass is also compared with the GPU's layer-0 outputs
    (every row, within the tolerance bound). The oracle packs layer 0's trits itself (untimed)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
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
    return {"value": round(layer_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of the set (7 matrices, {int(layer_bytes)} algorithmic bytes), {passes} passes in "
                      f"{time.time() - t0:.1f}s; full-set equivalent {1.0 / (dt * layers):.3f} steps/s",
            "gpu_speedup": round((dt * layers) / (gpu_ms * 1e-3), 1)}


# ----------------------------------------------------------------------------- other workloads

def bench_rotated(args, torch, tgs, synth):
    """27B-class rotated-basis GEMV, base-3: gate/up 17408x5120 and down 5120x17408 per layer."""
    layers = args.layers or 64
    block = args.rot_block
    shapes = [("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]
    res = []
    for m in (1, 8):
        log(f"[bench] rotated base-3 set, {layers} layers, m={m}, rotation block {block}")
        mats, xs, ys, sg = [], [], [], {}
        for k in (5120, 17408):
            sg[k] = torch.from_numpy(synth.signs(0, synth.stream_id("rot/signs", k), k)).cuda()
        for L in range(layers):
            for name, n, k in shapes:
                w, _, _ = build_matrix(torch, tgs, synth, 2, 0, f"rot/L{L}/{name}", n, k, 0.5, rotated=block)
                mats.append(w)
                ys.append(torch.empty((m, n), dtype=torch.float32, device="cuda"))
            xg = x_f16_dev(torch, synth, 0, f"rot/L{L}/in{m}", m, 5120)[0]
            xd = x_f16_dev(torch, synth, 0, f"rot/L{L}/mid{m}", m, 17408)[0]
            xs += [xg, xg, xd]
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

        ms, _ = time_graph(torch, one_pass, args.steps, args.warmup)
        log(f"[bench] rotated m={m}: step {ms * 1e3:.1f} us -> {nb / ms / 1e6:.0f} GB/s")

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

        ms2, _ = time_graph(torch, two_pass, args.steps, args.warmup)
        log(f"[bench] rotated m={m}, two passes: step {ms2 * 1e3:.1f} us -> {nb / ms2 / 1e6:.0f} GB/s")
        res.append({"metric": "rotated ternary GEMV achieved GB/s, 27B-class set", "value": round(nb / ms / 1e6, 1),
                    "unit": "GB/s", "m": m, "ms_per_step": round(ms, 4), "launches_per_step": len(launches),
                    "two_pass": {"gbs": round(nb / ms2 / 1e6, 1), "ms_per_step": round(ms2, 4),
                                 "launches_per_step": len(two)},
                    "config": {"workload": f"27B-class rotated GEMV set, base-3, {layers} layers, M={m}, "
                                           f"rotation block {block}",
                               "bytes_per_step": int(nb)}})
        del mats, xs, ys, plain, xr
        torch.cuda.empty_cache()
    return res


def bench_gemm(args, torch, tgs, synth):
    """27B-class prefill GEMM (slot-2, or binary codes): gate/up 17408x5120 and down 5120x17408, M in
    {16, 128, 2048}. With --gemm-rot-block the weights are in the rotated basis: every product first
    rotates its fp16 activations into a bf16 buffer (hadamard_rotate), then multiplies that buffer
    with a plain-basis descriptor of the same codes; the line reports both launches together and
    the rotation alone."""
    res = []
    copies = 16
    rot = args.gemm_rot_block
    layout, p_zero = (3, 0.0) if args.gemm_layout == "binary" else (1, 0.4)
    for n, k in ((17408, 5120), (5120, 17408)):
        ws = [build_matrix(torch, tgs, synth, layout, 0, f"gemm/{n}x{k}/{i}", n, k, p_zero)[0] for i in range(copies)]
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

            ms, _ = time_graph(torch, one_pass, max(2, args.steps // 4), 1)
            per = ms / copies
            flops = 2.0 * m * n * k
            nb = ws[0].nbytes + m * k * 2 + m * n * 4
            line = {"metric": "ternary GEMM TFLOP/s", "value": round(flops / per / 1e9, 2), "unit": "TFLOP/s",
                    "pct_of_bf16_peak": round(100 * flops / per / 1e9 / BF16_MFMA_PEAK_TFLOPS, 2),
                    "gbs": round(nb / per / 1e6, 1), "us": round(per * 1e3, 2),
                    "config": {"workload": f"27B-class prefill GEMM {n}x{k}, M={m}, {LAYOUT_NAME[layout]}"
                                           + (f", rotated basis ({rot}-blocks, rotation + GEMM)" if rot else "")}}
            if rot:
                def rotations():
                    for _ in range(copies):
                        rotate()

                rms, _ = time_graph(torch, rotations, max(2, args.steps // 4), 1)
                line["rotate_us"] = round(rms / copies * 1e3, 2)
            res.append(line)
            log(f"[bench] gemm {n}x{k} m={m}{' rot ' + str(rot) if rot else ''}: {per * 1e3:.1f} us, "
                f"{flops / per / 1e9:.1f} TFLOP/s" + (f" (rotation {line['rotate_us']} us)" if rot else ""))
        del ws
        torch.cuda.empty_cache()
    return res


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
                "roofline": {"bound": "hbm" if layout == 1 else "alu", "achieved": round(gbs, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "kernel": "code_flip_kernel"}}
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
    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "8b":
        out = [bench_8b(args, torch, tgs, synth)]
    elif args.workload == "base3":
        out = [bench_8b(args, torch, tgs, synth, layout=2, p_zero=0.5, tag="8b3",
                        workload_name="8B-class decode GEMV set, base-3 layout, M=1")]
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
        args.layers = 1
        out = [bench_8b(args, torch, tgs, synth)]
    for line in out:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
