#!/usr/bin/env python3
"""Benchmark: the quantized nn.Linear(3072 -> 4096) hot path at M=32 on one MI355X.

One step = one pass of the whole hot path over one batch X[32, 3072] (bf16):
the four weight-only dequant-GEMMs (INT4 group-128, FP8 per-row, NVFP4, MXFP4;
each y = x . deq(W)^T + b, bf16 out) and the static-FP8 Linear (activation Q to
E4M3, then the FP8 GEMM).  Weights stay packed in HBM in the library's kernel
tile order (layout 1, made once by wq_repack; the canonical rows layout is
timed beside it per format); every launch reads a
different copy of the packed weight + scales (copies per format total
>= 512 MiB, twice the 256 MB Infinity Cache), so the weight stream is cold.  X
and bias stay warm (they are the previous layer's output).

Timed region (one pair of device synchronizations): the K-step graph, then,
for each single kernel of the step, a graph of K back-to-back launches of it
alone, then a graph of K launches of a plain read-only stream of each format's
weight bytes over the same kind of cold rotation (the achievable ceiling), and
each format's kernel on one hot copy.  HIP events on the replay stream
separate the parts; a kernel's figure is its graph time / K.

Metric: effective weight-stream bandwidth = (packed weight + scale bytes) /
time.  `value` is the step's effective bytes / ms_per_step.  `roofline` is for
the slowest single kernel: algorithmic bytes (weights, scales, X, bias, Y) per
launch / its average duration.  `traffic` comes from the committed
FETCH_SIZE / WRITE_SIZE counter profile when the kernel sources still hash to
the value recorded there, else null.

Also: `python bench.py --trace-summary DIR --out FILE` and
`python bench.py --counters-summary FETCH_DIR WRITE_DIR --out FILE` turn
rocprofv3 output directories of this script into the text summaries kept
under profiles/.
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight-stream TB/s (+% HBM peak), 3072→4096 Linear, M=32, per format"
HBM_PEAK_GBS = 8000.0
M, N, K = 32, 4096, 3072
FORMATS = ["int4", "fp8", "nvfp4", "mxfp4"]
STEP = FORMATS + ["static_fp8"]                      # the step: static_fp8 = act Q + FP8 GEMM
KERNELS = FORMATS + ["static_q", "static_gemm"]      # single kernels of the step
COLD_BYTES = 512 << 20
STREAM_POOL = 768 << 20
CSRC = os.path.join(ROOT, "weight_only_bit_dequant_amd", "csrc")
COUNTERS_PROFILE = os.path.join(ROOT, "profiles", "linear_m32_hbm_counters.md")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the M sweep (MXFP4 M=1..4096, static FP8 M=4096)")
    p.add_argument("--trace-summary", metavar="DIR", help="summarize a rocprofv3 --kernel-trace directory")
    p.add_argument("--pmc-summary", metavar="DIR", help="summarize a rocprofv3 --pmc directory (mean per kernel)")
    p.add_argument("--counters-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarize two rocprofv3 --pmc directories (FETCH_SIZE, WRITE_SIZE)")
    p.add_argument("--sweep-only", action="store_true", help="only the M sweep (e.g. for counter runs at large M)")
    p.add_argument("--no-hot", action="store_true", help="skip the hot (one copy) graphs, e.g. for counter runs")
    p.add_argument("--out", help="file for the summary (default: stdout)")
    p.add_argument("--title", default="", help="first line of the summary")
    p.add_argument("--cmd", default="", help="the command that produced the rocprofv3 output (recorded)")
    return p.parse_args()


# ------------------------------------------------------------------ byte counts


def layout(fmt):
    from weight_only_bit_dequant_amd import wq

    return wq.wq_layout("fp8" if fmt in ("static_fp8", "static_gemm") else fmt, N, K)


def effective_bytes(name):
    """Metric numerator: packed weight + scale bytes one launch streams."""
    if name == "static_q":
        return 0
    _, pb, sb, gb = layout(name)
    if name in ("static_fp8", "static_gemm"):
        return pb + sb + 4  # + the activation scale
    return pb + sb + gb


def algorithmic_bytes(name):
    """Bytes a launch must move at minimum: weight stream + activations + bias + Y."""
    xb, yb = M * K * 2, M * N * 2
    if name == "static_q":
        return xb + M * K + 4              # bf16 X in, E4M3 X out, act_scale
    if name == "static_gemm":
        return effective_bytes(name) + M * K + yb
    if name == "static_fp8":
        return effective_bytes(name) + xb + yb  # the E4M3 copy of X stays in L2
    return effective_bytes(name) + xb + N * 2 + yb


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")) +
                    glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic():
    """Per-kernel HBM bytes per launch from the committed counter profile, if
    it was taken on the current kernel sources; else {}."""
    try:
        text = open(COUNTERS_PROFILE).read()
    except OSError:
        return {}
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text, re.S)
    if not m:
        return {}
    rec = json.loads(m.group(1))
    if rec.get("src_sha256") != kernel_source_hash():
        return {}
    return rec.get("bytes_per_launch", {})


# ------------------------------------------------------------------ CPU oracle baseline


def cpu_baseline(seconds_per_format=3.0):
    """The CPU oracle on the step's work (dequantize + fp64 GEMM + bias per
    weight-only format; E4M3 act Q + fp64 DQ-GEMM for static FP8) on the full
    4096x3072 layer at M=32, with all host threads and with one."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import gemm as G
    from oracle import quant as Q
    from oracle import static_fp8 as S
    from weight_only_bit_dequant_amd import synth

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    cases = {}
    quant_s = {}
    for name in STEP:
        info = synth.WORKLOADS[name]
        W, b, X = synth.linear_case(N, K, M, cfg=info["cfg"], bias=info["bias"])
        t0 = time.perf_counter()
        if name == "static_fp8":
            wq_, ws_ = Q.quantize_fp8_row(W)
            cal = [synth.activations(M, K, synth.SEED_CAL + 100 + i) for i in range(10)]
            s = S.scale_from_amax(max(S.absmax(c) for c in cal))
            cases[name] = lambda X=X, s=s, wq_=wq_, ws_=ws_: S.static_linear_fp64(S.quantize_act(X, s), s, wq_, ws_)
        else:
            codes, scales, g = Q.quantize(name, W)
            cases[name] = lambda n=name, c=codes, sc=scales, g=g, X=X, b=b: G.linear_fp64(X, Q.dequant(n, c, sc, g), b)
        quant_s[name] = round(time.perf_counter() - t0, 3)

    def timed(fn, budget, min_reps):
        reps = []
        t_all = time.perf_counter()
        while len(reps) < min_reps or time.perf_counter() - t_all < budget:
            t0 = time.perf_counter()
            fn()
            reps.append(time.perf_counter() - t0)
        return float(np.median(reps))

    per, per1 = {}, {}
    for name, fn in cases.items():
        per[name] = timed(fn, seconds_per_format, 3)
        with threadpool_limits(1):
            per1[name] = timed(fn, 0.0, 1)
    eff = sum(effective_bytes(n) for n in STEP)
    return {
        "value": eff / sum(per.values()) / 1e12,
        "unit": "TB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "one full step on the host: the full 4096x3072 layer at M=32 for each of INT4, FP8, NVFP4, "
                  "MXFP4 (dequantize + fp64 GEMM + bias) and static FP8 (E4M3 act Q + fp64 DQ-GEMM), median of "
                  ">=3 runs (~3 s) per format; step effective weight bytes / summed oracle time",
        "seconds_per_format": {k: round(v, 4) for k, v in per.items()},
        "single_thread": {"cores": 1, "value": eff / sum(per1.values()) / 1e12,
                          "seconds_per_format": {k: round(v, 4) for k, v in per1.items()}},
        "oracle_quantize_seconds": quant_s,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------ GPU timing


LAYOUT = 1  # the packed weights' layout in the step: kernel tile order


def m_sweep(layers, dev, capture, reps_small=200, reps_large=30):
    """The other workload points, reported beside the M=32 line: MXFP4 at
    M in {1, 32, 256, 4096}, the static-FP8 layer at M=4096 and the MXFP4
    dynamic-activation path (MX act Q + E2M1 x E2M1 GEMM) at M in {32, 256,
    4096}, each timed as a graph of back-to-back launches over the same cold
    weight copies.  Large M is bound by the matrix cores: FLOP/s against the
    dense bf16 (MXFP4 weight-only), FP8 (static) or FP4 (MX dynamic) peak."""
    import torch

    from weight_only_bit_dequant_amd import synth, wq

    res = {}
    peak = {"mxfp4": 2500.0, "static_fp8": 5000.0, "mxfp4_dynamic": 10100.0}  # dense TFLOP/s (bf16 / fp8 / fp4)
    for fmt, Ms in (("mxfp4", (1, 32, 256, 4096)), ("static_fp8", (32, 4096)), ("mxfp4_dynamic", (32, 256, 4096))):
        lay = layers["mxfp4" if fmt == "mxfp4_dynamic" else fmt]  # the same cold weight copies
        for Mv in Ms:
            base = "mxfp4" if fmt == "mxfp4_dynamic" else fmt
            X = synth.as_torch_bf16(synth.activations(Mv, K, synth.SEED_X + synth.WORKLOADS[base]["cfg"]), dev)
            Y = torch.empty((Mv, N), dtype=torch.bfloat16, device=dev)
            if fmt == "static_fp8":
                ws = torch.zeros(max(1, wq.wq_fp8_static_workspace(Mv, N, K)), dtype=torch.uint8, device=dev)
            elif fmt == "mxfp4_dynamic":
                ws = torch.zeros(max(1, wq.wq_mxfp4_dynamic_workspace(Mv, K)), dtype=torch.uint8, device=dev)
            else:
                ws = torch.zeros(max(1, wq.wq_linear_workspace("mxfp4", Mv, N, K)), dtype=torch.uint8, device=dev)

            def run(first, count, lay=lay, X=X, Y=Y, ws=ws, fmt=fmt):
                for i in range(first, first + count):
                    r = lay["reps"][i % len(lay["reps"])]
                    if fmt == "static_fp8":
                        wq.wq_fp8_static_linear(X, lay["act_scale"], r["packed"], r["scales"], None, Y, ws, LAYOUT)
                    elif fmt == "mxfp4_dynamic":
                        wq.wq_mxfp4_dynamic_linear(X, r["packed"], r["scales"], lay["bias"], N, Y, ws, LAYOUT)
                    else:
                        wq.wq_linear("mxfp4", X, r["packed"], r["scales"], None, lay["bias"], N, Y, ws, LAYOUT)

            reps = reps_small if Mv <= 256 else reps_large
            # accuracy against the same layer in bf16 (outside the timed replays)
            run(0, 1)
            ref = wq.linear(X, wq.dense(lay["W"]), None if fmt == "static_fp8" else lay["bias"])
            torch.cuda.synchronize()
            sq = sqnr_db(ref, Y)
            del ref
            g = capture(run, reps)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            flop = 2.0 * Mv * N * K
            eff = effective_bytes(base)
            res[f"{fmt}_M{Mv}"] = {
                "us_per_launch": round(us, 3),
                "TFLOPs": round(flop / (us * 1e-6) / 1e12, 2),
                "pct_mfma_peak": round(100.0 * flop / (us * 1e-6) / 1e12 / peak[fmt], 2),
                "effective_TBps": round(eff / (us * 1e-6) / 1e12, 4),
                "launches": 1 if fmt == "mxfp4" else 2,
                "sqnr_db_vs_bf16": sq,
            }
            del g
    res.update(mlp2_timing(dev, capture, reps_small))
    return res


def sqnr_db(ref, y):
    """10 log10(sum ref^2 / sum (ref - y)^2) of two bf16 device tensors, in fp64."""
    r = ref.double().cpu()
    e = r - y.double().cpu()
    den = float((e * e).sum())
    return round(10.0 * math.log10(float((r * r).sum()) / den), 2) if den > 0 else float("inf")


def mlp2_timing(dev, capture, reps):
    """The static page's model (32 x 256 -> 512 -> 128, no bias) as one fused
    kernel and as two unfused static layers (four launches); weights warm."""
    import torch

    from weight_only_bit_dequant_amd import synth, wq

    W1, W2 = (synth.as_torch_bf16(w, dev) for w in synth.mlp_weights())
    cal = [synth.as_torch_bf16(b, dev) for b in synth.calibration_batches(32, 256)]
    s1, _ = wq.calibrate_act_scale(cal)
    s2, _ = wq.calibrate_act_scale([wq.linear(x, wq.dense(W1)) for x in cal])
    q1, q2 = wq.quantize("fp8", W1), wq.quantize("fp8", W2)
    X = synth.as_torch_bf16(synth.activations(32, 256, synth.SEED_X + 5), dev)
    Y = torch.empty((32, 128), dtype=torch.bfloat16, device=dev)

    def fused(first, count):
        for _ in range(count):
            wq.wq_fp8_static_mlp2(X, s1, q1["codes"], q1["scales"], None, s2, q2["codes"], q2["scales"], None, Y)

    H = torch.empty((32, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(1, wq.wq_fp8_static_workspace(32, 512, 256), wq.wq_fp8_static_workspace(32, 128, 512)),
                     dtype=torch.uint8, device=dev)

    def unfused(first, count):
        for _ in range(count):
            wq.wq_fp8_static_linear(X, s1, q1["codes"], q1["scales"], None, H, ws)
            wq.wq_fp8_static_linear(H, s2, q2["codes"], q2["scales"], None, Y, ws)

    out = {}
    # accuracy of the quantized model against the same model in bf16 (the
    # page reports SQNR in dB): the fused kernel's output against two dense
    # bf16 Linears (bf16 hidden layer), on the same input
    fused(0, 1)
    Yf = wq.linear(wq.linear(X, wq.dense(W1)), wq.dense(W2))
    torch.cuda.synchronize()
    out["static_mlp2_sqnr_db_vs_bf16"] = sqnr_db(Yf, Y)
    for name, fn, launches in (("static_mlp2_fused_M32", fused, 1), ("static_mlp2_unfused_M32", unfused, 4)):
        g = capture(fn, reps)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out[name] = {"us_per_call": round(a.elapsed_time(b) * 1e3 / reps, 3), "launches": launches}
        del g
    return out


def main_bench(args):
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch

    from weight_only_bit_dequant_amd import synth, wq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Kst = args.steps

    # ---------------- data: seeded synthetic layer per format, quantized on the GPU
    layers = {}
    for fmt in (["mxfp4", "static_fp8"] if args.sweep_only else STEP):
        info = synth.WORKLOADS[fmt]
        W, b, X = synth.linear_case(N, K, M, cfg=info["cfg"], bias=info["bias"])
        qfmt = "fp8" if fmt == "static_fp8" else fmt
        q0 = wq.quantize(qfmt, synth.as_torch_bf16(W, dev))
        q = wq.repack(q0, LAYOUT)
        eff = effective_bytes(fmt)
        copies = max(2, -(-COLD_BYTES // eff))
        reps = [{"packed": q["packed"], "scales": q["scales"], "global": q["global"]}]
        for _ in range(copies - 1):
            reps.append({"packed": q["packed"].clone(), "scales": q["scales"].clone(),
                         "global": None if q["global"] is None else q["global"].clone()})
        # the same weights in the canonical rows layout (the comparison graphs)
        rows = [{"packed": q0["packed"], "scales": q0["scales"], "global": q0["global"]}]
        for _ in range(copies - 1):
            rows.append({"packed": q0["packed"].clone(), "scales": q0["scales"].clone(),
                         "global": None if q0["global"] is None else q0["global"].clone()})
        lay = {"reps": reps, "rows": rows, "X": synth.as_torch_bf16(X, dev), "W": synth.as_torch_bf16(W, dev),
               "bias": synth.as_torch_bf16(b, dev) if b is not None else None,
               "Y": torch.empty((M, N), dtype=torch.bfloat16, device=dev), "fmt": qfmt}
        if fmt == "static_fp8":
            cal = [synth.as_torch_bf16(synth.activations(M, K, synth.SEED_CAL + 100 + i), dev) for i in range(10)]
            lay["act_scale"], _ = wq.calibrate_act_scale(cal)
            lay["Xq"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
        layers[fmt] = lay
    if args.sweep_only:
        def capture_only(fn, count):
            g = torch.cuda.CUDAGraph()
            fn(0, 1)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                fn(1, count)
            torch.cuda.synchronize()
            return g
        print(json.dumps({"m_sweep": m_sweep(layers, dev, capture_only, reps_small=20, reps_large=5)}))
        return
    ws_bytes = max([wq.wq_linear_workspace(f, M, N, K) for f in FORMATS] + [wq.wq_fp8_static_workspace(M, N, K)])
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream_pool = torch.empty(STREAM_POOL, dtype=torch.uint8, device=dev)
    sink = torch.zeros(wq.wq_read_stream_words(STREAM_POOL), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def launch(name, i, hot=False, rows=False):
        lay = layers["static_fp8" if name.startswith("static") else name]
        pool = lay["rows"] if rows else lay["reps"]
        lo = 0 if rows else LAYOUT
        r = pool[0 if hot else i % len(pool)]
        if name == "static_fp8":
            wq.wq_fp8_static_linear(lay["X"], lay["act_scale"], r["packed"], r["scales"], lay["bias"], lay["Y"], ws,
                                    lo)
        elif name == "static_q":
            wq.wq_fp8_quantize_act(lay["X"], lay["act_scale"], lay["Xq"])
        elif name == "static_gemm":
            wq.wq_fp8_linear(lay["Xq"], lay["act_scale"], r["packed"], r["scales"], lay["bias"], lay["Y"], ws, lo)
        else:
            wq.wq_linear(lay["fmt"], lay["X"], r["packed"], r["scales"], r["global"], lay["bias"], N, lay["Y"], ws, lo)

    def stream_launch(fmt, i):
        size = -(-effective_bytes(fmt) // 256) * 256
        slots = STREAM_POOL // size
        off = (i % slots) * size
        wq.wq_read_stream(stream_pool[off:off + size], sink, effective_bytes(fmt) // 16 * 16)

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0, 1)  # eager run on the capture stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn(1, count)
        torch.cuda.synchronize()
        return g

    def steps_fn(first, count):
        for st in range(first, first + count):
            for f in STEP:
                launch(f, st)

    # ---------------- graphs: the step, each single kernel, the stream ceiling, the hot case
    parts = [("step", capture(steps_fn, Kst))]
    for k in KERNELS:
        parts.append((k, capture(lambda a, c, k=k: [launch(k, i) for i in range(a, a + c)], Kst)))
    for f in STEP:
        parts.append(("stream_" + f, capture(lambda a, c, f=f: [stream_launch(f, i) for i in range(a, a + c)], Kst)))
    for f in ([] if args.no_hot else FORMATS):
        parts.append(("hot_" + f, capture(lambda a, c, f=f: [launch(f, i, hot=True) for i in range(a, a + c)], Kst)))
    for k in ([] if args.no_hot else FORMATS + ["static_gemm"]):
        parts.append(("rows_" + k, capture(lambda a, c, k=k: [launch(k, i, rows=True) for i in range(a, a + c)], Kst)))
    g_warm = capture(steps_fn, max(1, args.warmup))
    g_warm.replay()
    for _, g in parts[1:]:
        g.replay()
    torch.cuda.synchronize()

    # ---------------- timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ev[0].record()
    for i, (_, g) in enumerate(parts):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    us = {name: ev[i].elapsed_time(ev[i + 1]) * 1e3 / Kst for i, (name, _) in enumerate(parts)}
    ms_per_step = us["step"] / 1e3
    step_eff = sum(effective_bytes(f) for f in STEP)
    value = step_eff / (ms_per_step * 1e-3) / 1e12

    traffic = committed_traffic()
    per_kernel = {}
    for k in KERNELS:
        eff, alg = effective_bytes(k), algorithmic_bytes(k)
        d = {"us_per_launch": round(us[k], 3), "algorithmic_bytes": alg,
             "algorithmic_GBps": round(alg / (us[k] * 1e-6) / 1e9, 1)}
        if eff:
            d.update({"effective_bytes": eff, "effective_TBps": round(eff / (us[k] * 1e-6) / 1e12, 4),
                      "pct_hbm_peak": round(100.0 * eff / (us[k] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)})
        if k in FORMATS:
            d["copies"] = len(layers[k]["reps"])
            if "hot_" + k in us:
                d["hot_us_per_launch"] = round(us["hot_" + k], 3)
        if "rows_" + k in us:
            d["rows_layout_us_per_launch"] = round(us["rows_" + k], 3)
        if k == "static_gemm":
            d["copies"] = len(layers["static_fp8"]["reps"])
        if k in traffic:
            d["traffic_bytes"] = traffic[k]
        per_kernel[k] = d
    per_format = {}
    for f in STEP:
        eff = effective_bytes(f)
        if f == "static_fp8":
            t = us["static_q"] + us["static_gemm"]
        else:
            t = us[f]
        per_format[f] = {
            "us_per_launch": round(t, 3),
            "effective_TBps": round(eff / (t * 1e-6) / 1e12, 4),
            "pct_hbm_peak": round(100.0 * eff / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "stream_ceiling_us": round(us["stream_" + f], 3),
            "pct_of_stream_ceiling": round(100.0 * us["stream_" + f] / t, 1),
            "launches": 2 if f == "static_fp8" else 1,
        }

    dominant = max(KERNELS, key=lambda k: us[k])
    d = per_kernel[dominant]
    achieved = d["algorithmic_bytes"] / (us[dominant] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic.get(dominant), "kernel": dominant,
                "algorithmic_bytes_per_launch": d["algorithmic_bytes"], "us_per_launch": d["us_per_launch"]}

    sweep = None if args.no_sweep else m_sweep(layers, dev, capture)

    # accuracy against the unquantized layer: each step kernel's M=32 output
    # against the same layer in bf16 (dense bf16 weight, the library's bf16
    # Linear), outside the timed region
    sqnr = {}
    for name in STEP:
        lay = layers[name]
        launch(name, 0, hot=True)
        ref = wq.linear(lay["X"], wq.dense(lay["W"]), lay["bias"])
        torch.cuda.synchronize()
        sqnr[name] = sqnr_db(ref, lay["Y"])

    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": Kst,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "nn.Linear(3072->4096) bf16+bias, M=32: INT4-g128 / FP8-row / NVFP4 / MXFP4 "
                               "weight-only dequant-GEMMs + static-FP8 (act Q + FP8 GEMM), cold weight copies",
                   "M": M, "N": N, "K": K, "formats": STEP, "cold": True,
                   "weight_layout": "kernel tile order (layout 1)" if LAYOUT == 1 else "rows (layout 0)"},
        "roofline": roofline,
        "per_format": per_format,
        "per_kernel": per_kernel,
        "sqnr_db_vs_bf16": sqnr,
        "kernel_source_sha256": kernel_source_hash(),
        "wall_s_timed": round(t_wall, 4),
    }
    if sweep is not None:
        out["m_sweep"] = sweep
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


# ------------------------------------------------------------------ rocprofv3 summaries

KERNEL_LABELS = {1: "int4", 2: "fp8", 3: "nvfp4", 4: "mxfp4", 5: "static_gemm"}


def label_of(name):
    """Step label of a kernel name in an M=32 run (`--no-sweep`), else None;
    small-M kernels reading the rows layout (the comparison graphs) get a
    "rows_" prefix."""
    m = re.search(r"k_linear<(\d+), [^>]*?, (\d+)>", name)
    if m:
        lab = KERNEL_LABELS.get(int(m.group(1)))
        return lab if lab is None or int(m.group(2)) == LAYOUT else "rows_" + lab
    if "k_quant_act" in name:
        return "static_q"
    if "k_read_stream" in name:
        return "stream"
    return None


def _rows(d, suffix):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _short(name, n=90):
    return name if len(name) <= n else name[:n]


def trace_summary(d, cmd):
    import numpy as np

    rows = _rows(d, "kernel_trace.csv")
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | calls | avg µs | p10 | p50 | p90 | min | max |", "|---|---|---|---|---|---|---|---|"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        a = np.asarray(v)
        lines.append("| `%s` | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f |" % (
            _short(name), len(a), a.mean(), np.percentile(a, 10), np.percentile(a, 50), np.percentile(a, 90),
            a.min(), a.max()))
    return "Command (from /tmp with TMPDIR=/tmp, repo at $R):\n\n```\n%s\n```\n\n%s\n" % (cmd, "\n".join(lines))


def counters_summary(fetch_dir, write_dir, cmd):
    import numpy as np

    out = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            out.setdefault((r["Kernel_Name"], cname), []).append(float(r["Counter_Value"]))
    # calibration: the FP8 pack is a plain 16-byte copy of N*K bytes
    copy_bytes = N * K
    cal = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        v = [x for (n, c), xs in out.items() if c == cname and "k_copy16" in n for x in xs]
        if not v:
            raise SystemExit("no k_copy16 dispatch for %s calibration" % cname)
        cal[cname] = copy_bytes / (float(np.mean(v)) * 1024.0)
    per = {}
    lines = ["| kernel | label | counter | dispatches | mean KiB / dispatch | scaled bytes / dispatch |",
             "|---|---|---|---|---|---|"]
    for (name, cname), xs in sorted(out.items()):
        kib = float(np.mean(xs))
        scaled = kib * 1024.0 * cal[cname]
        lab = label_of(name)
        lines.append("| `%s` | %s | %s | %d | %.1f | %.0f |" % (_short(name, 70), lab or "", cname, len(xs), kib, scaled))
        if lab and lab != "stream" and not lab.startswith("rows_"):
            per.setdefault(lab, 0.0)
            per[lab] += scaled
    rec = {"src_sha256": kernel_source_hash(), "calibration": {k: round(v, 4) for k, v in cal.items()},
           "bytes_per_launch": {k: int(round(v)) for k, v in per.items()}}
    text = ("Commands (each counter in its own run; from /tmp with TMPDIR=/tmp, repo at $R):\n\n```\n%s\n```\n\n"
            "Calibration: `k_copy16` (the FP8 pack, a plain 16-byte copy of N*K = %d bytes) reads and writes %d "
            "bytes; FETCH_SIZE x %.4f and WRITE_SIZE x %.4f give bytes.  Per-launch HBM traffic (FETCH + WRITE, "
            "scaled): %s.\n\n%s\n\n<!-- traffic %s -->\n" % (
                cmd, copy_bytes, copy_bytes, cal["FETCH_SIZE"], cal["WRITE_SIZE"],
                ", ".join("%s %d B" % kv for kv in sorted(rec["bytes_per_launch"].items())), "\n".join(lines),
                json.dumps(rec)))
    return text


def pmc_summary(d, cmd):
    """Mean of every collected counter per kernel name."""
    import numpy as np

    vals = {}
    for r in _rows(d, "counter_collection.csv"):
        vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    lines = ["| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k, v in sorted(vals.items()):
        n = max(len(x) for x in v.values())
        lines.append("| `%s` | %d | %s |" % (_short(k), n, " | ".join(
            "%.2f" % float(np.mean(v[c])) if c in v else "" for c in names)))
    return "Command (from /tmp with TMPDIR=/tmp, repo at $R):\n\n```\n%s\n```\n\n%s\n" % (cmd, "\n".join(lines))


def main():
    args = parse()
    if args.trace_summary or args.counters_summary or args.pmc_summary:
        if args.trace_summary:
            text = trace_summary(args.trace_summary, args.cmd)
        elif args.pmc_summary:
            text = pmc_summary(args.pmc_summary, args.cmd)
        else:
            text = counters_summary(args.counters_summary[0], args.counters_summary[1], args.cmd)
        if args.title:
            text = "# %s\n\n%s" % (args.title, text)
        if args.out:
            with open(args.out, "w") as fh:
                fh.write(text)
        else:
            print(text)
        return
    main_bench(args)


if __name__ == "__main__":
    main()
