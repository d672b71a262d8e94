#!/usr/bin/env python3
"""Benchmark: the quantized nn.Linear(3072 -> 4096) hot path at M=32 on one MI355X.

One step = one pass of the whole hot path over one batch X[32, 3072] (bf16):
the four weight-only dequant-GEMMs (INT4 group-128, FP8 per-row, NVFP4, MXFP4;
each y = x . deq(W)^T + b, bf16 out) and the static-FP8 Linear (activation Q to
E4M3 + FP8 GEMM).  Weights stay packed in HBM; every launch reads a different
copy of the packed weight + scales (copies per format total >= 512 MiB, twice
the 256 MB Infinity Cache), so the weight stream is cold.  X and bias stay warm
(they are the previous layer's output).  The timed steps run as one HIP graph
replay between two synchronizations.

Metric: effective weight-stream bandwidth = (packed weight + scale bytes) /
time.  `value` is the whole step's effective bytes / ms_per_step; per-format
kernel figures come from HIP-event-timed graphs of back-to-back launches of that
kernel alone (its average launch duration).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight-stream TB/s (+% HBM peak), 3072→4096 Linear, M=32, per format"
HBM_PEAK_GBS = 8000.0
M, N, K = 32, 4096, 3072
FORMATS = ["int4", "fp8", "nvfp4", "mxfp4"]
COLD_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--kernel-reps", type=int, default=400, help="launches per per-kernel timing graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--hot", action="store_true", help="one weight copy per format (cache-resident)")
    p.add_argument("--only", default=None, help="time only this format's kernel (profiling aid)")
    p.add_argument("--no-sweep", action="store_true", help="skip the M sweep (MXFP4 M=1..4096, static FP8 M=4096)")
    return p.parse_args()


def effective_bytes(fmt):
    from weight_only_bit_dequant_amd import wq

    if fmt == "static_fp8":
        _, pb, sb, _ = wq.wq_layout("fp8", N, K)
        return pb + sb + 4  # + the activation scale
    _, pb, sb, gb = wq.wq_layout(fmt, N, K)
    return pb + sb + gb


def algorithmic_bytes(fmt):
    """Bytes one launch must move at minimum: weight stream + X + bias + Y."""
    xb = M * K * 2
    yb = M * N * 2
    if fmt == "static_fp8":
        return effective_bytes(fmt) + xb + yb  # X read once by the act-Q (fp8 copy stays on chip/L2)
    return effective_bytes(fmt) + xb + N * 2 + yb


def cpu_baseline(seconds_budget=12.0):
    """Time the CPU oracle (dequantize + fp64 GEMM + bias) per format on the
    full 4096x3072 layer at M=32 -- the same computation the step does."""
    import numpy as np

    from oracle import gemm as G
    from oracle import quant as Q
    from weight_only_bit_dequant_amd import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    total_bytes = 0
    total_time = 0.0
    per = {}
    per_fmt_budget = seconds_budget / len(FORMATS)
    for fmt in FORMATS:
        cfg = synth.WORKLOADS[fmt]["cfg"]
        W, b, X = synth.linear_case(N, K, M, cfg=cfg)
        codes, scales, g = Q.quantize(fmt, W)
        reps = []
        t_fmt = time.perf_counter()
        while len(reps) < 3 or time.perf_counter() - t_fmt < per_fmt_budget:
            t0 = time.perf_counter()
            Wd = Q.dequant(fmt, codes, scales, g)
            G.linear_fp64(X, Wd, b)
            reps.append(time.perf_counter() - t0)
        t = float(np.median(reps))
        per[fmt] = t
        total_bytes += effective_bytes(fmt)
        total_time += t
    return {
        "value": total_bytes / total_time / 1e12,
        "unit": "TB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "full 4096x3072 layer at M=32: dequantize + fp64 GEMM + bias per weight-only format "
                  "(INT4, FP8, NVFP4, MXFP4), repeated for ~3 s per format, median; effective weight bytes / "
                  "oracle time",
        "seconds_per_format": {k: round(v, 4) for k, v in per.items()},
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def m_sweep(layers, dev, capture):
    """The other workload points (reported beside the M=32 line): MXFP4 at
    M in {1, 32, 256, 4096} and the static-FP8 layer at M=4096, each timed as a
    graph of back-to-back launches over the same cold weight copies.  Large M
    is bound by the matrix cores: FLOP/s against the dense bf16 (MXFP4) or
    FP8 (static) peak."""
    import torch

    from weight_only_bit_dequant_amd import synth, wq

    res = {}
    peak = {"mxfp4": 2500.0, "static_fp8": 5000.0}  # dense TFLOP/s (bf16 / fp8)
    for fmt, Ms in (("mxfp4", (1, 32, 256, 4096)), ("static_fp8", (32, 4096))):
        lay = layers[fmt]
        for Mv in Ms:
            X = synth.as_torch_bf16(synth.activations(Mv, K, synth.SEED_X + synth.WORKLOADS[fmt]["cfg"]), dev)
            Y = torch.empty((Mv, N), dtype=torch.bfloat16, device=dev)
            if fmt == "static_fp8":
                ws = torch.zeros(max(1, wq.wq_fp8_static_workspace(Mv, N, K)), dtype=torch.uint8, device=dev)
            else:
                ws = torch.zeros(max(1, wq.wq_linear_workspace("mxfp4", Mv, N, K)), dtype=torch.uint8, device=dev)

            def run(first, count, lay=lay, X=X, Y=Y, ws=ws, fmt=fmt):
                for i in range(first, first + count):
                    r = lay["reps"][i % len(lay["reps"])]
                    if fmt == "static_fp8":
                        wq.wq_fp8_static_linear(X, lay["act_scale"], r["packed"], r["scales"], None, Y, ws)
                    else:
                        wq.wq_linear("mxfp4", X, r["packed"], r["scales"], None, lay["bias"], N, Y, ws)

            reps = 200 if Mv <= 256 else 30
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
            eff = effective_bytes(fmt)
            res[f"{fmt}_M{Mv}"] = {
                "us_per_launch": round(us, 3),
                "TFLOPs": round(flop / (us * 1e-6) / 1e12, 2),
                "pct_mfma_peak": round(100.0 * flop / (us * 1e-6) / 1e12 / peak[fmt], 2),
                "effective_TBps": round(eff / (us * 1e-6) / 1e12, 4),
                "launches": 2 if fmt == "static_fp8" else 1,
            }
            del g
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch

    from weight_only_bit_dequant_amd import synth, wq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- data: seeded synthetic layer per format, quantized on the GPU
    layers = {}
    for fmt in FORMATS + ["static_fp8"]:
        info = synth.WORKLOADS[fmt]
        W, b, X = synth.linear_case(N, K, M, cfg=info["cfg"], bias=info["bias"])
        qfmt = "fp8" if fmt == "static_fp8" else fmt
        q = wq.quantize(qfmt, synth.as_torch_bf16(W, dev))
        eff = effective_bytes(fmt)
        copies = 1 if args.hot else max(2, -(-COLD_BYTES // eff))
        reps = [{"packed": q["packed"], "scales": q["scales"], "global": q["global"]}]
        for _ in range(copies - 1):
            reps.append({"packed": q["packed"].clone(), "scales": q["scales"].clone(),
                         "global": None if q["global"] is None else q["global"].clone()})
        lay = {"reps": reps, "X": synth.as_torch_bf16(X, dev),
               "bias": synth.as_torch_bf16(b, dev) if b is not None else None,
               "Y": torch.empty((M, N), dtype=torch.bfloat16, device=dev), "fmt": qfmt}
        if fmt == "static_fp8":
            cal = [synth.as_torch_bf16(synth.activations(M, K, synth.SEED_CAL + 100 + i), dev) for i in range(10)]
            lay["act_scale"], _ = wq.calibrate_act_scale(cal)
        layers[fmt] = lay
    ws_bytes = max([wq.wq_linear_workspace(f, M, N, K) for f in FORMATS] + [wq.wq_fp8_static_workspace(M, N, K)])
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def launch(fmt, i):
        lay = layers[fmt]
        r = lay["reps"][i % len(lay["reps"])]
        if fmt == "static_fp8":
            wq.wq_fp8_static_linear(lay["X"], lay["act_scale"], r["packed"], r["scales"], lay["bias"], lay["Y"], ws)
        else:
            wq.wq_linear(lay["fmt"], lay["X"], r["packed"], r["scales"], r["global"], lay["bias"], N, lay["Y"], ws)

    step_fmts = [args.only] if args.only else FORMATS + ["static_fp8"]

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
            for f in step_fmts:
                launch(f, st)

    # ---------------- whole-step timing
    g_warm = capture(steps_fn, max(1, args.warmup))
    g_timed = capture(steps_fn, args.steps)
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    step_eff = sum(effective_bytes(f) for f in step_fmts)
    value = step_eff / (ms_per_step * 1e-3) / 1e12

    # ---------------- per-kernel timing (back-to-back launches of one kernel)
    per_format = {}
    for f in step_fmts:
        g = capture(lambda first, count, f=f: [launch(f, i) for i in range(first, first + count)], args.kernel_reps)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.kernel_reps
        eff = effective_bytes(f)
        per_format[f] = {
            "us_per_launch": round(us, 3),
            "effective_TBps": round(eff / (us * 1e-6) / 1e12, 4),
            "pct_hbm_peak": round(100.0 * eff / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "effective_bytes": eff,
            "algorithmic_bytes": algorithmic_bytes(f),
            "copies": len(layers[f]["reps"]),
            "launches": 2 if f == "static_fp8" else 1,
        }
        del g

    sweep = None if (args.no_sweep or args.only) else m_sweep(layers, dev, capture)

    dominant = max(per_format, key=lambda f: per_format[f]["us_per_launch"])
    d = per_format[dominant]
    achieved = d["algorithmic_bytes"] / (d["us_per_launch"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dominant,
                "algorithmic_bytes_per_launch": d["algorithmic_bytes"]}

    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "nn.Linear(3072->4096) bf16+bias, M=32: INT4-g128 / FP8-row / NVFP4 / MXFP4 "
                               "weight-only dequant-GEMMs + static-FP8 (act Q + FP8 GEMM), cold weight copies",
                   "M": M, "N": N, "K": K, "formats": step_fmts, "cold": not args.hot},
        "roofline": roofline,
        "per_format": per_format,
        "wall_s_timed": round(t_wall, 4),
    }
    if sweep is not None:
        out["m_sweep"] = sweep
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
