#!/usr/bin/env python3
"""Benchmark of the gfx950 fp32 GEMM: GFLOP/s (2MNK/t) at 4096^3 and its
fraction of the MI355X fp32 MFMA peak.

One step = one gemm_f32 call (C = A x B, fp32, row-major) on the 4096^3
workload with A and B already resident in HBM.  W untimed warm-up steps, then
K timed steps bracketed by a device synchronisation on both sides.  Prints
ONE JSON line.

Kernel time is measured with HIP events recorded on the stream the library
launches on (torch's current stream), one pair per launch; the roofline
fraction uses the mean launch duration.  The skinny 8 x 8192 x 8192 workload
is timed the same way (with rotating copies of B so it streams from HBM, not
from the 256 MB last-level cache) and reported under "secondary".

cpu_baseline: the CPU oracle (binary64 triple loop) timed on a bounded sample
of the same workload (the first R rows of A), scaled to GFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    return ap.parse_args()


def time_launches(fn, steps, warmup, stream):
    """Run fn() warmup times, then steps times with an event pair around each
    launch on `stream`.  Returns (wall ms per step, list of per-launch ms)."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in evs]
    return wall, per


def traffic_for(kernel_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it was taken on a different kernel source."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get(kernel_name)
    except ValueError:
        return None
    from dense_fp32_gemm_f32_amd.prof_summary import source_hash
    if not rec or rec.get("source_sha256") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, target_s):
    """The oracle on the first R rows of A; R sized from a short probe."""
    import numpy as np
    import oracle
    from dense_fp32_gemm_f32_amd import inputs
    A, B = inputs.workload_inputs(w)
    A, B = A.numpy(), B.numpy()
    threads = oracle.max_threads()
    probe_rows = 32
    t0 = time.perf_counter()
    oracle.gemm(np.ascontiguousarray(A[:probe_rows]), B, want_f64=False)
    dt = time.perf_counter() - t0
    rows = int(min(w.M, max(probe_rows, probe_rows * target_s / max(dt, 1e-6))))
    rows = max(probe_rows, rows // 32 * 32)
    t0 = time.perf_counter()
    oracle.gemm(np.ascontiguousarray(A[:rows]), B, want_f64=False)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of A ({rows}x{w.N}x{w.K}, binary64 "
                      f"accumulation), {dt:.2f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs

    binding.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    props = torch.cuda.get_device_properties(dev)

    # ---- headline: 4096^3 ----------------------------------------------------
    w = inputs.WORKLOADS[inputs.HEADLINE]
    A_cpu, B_cpu = inputs.workload_inputs(w)
    A, B = A_cpu.to(dev), B_cpu.to(dev)
    C = torch.empty((w.M, w.N), device=dev)
    kname = binding.selected_kernel(A, B, C)
    wall_ms, per = time_launches(lambda i: binding.gemm(A, B, C), args.steps, args.warmup,
                                 stream)
    mean_launch_ms = sum(per) / len(per)
    flops = w.flops
    value = flops / (wall_ms * 1e-3) / 1e9
    achieved_tflops = flops / (mean_launch_ms * 1e-3) / 1e12
    traffic = traffic_for(kname)
    result = {
        "metric": "fp32 GEMM GFLOP/s (2MNK/t) at 4096^3 and % of MI355X fp32 MFMA peak",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": "row-major",
                   "inputs": "A,B ~ U[-1,1) seed 1003", "kernel": kname,
                   "pct_fp32_mfma_peak": round(100 * value / 1e3 / PEAK_FP32_MFMA_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tflops, 2),
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": traffic,
                     "launch_ms_mean": round(mean_launch_ms, 4),
                     "launch_ms_min": round(min(per), 4)},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
    }
    del A, B, C
    torch.cuda.empty_cache()

    # ---- secondary: the skinny bandwidth-bound workload -------------------------
    if not args.no_secondary:
        ws = inputs.WORKLOADS[inputs.SKINNY]
        copies = 4   # 4 x 256 MiB of B > the 256 MB last-level cache
        As, Bs = [], []
        for c in range(copies):
            a_cpu, b_cpu = inputs.make_ab(ws.M, ws.N, ws.K, ws.dist_a, ws.dist_b, ws.seed + 100 * c)
            As.append(a_cpu.to(dev))
            Bs.append(b_cpu.to(dev))
        Cs = [torch.empty((ws.M, ws.N), device=dev) for _ in range(copies)]
        sk = binding.selected_kernel(As[0], Bs[0], Cs[0])
        wall_s, per_s = time_launches(
            lambda i: binding.gemm(As[i % copies], Bs[i % copies], Cs[i % copies]),
            max(args.steps, 20), args.warmup, stream)
        mean_s = sum(per_s) / len(per_s)
        gbs = ws.algo_bytes / (mean_s * 1e-3) / 1e9
        result["secondary"] = {ws.name: {
            "kernel": sk, "launch_us_mean": round(mean_s * 1e3, 2),
            "launch_us_min": round(min(per_s) * 1e3, 2),
            "GFLOP/s": round(ws.flops / (mean_s * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for(sk)}}}
        del As, Bs, Cs
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
