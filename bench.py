#!/usr/bin/env python3
"""Benchmark of the gfx950 fp32 GEMM: GFLOP/s (2MNK/t) at 4096^3 and its
fraction of the MI355X fp32 MFMA peak.

One step = one gemm_f32 call (C = A x B, fp32, row-major) on the 4096^3
workload with A and B already resident in HBM.  --settle seconds (0.3 by
default) of untimed calls, W untimed warm-up steps, then K timed steps
bracketed by a device synchronisation on both sides.  Prints ONE JSON line;
its "timing" object declares the settle and holds every launch's duration,
the means of the first and last quarter of the timed launches, and the shader
clock (gemm_f32_clock_probe) before the settle and right after the timed
steps.

Kernel time is measured with HIP events recorded on the stream the library
launches on (torch's current stream), one pair per launch; the roofline
fraction uses the mean launch duration.  The skinny 8 x 8192 x 8192 workload
is timed the same way (with rotating copies of B so it streams from HBM, not
from the 256 MB last-level cache) and reported under "secondary"; each
secondary measurement first runs its own call untimed for 300 ms, so that
short kernels are not timed at the idle clocks the host-side work before
them leaves.  Also under "secondary": 64 batched 512^3 products, the sum of
2^26 floats, 4096^3 with bias and ReLU, 4096^3 with an operand stored
transposed (nt, tn, tt), and the skinny product with B stored transposed
(8 and 16 rows).

cpu_baseline: the CPU oracle (binary64 triple loop) timed on a bounded sample
of the same workload (the first R rows of A), scaled to GFLOP/s.

--configs: one JSON line per workload instead (median and min of 20 timed
calls, rate and fraction of peak, bitwise rerun check, and the oracle's time
on the host with the GPU result's agreement with it).

--shards: the same lines for one GPU's share of the 4096^3 and skinny
products split 8 ways (the kernels at the shapes each GPU of a split would
run; the collectives around them are not built).
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed headline calls before the --warmup steps, so the "
                         "timed steps do not start at the idle clocks input generation leaves "
                         "(declared in the record; 0 for none)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the single headline line, print one JSON line per "
                         "workload (median/min time, rate, reruns, oracle time and agreement)")
    ap.add_argument("--shards", action="store_true",
                    help="the same per-workload lines for one GPU's share of the 4096^3 and "
                         "skinny products split 8 ways (along M, N or K)")
    return ap.parse_args()


def settle(fn, seconds=0.3):
    """Untimed: keep calling fn for `seconds`, so that the GPU clocks have left
    the idle state that host-side work (input generation, oracle checks) puts
    them in; a few dozen warm-up launches of a 50 us kernel take 2 ms, too
    short for that.  Returns the number of calls made."""
    import torch
    t_end, i = time.perf_counter() + seconds, 0
    while time.perf_counter() < t_end:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_launches(fn, steps, warmup, stream, settle_s=0.3, stats=None):
    """Settle the clocks (settle_s seconds of untimed calls), run fn() warmup
    times, then steps times with an event pair around each launch on
    `stream`.  Returns (wall ms per step, list of per-launch ms); the number
    of settle calls goes to stats["settle_calls"] when stats is a dict."""
    import torch
    if settle_s > 0:
        n = settle(fn, settle_s)
        if stats is not None:
            stats["settle_calls"] = n
    # fn(i) takes input copy i % copies: consecutive calls read different
    # copies, so none finds its inputs in the cache from the call before
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        fn(warmup + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in evs]
    return wall, per


def profile_record(kernel_name: str, workload: str):
    """The committed rocprofv3 record of a kernel (profiles/traffic.json), or
    None if there is none, it was taken on another workload, or on a
    different kernel source."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get(kernel_name)
    except ValueError:
        return None
    from dense_fp32_gemm_f32_amd.prof_summary import source_hash
    if not rec or rec.get("workload") != workload:
        return None
    if rec.get("source_sha256") != source_hash(kernel_name):
        return None
    return rec


def traffic_for(kernel_name: str, workload: str):
    """HBM bytes per launch of the kernel on this workload from the committed
    rocprofv3 counter summary, or None if there is no such summary or it was
    taken on a different kernel source."""
    rec = profile_record(kernel_name, workload)
    return rec.get("hbm_bytes_per_launch") if rec else None


def _clock_summary(probe):
    """Median, min and max of the per-workgroup clocks of one probe, in GHz,
    with the counter rates it was read against."""
    ghz, wall_khz, peak_khz = probe
    if not ghz:
        return None
    g = sorted(ghz)
    return {"median": round(g[len(g) // 2], 4), "min": round(g[0], 4), "max": round(g[-1], 4),
            "wall_counter_khz": wall_khz, "device_peak_khz": peak_khz}


def launch_amortisation(stream, steps, warmup, batch=64, n=512):
    """Many small products (batch x 512^3, the pages' N = 512 size): per-product
    time for separate gemm_f32 calls, one gemm_f32_batched call, and a HIP
    graph replaying the separate calls.  Event-timed on the launch stream."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    A = torch.stack([inputs.draw_matrix(n, n, "u11", 1100 + b) for b in range(batch)]).cuda()
    B = torch.stack([inputs.draw_matrix(n, n, "u11", 1200 + b) for b in range(batch)]).cuda()
    C = torch.empty((batch, n, n), device="cuda")
    flops = 2.0 * n * n * n * batch

    def separate(_i):
        for b in range(batch):
            binding.gemm(A[b], B[b], C[b])

    def batched(_i):
        binding.gemm_batched(A, B, C)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        separate(0)   # the split-K workspace of the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        separate(0)
    torch.cuda.synchronize()

    out = {"products": batch, "M": n, "N": n, "K": n,
           "kernel_separate": binding.selected_kernel(A[0], B[0]),
           "kernel_batched": binding.selected_kernel_batched(A, B, C)}
    for name, fn in (("separate_calls", separate), ("one_batched_call", batched),
                     ("graph_of_separate_calls", lambda _i: g.replay())):
        _, per = time_launches(fn, steps, warmup, stream)
        mean_ms = sum(per) / len(per)
        out[name] = {"us_per_product": round(mean_ms * 1e3 / batch, 3),
                     "TFLOP/s": round(flops / (mean_ms * 1e-3) / 1e12, 2)}
    return out


def sum_bandwidth(stream, steps, warmup, n=2 ** 26, copies=4):
    """reduce_sum_f32 on 2^26 floats (the pages' reduction size), rotating 4
    copies (1 GiB > the 256 MB last-level cache) so it streams from HBM."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    xs = [inputs.draw_matrix(1, n, "u11", 1300 + c).reshape(-1).cuda() for c in range(copies)]
    out = torch.empty(1, device="cuda")
    _, per = time_launches(lambda i: binding.reduce_sum(xs[i % copies], out), steps, warmup,
                           stream)
    mean_ms = sum(per) / len(per)
    gbs = 4.0 * n / (mean_ms * 1e-3) / 1e9
    return {"n": n, "launch_us_mean": round(mean_ms * 1e3, 2),
            "launch_us_min": round(min(per) * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def fused_epilogue(stream, steps, warmup):
    """4096^3 with a bias row and ReLU: gemm_f32_fused (applied as C is stored)
    against gemm_f32 followed by a separate bias + ReLU pass over C (torch
    elementwise ops, one more read and write of the 64 MiB C)."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    w = inputs.WORKLOADS[inputs.HEADLINE]
    A_cpu, B_cpu = inputs.workload_inputs(w)
    A, B = A_cpu.cuda(), B_cpu.cuda()
    C = torch.empty((w.M, w.N), device="cuda")
    bias = inputs.uniform_matrix(1, w.N, 1400).reshape(-1).cuda()

    def fused(_i):
        binding.gemm_fused(A, B, C, bias=bias, act=binding.ACT_RELU)

    def separate(_i):
        binding.gemm(A, B, C)
        torch.relu_(C.add_(bias))

    out = {"kernel": binding.selected_kernel_ex(A, B, C, alpha=1.0, beta=0.0)}
    for name, fn in (("fused", fused), ("gemm_then_bias_relu", separate)):
        _, per = time_launches(fn, steps, warmup, stream)
        mean_ms = sum(per) / len(per)
        out[name] = {"ms": round(mean_ms, 4),
                     "TFLOP/s": round(w.flops / (mean_ms * 1e-3) / 1e12, 2)}
    return out


def transposed_layouts(stream, steps, warmup):
    """4096^3 with an operand stored transposed (gemm_f32_ex; B stored N x K,
    A stored K x M, or both), the same inputs as the headline."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    w = inputs.WORKLOADS[inputs.HEADLINE]
    A_cpu, B_cpu = inputs.workload_inputs(w)
    C = torch.empty((w.M, w.N), device="cuda")
    out = {}
    for lay in ("nt", "tn", "tt"):
        ta, tb = lay[0] == "t", lay[1] == "t"
        A = (A_cpu.t().contiguous() if ta else A_cpu).cuda()
        B = (B_cpu.t().contiguous() if tb else B_cpu).cuda()
        kname = binding.selected_kernel_ex(A, B, C, trans_a=ta, trans_b=tb)
        _, per = time_launches(lambda _i: binding.gemm_ex(A, B, C, trans_a=ta, trans_b=tb),
                               steps, warmup, stream)
        mean_ms = sum(per) / len(per)
        tflops = w.flops / (mean_ms * 1e-3) / 1e12
        out[lay] = {"kernel": kname, "ms": round(mean_ms, 4), "TFLOP/s": round(tflops, 2),
                    "frac": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4)}
        del A, B
    return out


def skinny_transposed(stream, steps, warmup, copies=4):
    """The skinny product with B stored transposed (gemm_f32_ex, N x K), M = 8
    (the skinny workload's shape) and M = 16: 4 rotating copies of B^T (1 GiB)
    so it streams from HBM, against 8 TB/s."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    ws = inputs.WORKLOADS[inputs.SKINNY]
    out = {}
    for M in (8, 16):
        As, Bs = [], []
        for c in range(copies):
            a_cpu, b_cpu = inputs.make_ab(M, ws.N, ws.K, ws.dist_a, ws.dist_b, ws.seed + 100 * c)
            As.append(a_cpu.cuda())
            Bs.append(b_cpu.t().contiguous().cuda())
        Cs = [torch.empty((M, ws.N), device="cuda") for _ in range(copies)]
        kname = binding.selected_kernel_ex(As[0], Bs[0], Cs[0], trans_b=True)
        _, per = time_launches(
            lambda i: binding.gemm_ex(As[i % copies], Bs[i % copies], Cs[i % copies],
                                      trans_b=True), steps, warmup, stream)
        mean_ms = sum(per) / len(per)
        algo = 4.0 * (M * ws.K + ws.K * ws.N + M * ws.N)
        gbs = algo / (mean_ms * 1e-3) / 1e9
        out[f"{M}x{ws.N}x{ws.K}_nt"] = {
            "kernel": kname, "launch_us_mean": round(mean_ms * 1e3, 2),
            "launch_us_min": round(min(per) * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for(kname, f"skinny_{M}x{ws.N}x{ws.K}_bt")}}
        del As, Bs, Cs
        torch.cuda.empty_cache()
    return out


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


def cpu_baseline_config(w, C_gpu, C_gpu_int):
    """The oracle over the whole workload on the host cores: its time, and how
    the GPU results of the same inputs compare with it (float: max of
    |dC| / sum|a||b|; integer inputs: bit-exact)."""
    import numpy as np
    import oracle
    from dense_fp32_gemm_f32_amd import inputs
    A, B = inputs.workload_inputs(w)
    t0 = time.perf_counter()
    C_ref, _, ABS = oracle.gemm(A.numpy(), B.numpy(), want_f64=True)
    dt = time.perf_counter() - t0
    err = np.abs(C_gpu.astype(np.float64) - C_ref.astype(np.float64))
    ratio = float(np.max(np.where(ABS > 0, err / np.where(ABS > 0, ABS, 1.0), err)))
    Ai, Bi = inputs.workload_inputs(w, integer=True)
    Ci_ref, _, _ = oracle.gemm(Ai.numpy(), Bi.numpy(), want_f64=True)
    return {"oracle_s": round(dt, 3), "oracle_cores": oracle.max_threads(),
            "oracle_gflops": round(w.flops / dt / 1e9, 3),
            "max_err_ratio": ratio, "int_bitexact": bool(np.array_equal(C_gpu_int, Ci_ref))}


def _rocprof_fields(kname, workload):
    """The committed profile summary of the kernel on this workload and its
    calibrated HBM bytes per launch against the algorithmic bytes (None if
    there is none or it is stale)."""
    rec = profile_record(kname, workload)
    if not rec:
        return None
    return {"summary": "profiles/" + rec["summary"], "workload": rec["workload"],
            "hbm_bytes_per_launch": rec["hbm_bytes_per_launch"],
            "x_algorithmic": round(rec["hbm_bytes_per_launch"] / rec["algo_bytes"], 3)}


def copies_parity(As, Bs, Cs):
    """Each rotated input copy's output from the timed calls (the last call on
    that copy) against the oracle: the largest |dC| / sum|a||b| over the
    copies, and whether every copy is within the 1e-4 gate."""
    import numpy as np
    import oracle
    worst = 0.0
    for A, B, C in zip(As, Bs, Cs):
        C_ref, _, ABS = oracle.gemm(A.cpu().numpy(), B.cpu().numpy(), want_f64=True)
        err = np.abs(C.cpu().numpy().astype(np.float64) - C_ref.astype(np.float64))
        ok = err <= 1e-4 * ABS
        worst = max(worst, float(np.max(np.where(ABS > 0, err / np.where(ABS > 0, ABS, 1.0),
                                                 np.where(ok, 0.0, np.inf)))))
    return {"copies": len(As), "copies_max_err_ratio": worst,
            "copies_within_tol": bool(worst <= 1e-4)}


def per_config(args, workloads, share_of=None):
    """One JSON line per workload (the per-config record of the measurement
    plan): 300 ms of untimed calls, 5 warm-up calls, then 20 event-timed
    calls; median and min.  An HBM-bound workload (M <= 16) rotates copies of
    its inputs (at least 4, about 1 GiB of B in all, at most 16) so that B
    streams from HBM rather than from the 256 MB last-level cache."""
    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs
    binding.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    props = torch.cuda.get_device_properties(dev)
    for name, w in workloads.items():
        hbm_bound = w.M <= 16
        copies = max(4, -(-1024 * 2 ** 20 // (4 * w.K * w.N))) if hbm_bound else 1
        copies = min(copies, 16)
        As, Bs, Cs = [], [], []
        for c in range(copies):
            a, b = (inputs.workload_inputs(w) if c == 0 else
                    inputs.make_ab(w.M, w.N, w.K, w.dist_a, w.dist_b, w.seed + 100 * c))
            As.append(a.to(dev))
            Bs.append(b.to(dev))
            Cs.append(torch.empty((w.M, w.N), device=dev))
        kname = binding.selected_kernel(As[0], Bs[0], Cs[0])
        call = lambda i: binding.gemm(As[i % copies], Bs[i % copies], Cs[i % copies])  # noqa: E731
        # 300 ms of calls to settle the clocks, then 5 warm-up and 20 timed ones
        _, per = time_launches(call, 20, 5, stream)
        per = sorted(per)
        t_med, t_min = per[len(per) // 2], per[0]
        C1 = binding.gemm(As[0], Bs[0]).cpu()
        C2 = binding.gemm(As[0], Bs[0]).cpu()
        ai, bi = inputs.workload_inputs(w, integer=True)
        Ci = binding.gemm(ai.to(dev), bi.to(dev)).cpu()
        torch.cuda.synchronize()
        rec = {"config": name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda or w.K,
               "ldb": w.ldb or w.N, "ldc": w.ldc or w.N, "seed": w.seed, "kernel_entry": kname,
               "t_median_us": round(t_med * 1e3, 2), "t_min_us": round(t_min * 1e3, 2),
               "gflops": round(w.flops / (t_med * 1e-3) / 1e9, 1),
               "pct_mfma_peak": round(100 * w.flops / (t_med * 1e-3) / 1e12
                                      / PEAK_FP32_MFMA_TFLOPS, 2),
               "gbps": round(w.algo_bytes / (t_med * 1e-3) / 1e9, 1),
               "pct_hbm_peak": round(100 * w.algo_bytes / (t_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
               "repro_bitexact": bool(torch.equal(C1, C2)),
               "traffic": traffic_for(kname, name) if share_of is None else None,
               "rocprof": _rocprof_fields(kname, name) if share_of is None else None,
               "device": {"name": props.name, "CUs": props.multi_processor_count,
                          "arch": getattr(props, "gcnArchName", ""),
                          "peak_tflops": PEAK_FP32_MFMA_TFLOPS,
                          "peak_tbps": PEAK_HBM_GBS / 1e3}}
        if share_of is not None:
            rec["share_of"] = {"workload": share_of[name], "ways": inputs.SHARD_WAYS}
        if not args.no_cpu_baseline:
            rec.update(cpu_baseline_config(w, C1.numpy(), Ci.numpy()))
            if copies > 1:
                rec.update(copies_parity(As, Bs, Cs))
        print(json.dumps(rec), flush=True)
        del As, Bs, Cs
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.configs or args.shards:
        from dense_fp32_gemm_f32_amd import inputs
        if args.configs:
            per_config(args, inputs.WORKLOADS)
        if args.shards:
            per_config(args, inputs.SHARDS, inputs.SHARD_OF)
        return

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
    # The shader clock as the timed region is entered from idle, then the
    # declared settle (--settle seconds of the same call, untimed), the W
    # warm-up steps and the K timed steps; the clock again right after them.
    clock_before = _clock_summary(binding.clock_probe())
    st = {"settle_calls": 0}
    wall_ms, per = time_launches(lambda i: binding.gemm(A, B, C), args.steps, args.warmup,
                                 stream, settle_s=args.settle, stats=st)
    clock_after = _clock_summary(binding.clock_probe())
    mean_launch_ms = sum(per) / len(per)
    q = max(1, len(per) // 4)
    flops = w.flops
    value = flops / (wall_ms * 1e-3) / 1e9
    achieved_tflops = flops / (mean_launch_ms * 1e-3) / 1e12
    traffic = traffic_for(kname, w.name)
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
        # how the timed steps were reached, and the clock they ran at
        "timing": {"settle_s": args.settle, "settle_calls": st["settle_calls"],
                   "warmup_steps": args.warmup, "events": "one HIP event pair per launch on "
                   "the launch stream",
                   "launch_ms": [round(x, 4) for x in per],
                   "first_quarter_ms_mean": round(sum(per[:q]) / q, 4),
                   "last_quarter_ms_mean": round(sum(per[-q:]) / q, 4),
                   "clock_ghz_before_settle": clock_before,
                   "clock_ghz_after_timed": clock_after,
                   "clock_method": "gemm_f32_clock_probe: s_memtime cycles over s_memrealtime "
                                   "ticks (at wall_counter_khz) across ~1 ms of fp32 MFMA load "
                                   "on every SIMD, median over 1024 workgroups",
                   "peak_at_clock_after_tflops": round(
                       256 * 256 * clock_after["median"] / 1e3, 1) if clock_after else None},
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
                         "traffic": traffic_for(sk, ws.name)}}}
        del As, Bs, Cs
        torch.cuda.empty_cache()

    if not args.no_secondary:
        result.setdefault("secondary", {})["batched_64x512"] = launch_amortisation(
            stream, max(args.steps, 20), args.warmup)
        result["secondary"]["sum_2^26"] = sum_bandwidth(stream, max(args.steps, 20),
                                                        args.warmup)
        result["secondary"]["fused_bias_relu_4096"] = fused_epilogue(stream, args.steps,
                                                                     args.warmup)
        result["secondary"]["transposed_4096"] = transposed_layouts(stream, args.steps,
                                                                    args.warmup)
        result["secondary"]["skinny_b_transposed"] = skinny_transposed(
            stream, max(args.steps, 20), args.warmup)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
