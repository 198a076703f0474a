"""Time every kernel of the table on given shapes (the sweep that the gfx950
tuning table in ``csrc/tuning_gfx950.h`` is chosen from).

    python -m dense_fp32_gemm_f32_amd.tune --shapes 4096x4096x4096,8x8192x8192 \
        [--filter mfma_] [--reps 10] [--json out.json]

A shape is MxNxK (row-major, packed pitches, 16-byte aligned bases).  Each
kernel that accepts the shape runs ``--warmup`` times, then ``--reps`` times
with a HIP event pair on the launch stream around each call, the candidates
taking turns (after --spin-ms of load to settle the clocks), each timed call
right after --lead untimed calls of the same kernel; the median is reported.
Inputs rotate over enough copies to exceed the 256 MB last-level cache when B
is large or the shape is skinny (M <= 16), so bandwidth-bound shapes stream
from HBM.  Prints one line per (shape, kernel).

``--sweep`` loads the sweep build of the library (``python -m
dense_fp32_gemm_f32_amd.build_lib --sweep``), whose table also holds the
variants that are not in the default build.
"""
from __future__ import annotations

import argparse
import json
import sys
import time


def parse_shape(s: str):
    m, n, k = (int(x) for x in s.lower().split("x"))
    return m, n, k


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default="4096x4096x4096")
    ap.add_argument("--filter", default="", help="comma-separated kernel-name prefixes")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--lead", type=int, default=1,
                    help="untimed calls of a candidate right before each of its timed calls")
    ap.add_argument("--spin-ms", type=float, default=300.0,
                    help="keep the GPU busy this long before timing a shape")
    ap.add_argument("--json", default="")
    ap.add_argument("--with-torch", action="store_true",
                    help="also time torch.matmul in fp32 (vendor library, context only)")
    ap.add_argument("--layout", default="nn", choices=["nn", "nt", "tn", "tt"],
                    help="op(A) op(B): n = stored as is, t = stored transposed "
                         "(gemm_f32_ex kernels); the plain kernels run only for nn")
    ap.add_argument("--alpha", type=float, default=1.0)
    ap.add_argument("--beta", type=float, default=0.0)
    ap.add_argument("--sweep", action="store_true",
                    help="time the kernels of the sweep build (libgemm_f32_sweep.so)")
    args = ap.parse_args(argv)

    import torch
    from dense_fp32_gemm_f32_amd import binding, build_lib, inputs

    binding.load(build_lib.SWEEP_LIB if args.sweep else None)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    names = binding.kernel_names()
    prefixes = [p for p in args.filter.split(",") if p]
    rows = []
    for shape in args.shapes.split(","):
        M, N, K = parse_shape(shape)
        b_bytes = 4 * K * N
        if M <= 16 and b_bytes >= 2 ** 20:
            # bound by HBM: about 1 GiB of B in rotation
            copies = max(1, min(32, -(-1024 * 2 ** 20 // b_bytes)))
        elif b_bytes > 32 * 2 ** 20:
            copies = max(1, min(4, -(-1024 * 2 ** 20 // b_bytes)))
        else:
            copies = 1
        As, Bs, Cs = [], [], []
        ta, tb = args.layout[0] == "t", args.layout[1] == "t"
        for c in range(copies):
            a, b = inputs.make_ab(M, N, K, "u11", "u11", 9000 + c)
            # the stored operands: A^T (K x M) and B^T (N x K) when transposed
            As.append((a.t().contiguous() if ta else a).to(dev))
            Bs.append((b.t().contiguous() if tb else b).to(dev))
            Cs.append(torch.zeros((M, N), device=dev))
        lda, ldb = (M if ta else K), (K if tb else N)
        flops = 2.0 * M * N * K
        algo_bytes = 4.0 * (M * K + K * N + M * N)
        default = binding.gemm_f32_selected_kernel_ex(
            int(ta), int(tb), M, N, K, lda, ldb, N, args.alpha, args.beta,
            As[0].data_ptr(), Bs[0].data_ptr(), Cs[0].data_ptr())
        cands = [(i, n) for i, n in enumerate(names)
                 if not prefixes or any(n.startswith(p) for p in prefixes)]
        if args.with_torch:
            cands.append((-1, "torch.matmul"))
        calls = []
        for idx, name in cands:
            if idx >= 0:
                s = stream.cuda_stream

                def call(i, idx=idx):
                    a, b, c = As[i % copies], Bs[i % copies], Cs[i % copies]
                    return binding.gemm_f32_run_kernel_ex(
                        idx, int(ta), int(tb), M, N, K, args.alpha, a.data_ptr(), lda,
                        b.data_ptr(), ldb, args.beta, c.data_ptr(), N, s)
                if call(0) != 0:
                    continue   # kernel does not accept this shape
            else:
                torch.backends.cuda.matmul.allow_tf32 = False

                def call(i):
                    a = As[i % copies].t() if ta else As[i % copies]
                    b = Bs[i % copies].t() if tb else Bs[i % copies]
                    if args.alpha == 1.0 and args.beta == 0.0:
                        torch.matmul(a, b, out=Cs[i % copies])
                    else:
                        torch.addmm(Cs[i % copies], a, b, beta=args.beta, alpha=args.alpha,
                                    out=Cs[i % copies])
                    return 0
            calls.append((name, call))
        if not calls:
            continue
        # Every call takes the next copy in rotation, whichever candidate
        # makes it, so that no call finds its inputs left in the last-level
        # cache by the call before it (with the same copy for every candidate
        # of a round, all but the first would read B partly from the cache).
        seq = iter(range(1 << 62))
        # settle the clocks: keep the GPU busy for --spin-ms before timing
        torch.cuda.synchronize()
        t_end = time.perf_counter() + args.spin_ms * 1e-3
        while time.perf_counter() < t_end:
            for _, call in calls:
                call(next(seq))
            torch.cuda.synchronize()
        for _, call in calls:
            for _ in range(args.warmup):
                call(next(seq))
        torch.cuda.synchronize()
        # round-robin over the candidates so that clock drift hits all alike;
        # each timed call follows --lead untimed calls of the same kernel, so
        # it never runs right after another candidate (a streaming kernel
        # without the non-temporal hint leaves the caches in a state that
        # costs the next kernel about 10 us at 16 x 8192 x 8192)
        evs = {name: [] for name, _ in calls}
        for r in range(args.reps):
            for name, call in calls:
                for _ in range(args.lead):
                    call(next(seq))
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                call(next(seq))
                b.record(stream)
                evs[name].append((a, b))
        torch.cuda.synchronize()
        for name, _ in calls:
            ms = sorted(a.elapsed_time(b) for a, b in evs[name])
            mean = sum(ms) / len(ms)
            med = ms[len(ms) // 2]
            row = {"shape": f"{M}x{N}x{K}", "layout": args.layout, "kernel": name,
                   "default": name == default,
                   "mean_us": round(mean * 1e3, 2), "median_us": round(med * 1e3, 2),
                   "min_us": round(ms[0] * 1e3, 2),
                   "tflops": round(flops / (med * 1e-3) / 1e12, 2),
                   "gbs": round(algo_bytes / (med * 1e-3) / 1e9, 1)}
            rows.append(row)
            print(f"{row['shape']:>16} {name:<40} {'*' if row['default'] else ' '} "
                  f"median {row['median_us']:>10.2f} us  mean {row['mean_us']:>10.2f}  "
                  f"min {row['min_us']:>10.2f}  {row['tflops']:>8.2f} TFLOP/s  "
                  f"{row['gbs']:>9.1f} GB/s", flush=True)
        del As, Bs, Cs
        torch.cuda.empty_cache()
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rows, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
