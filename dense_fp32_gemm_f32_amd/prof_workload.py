"""A short, profiler-friendly run of one GEMM workload plus a copy of known
size, for rocprofv3 kernel traces and hardware counters.

    rocprofv3 --kernel-trace --stats -d OUT -o run -f csv -- \
        python3 -m dense_fp32_gemm_f32_amd.prof_workload --workload square_4096
    rocprofv3 --pmc FETCH_SIZE -d OUT -o fetch -f csv -- \
        python3 -m dense_fp32_gemm_f32_amd.prof_workload --workload square_4096

A run with ``--settle-ms`` (a trace run) also prints the shader clock right
after the launches (``gemm_f32_clock_probe``), which ``prof_summary --log``
quotes.

The copy (``torch.Tensor.copy_`` of ``--copy-mib`` MiB, a plain streaming
kernel that reads and writes exactly that many bytes) calibrates the
FETCH_SIZE / WRITE_SIZE counters: HBM bytes of a GEMM launch are its counter
value scaled by (known copy bytes / copy counter value).
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="square_4096")
    ap.add_argument("--kernel", default="", help="run this kernel instead of the dispatcher's")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--copies", type=int, default=0,
                    help="rotate this many input copies (0: 4 when B exceeds 128 MiB)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--torch", action="store_true",
                    help="run torch.matmul in fp32 (the vendor library, for comparison) instead")
    ap.add_argument("--settle-ms", type=float, default=0.0,
                    help="before the --reps launches, repeat the same call for this long so the "
                         "clocks leave the idle state (for traces; counter runs leave it 0)")
    ap.add_argument("--trans-b", action="store_true",
                    help="B stored transposed (N x K), through gemm_f32_ex")
    ap.add_argument("--rows", type=int, default=0,
                    help="use this many rows of A instead of the workload's M")
    ap.add_argument("--reduce", type=int, default=0,
                    help="run reduce_sum_f32 on this many floats (4 copies) instead of a GEMM")
    args = ap.parse_args(argv)

    import torch
    from dense_fp32_gemm_f32_amd import binding, inputs

    binding.load()
    dev = torch.device("cuda:0")
    if args.reduce:
        xs = [inputs.draw_matrix(1, args.reduce, "u11", 1300 + c).reshape(-1).to(dev)
              for c in range(4)]
        out = torch.empty(1, device=dev)
        print(f"reduce_sum_f32 on {args.reduce} floats, {args.reps} launches over 4 copies",
              flush=True)
        _settle(lambda i: binding.reduce_sum(xs[i % 4], out), args.settle_ms)
        for i in range(args.reps):
            binding.reduce_sum(xs[i % 4], out)
        torch.cuda.synchronize()
        if args.settle_ms > 0:
            _clock(binding)
        _calibration_copy(dev, args.copy_mib)
        return 0
    w = inputs.WORKLOADS[args.workload]
    M = args.rows or w.M
    copies = args.copies or (4 if 4 * w.K * w.N > 128 * 2 ** 20 else 1)
    As, Bs, Cs = [], [], []
    for c in range(copies):
        a, b = inputs.make_ab(M, w.N, w.K, w.dist_a, w.dist_b, w.seed + 100 * c)
        As.append(a.contiguous().to(dev))
        Bs.append((b.t() if args.trans_b else b).contiguous().to(dev))
        Cs.append(torch.empty((M, w.N), device=dev))
    if args.torch:
        torch.backends.cuda.matmul.allow_tf32 = False
        print(f"workload {w.name}: torch.matmul, {args.reps} launches", flush=True)
        for i in range(args.reps):
            torch.matmul(As[i % copies], Bs[i % copies], out=Cs[i % copies])
        torch.cuda.synchronize()
        _calibration_copy(dev, args.copy_mib)
        return 0
    tb = args.trans_b
    name = args.kernel or (binding.selected_kernel_ex(As[0], Bs[0], Cs[0], trans_b=True) if tb
                           else binding.selected_kernel(As[0], Bs[0], Cs[0]))
    print(f"workload {w.name}{' with B stored transposed' if tb else ''}, {M} rows: kernel "
          f"{name}, {args.reps} launches over {copies} input copies", flush=True)

    def call(i):
        if tb:
            binding.gemm_ex(As[i % copies], Bs[i % copies], Cs[i % copies], trans_b=True,
                            kernel=name)
        else:
            binding.run_kernel(name, As[i % copies], Bs[i % copies], Cs[i % copies])
    _settle(call, args.settle_ms)
    for i in range(args.reps):
        call(i)
    torch.cuda.synchronize()
    if args.settle_ms > 0:
        _clock(binding)
    _calibration_copy(dev, args.copy_mib)
    return 0


def _clock(binding):
    """The shader clock right after the launches, from gemm_f32_clock_probe in
    the same process (its own kernel in the trace)."""
    ghz, wall_khz, peak_khz = binding.clock_probe()
    g = sorted(ghz)
    print(f"clock probe: median {g[len(g) // 2]:.4f} GHz (min {g[0]:.4f}, max {g[-1]:.4f}) "
          f"over {len(g)} workgroups; constant counter {wall_khz} kHz, device peak clock "
          f"{peak_khz} kHz", flush=True)


def _settle(fn, ms):
    """Repeat fn for `ms` milliseconds (no-op for 0)."""
    import time
    import torch
    if ms <= 0:
        return
    t_end, i = time.perf_counter() + ms * 1e-3, 0
    while time.perf_counter() < t_end:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _calibration_copy(dev, mib):
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty(n, device=dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"calibration copy: 3 x {mib} MiB read + {mib} MiB written", flush=True)


if __name__ == "__main__":
    sys.exit(main())
