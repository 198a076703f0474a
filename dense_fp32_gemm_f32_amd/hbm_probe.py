"""The HBM read rate this device sustains, beside the library's HBM-bound calls
on the same bytes.

    python -m dense_fp32_gemm_f32_amd.build_lib --sweep        # once
    python -m dense_fp32_gemm_f32_amd.hbm_probe

On four rotating copies of 2^26 floats (256 MiB each, 1 GiB in all, so that
no call finds its input in the 256 MB last-level cache left by the previous
one), each candidate is event-timed (median of --reps calls, one HIP event
pair per call on the launch stream, after --settle-ms of its own calls):

- ``read_probe_g<G>``: ``gemm_f32_read_probe`` of the sweep build with G
  workgroups, a pure streaming read of the copy;
- ``reduce_sum_f32``: the deterministic sum of the copy;
- ``skinny_8x8192x8192``: gemm_f32 with the copy as B (8192 x 8192) and an
  8 x 8192 A;
- ``skinny_16x8192x8192_bt``: gemm_f32_ex with the copy as B stored
  transposed and a 16 x 8192 A.

Each line gives the median time, the algorithmic bytes over it, and that rate
as a fraction of the 8 TB/s nominal peak and of the fastest read probe.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import statistics
import time

PEAK_HBM_GBS = 8000.0
N_FLOATS = 1 << 26
COPIES = 4


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0)
    args = ap.parse_args(argv)

    import torch
    from dense_fp32_gemm_f32_amd import binding, build_lib, inputs

    lib = binding.load(build_lib.SWEEP_LIB)
    lib.gemm_f32_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.gemm_f32_read_probe.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    xs = [inputs.draw_matrix(1, N_FLOATS, "u11", 1400 + c).reshape(-1).to(dev)
          for c in range(COPIES)]
    n = 8192
    a8 = inputs.draw_matrix(8, n, "u11", 1500).to(dev)
    a16 = inputs.draw_matrix(16, n, "u11", 1501).to(dev)
    out = torch.empty(8 * 1024, device=dev)
    c8 = torch.empty((8, n), device=dev)
    c16 = torch.empty((16, n), device=dev)
    red = torch.empty(1, device=dev)

    def probe(groups):
        def f(i):
            rc = lib.gemm_f32_read_probe(xs[i % COPIES].data_ptr(), N_FLOATS, groups,
                                         out.data_ptr(), s)
            if rc != 0:
                raise binding.GemmError(rc, "gemm_f32_read_probe")
        return f

    bytes_read = 4.0 * N_FLOATS
    cands = [(f"read_probe_g{g}", probe(g), bytes_read) for g in (256, 512, 1024)]
    cands.append(("reduce_sum_f32", lambda i: binding.reduce_sum(xs[i % COPIES], red),
                  bytes_read))
    cands.append(("skinny_8x8192x8192",
                  lambda i: binding.gemm(a8, xs[i % COPIES].view(n, n), c8),
                  bytes_read + 4.0 * 2 * 8 * n))
    cands.append(("skinny_16x8192x8192_bt",
                  lambda i: binding.gemm_ex(a16, xs[i % COPIES].view(n, n), c16, trans_b=True),
                  bytes_read + 4.0 * 2 * 16 * n))

    rows = []
    for name, fn, algo in cands:
        i = 0
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        evs = []
        for _ in range(args.reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i)
            b.record(stream)
            i += 1
            evs.append((a, b))
        torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)
        rows.append({"call": name, "median_us": round(us, 2),
                     "GBps": round(algo / (us * 1e-6) / 1e9, 1)})
    best = max(r["GBps"] for r in rows if r["call"].startswith("read_probe"))
    for r in rows:
        r["of_peak"] = round(r["GBps"] / PEAK_HBM_GBS, 4)
        r["of_read_probe"] = round(r["GBps"] / best, 4)
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
