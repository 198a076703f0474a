"""Where the time of one macro-tiled GEMM launch goes, workgroup by workgroup.

    python -m dense_fp32_gemm_f32_amd.build_lib --sweep        # once
    python -m dense_fp32_gemm_f32_amd.stamps --workload square_1024
    python -m dense_fp32_gemm_f32_amd.stamps --shape 4096x4096x4096 --kernel mfma_256x256x32_w64x128_d6_vec

Runs the tuning table's direct-to-LDS tile for the workload (or ``--kernel``)
through ``gemm_f32_stamped`` of the sweep library (``include/gemm_f32_sweep.h``):
an instrumented copy of the kernel whose workgroups stamp the 100 MHz counter
and the shader cycle counter at their start, after their K loop and after
their C stores.  After ``--settle-ms`` of load, the plain kernel is
event-timed (median of ``--reps`` calls, each bracketed by a HIP event pair on
the launch stream), then, after its own settle, the instrumented one is run
``--reps`` times back to back.  Prints one JSON line per instrumented run
with:

- ``start_spread_us``: first to last workgroup start;
- ``loop_us_mean`` / ``loop_us_max``: the K loop per workgroup;
- ``loop_us_by_xcd``: its mean over the workgroups of each XCD (launch index
  modulo 8);
- ``store_us_mean``: the C write-out per workgroup;
- ``span_us``: first start to last end;
- ``ghz``: shader cycles over wall time in the K loops (median workgroup);

and a closing line with the plain kernel's event-timed median, the medians of
the fields above over the runs, and whether the instrumented kernel's C is
bitwise the plain one's.  Synthetic inputs of the workload
(``inputs.WORKLOADS``), or U[-1, 1) for ``--shape``.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import statistics
import time


def _parse_shape(s: str):
    m, n, k = (int(x) for x in s.lower().split("x"))
    return m, n, k


NUM_XCD = 8   # MI355X deals workgroups to its 8 XCDs round-robin by launch index


def summarize(stamps, wall_khz: int) -> dict:
    """The fields above from a (workgroups x 6) integer tensor of stamps, row
    w for launch index w."""
    st = stamps.double()
    rt0, rt1, rt2, mt0, mt1, mt2 = st.unbind(1)
    us = 1e3 / wall_khz   # microseconds per tick of the constant counter
    t0 = rt0.min()
    loop = (rt1 - rt0) * us
    ghz = ((mt1 - mt0) / (rt1 - rt0)) * (wall_khz / 1e6)
    n = loop.numel() - loop.numel() % NUM_XCD
    by_xcd = loop[:n].view(-1, NUM_XCD).mean(0) if n else loop[:0]
    return {
        "start_spread_us": round(float((rt0.max() - t0) * us), 3),
        "loop_us_mean": round(float(loop.mean()), 3),
        "loop_us_max": round(float(loop.max()), 3),
        "loop_us_by_xcd": [round(float(x), 2) for x in by_xcd],
        "store_us_mean": round(float(((rt2 - rt1) * us).mean()), 3),
        "span_us": round(float((rt2.max() - t0) * us), 3),
        "ghz": round(float(ghz.median()), 4),
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="square_1024")
    ap.add_argument("--shape", default="", help="MxNxK with packed pitches instead of a workload")
    ap.add_argument("--kernel", default="", help="a mfma_*_d6_vec table entry (default: the "
                                                 "dispatcher's choice, which must be one)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0)
    args = ap.parse_args(argv)

    import torch
    from dense_fp32_gemm_f32_amd import binding, build_lib, inputs

    lib = binding.load(build_lib.SWEEP_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.gemm_f32_stamped.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp,
                                     i64, vp]
    lib.gemm_f32_stamped.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    if args.shape:
        M, N, K = _parse_shape(args.shape)
        a_cpu, b_cpu = inputs.make_ab(M, N, K, "u11", "u11", 9000)
        name = args.shape
    else:
        w = inputs.WORKLOADS[args.workload]
        M, N, K = w.M, w.N, w.K
        a_cpu, b_cpu = inputs.make_ab(M, N, K, w.dist_a, w.dist_b, w.seed)
        name = w.name
    A, B = a_cpu.to(dev), b_cpu.to(dev)
    C = torch.empty((M, N), device=dev)
    C_plain = torch.empty((M, N), device=dev)
    kname = args.kernel or binding.selected_kernel(A, B, C)
    idx = binding.kernel_index(kname)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    lda, ldb, ldc = A.stride(0), B.stride(0), C.stride(0)

    def plain(out):
        rc = binding.gemm_f32_run_kernel(idx, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                         out.data_ptr(), ldc, s)
        if rc != 0:
            raise binding.GemmError(rc, f"gemm_f32_run_kernel({kname})")

    # one stamp record (6 words) per workgroup, one workgroup per tile; one
    # row of records per instrumented run
    bm, bn = (int(x) for x in kname.split("_")[1].split("x")[:2])
    tiles = -(-M // bm) * -(-N // bn)
    words = 6 * tiles
    stamps = torch.zeros((args.reps, words), dtype=torch.int64, device=dev)

    def stamped(r):
        rc = lib.gemm_f32_stamped(idx, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                  C.data_ptr(), ldc, stamps[r].data_ptr(), words, s)
        if rc != 0:
            raise binding.GemmError(rc, f"gemm_f32_stamped({kname})")

    wall_khz = ctypes.c_int(0)
    probe = torch.zeros(4 * binding.CLOCK_PROBE_WORKGROUPS, dtype=torch.int64, device=dev)
    rc = binding.gemm_f32_clock_probe(1, probe.data_ptr(), ctypes.addressof(wall_khz), None, s)
    if rc != 0:
        raise binding.GemmError(rc, "gemm_f32_clock_probe")
    torch.cuda.synchronize()

    def settle(fn):
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    settle(lambda: plain(C_plain))
    evs = []
    for _ in range(args.reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plain(C_plain)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    plain_us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)

    # the instrumented runs back to back after their own settle, as the
    # plain calls were timed; each run stamps its own row
    settle(lambda: stamped(0))
    for r in range(args.reps):
        stamped(r)
    torch.cuda.synchronize()
    same = bool(torch.equal(C, C_plain))
    rows = []
    for r in range(args.reps):
        rec = summarize(stamps[r].view(-1, 6).cpu(), wall_khz.value)
        rec["run"] = r
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    keys = ["start_spread_us", "loop_us_mean", "loop_us_max", "store_us_mean", "span_us", "ghz"]
    med = {k: round(statistics.median(r[k] for r in rows), 3) for k in keys}
    med["loop_us_by_xcd"] = [round(statistics.median(r["loop_us_by_xcd"][x] for r in rows), 2)
                             for x in range(len(rows[0]["loop_us_by_xcd"]))]
    out = {"workload": name, "M": M, "N": N, "K": K, "kernel": kname, "workgroups": tiles,
           "plain_event_us_median": round(plain_us, 3),
           "median_over_runs": med,
           "same_as_plain": same}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
