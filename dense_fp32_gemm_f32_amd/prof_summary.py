"""Summarise rocprofv3 output (CSV) for ``profiles/``.

    python -m dense_fp32_gemm_f32_amd.prof_summary \
        --workload square_4096 --kernel mfma_128x128x16_w64x64_veca \
        --match mfma_gemm_kernel --trace OUT/trace --fetch OUT/fetch --write OUT/write \
        [--sq OUT/sq] --command "..." --out profiles/mfma_gemm_square_4096.md

--trace: a ``--kernel-trace --stats`` run (durations are taken from its
per-dispatch trace, optionally leaving out the first --skip dispatches); --fetch / --write: ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs of ``prof_workload`` (which ends with a copy of known
size); --sq: an optional run with SQ/GRBM counters.  HBM bytes per launch are
the kernel's FETCH_SIZE and WRITE_SIZE (KiB) scaled by the ratio of the copy's
known bytes to its own counter values.  The result is written as a short
markdown summary, and the per-launch bytes are recorded in
``profiles/traffic.json`` under the kernel's table name together with a hash of
the kernel sources (bench.py reports them only while the sources match).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
from collections import defaultdict
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_sources(kernel: str | None = None) -> list[str]:
    """The source files a table kernel is compiled from (every source when
    the name is unknown or None)."""
    csrc = ROOT / "dense_fp32_gemm_f32_amd" / "csrc"
    every = sorted(p.name for p in csrc.glob("*"))
    if not kernel:
        return every
    files = ["gemm_f32_internal.h"]
    if kernel.startswith("mfmaex_"):
        files += (["kernels_mfma_ex_dma.hip", "lds_dma.h"] if "_d6_" in kernel else
                  ["kernels_mfma_ex.hip"]) + ["mfma_common.h"]
    elif kernel.startswith("mfma_"):
        if "_d4_" in kernel:
            files += ["kernels_mfma_dma4.hip"]
        elif "_kw" in kernel:
            files += ["kernels_mfma_dma_ks.hip", "lds_dma.h"]
        elif "_d6_" in kernel:
            files += ["kernels_mfma_dma.hip", "lds_dma.h", "stamps.h"]
        else:
            files += ["kernels_mfma.hip"]
        files += ["mfma_common.h"]
        if "_sk_" in kernel:
            files.append("kernels_combine.hip")
    elif kernel.startswith("skinnyr_"):
        files += ["kernels_skinny_rows.hip", "kernels_combine.hip"]
    elif kernel.startswith("skinnyt_"):
        files += ["kernels_skinny_t.hip", "kernels_combine.hip", "mfma_common.h"]
    elif kernel.startswith(("skinnytl_", "skinnytm_", "skinnytc_")):
        files += ["kernels_skinny_tm.hip", "kernels_combine.hip", "lds_dma.h", "mfma_common.h"]
    elif kernel.startswith("skinny_"):
        files += ["kernels_skinny.hip", "kernels_combine.hip"]
    elif kernel.startswith("skinnyx_"):
        files += ["kernels_skinny.hip"]
    elif kernel.startswith("reduce_"):
        files += ["kernels_reduce.hip"]
    else:
        return every
    return sorted(files)


def source_hash(kernel: str | None = None) -> str:
    """Hash of the sources a kernel is built from: profiles record it, and a
    recorded traffic figure is used only while the kernel's sources match."""
    h = hashlib.sha256()
    csrc = ROOT / "dense_fp32_gemm_f32_amd" / "csrc"
    for name in kernel_sources(kernel):
        h.update(name.encode())
        h.update((csrc / name).read_bytes())
    return h.hexdigest()


def _find(d: Path, suffix: str) -> Path:
    hits = sorted(Path(d).rglob(f"*{suffix}"))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def counters(d: Path):
    """{kernel name: {counter: [values per dispatch]}} from a --pmc run."""
    out = defaultdict(lambda: defaultdict(list))
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def durations(d: Path, skip: int = 0, last: int = 0):
    """{kernel name: (calls, avg ns, min ns, max ns)} from a --kernel-trace run,
    leaving out the first `skip` dispatches of each kernel (clock warm-up), or
    keeping only its `last` dispatches (after a settle phase of the run)."""
    per = defaultdict(list)
    with open(_find(d, "kernel_trace.csv")) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    res = {}
    for name, ds in per.items():
        if last:
            ds = ds[-last:]
        else:
            ds = ds[skip:] if len(ds) > skip else ds
        res[name] = (len(ds), sum(ds) / len(ds), min(ds), max(ds))
    return res


def pick(names, match):
    hits = [n for n in names if match in n]
    if not hits:
        raise KeyError(f"no kernel matching {match!r} in {list(names)}")
    return hits


def mean(v):
    return sum(v) / len(v)


def by_launch_shape(d: Path):
    """Per (kernel, grid) dispatch durations of a --kernel-trace run: one kernel
    template launched on several shapes (a 4096^3 product and a batch of
    512^3 products, say) gets one row per grid."""
    per = defaultdict(list)
    with open(_find(d, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], f'{r["Grid_Size_X"]}x{r["Grid_Size_Y"]}x{r["Grid_Size_Z"]}',
                   f'{r["Workgroup_Size_X"]}x{r["Workgroup_Size_Y"]}x{r["Workgroup_Size_Z"]}')
            per[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per


def bench_summary(trace: Path, commands, out: Path, skip: int = 0, bench_log: Path | None = None,
                  last: int = 0):
    """Markdown table of a bench.py kernel trace, split by launch shape; with
    skip, the first `skip` dispatches of each (kernel, grid) are left out (the
    warm-up steps); with last, only the last `last` are kept (the timed steps,
    after the settle and warm-up calls); with bench_log the JSON line the
    traced run printed is quoted so that its event-timed launch mean can be set
    beside the trace."""
    lines = ["# bench.py kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "Command (from the repository root on the MI355X box):", ""]
    lines += [f"    {c}" for c in commands] + [""]
    if last:
        what = (f"The last {last} dispatches of each kernel and grid (the timed steps; the "
                "settle and warm-up calls come before them)")
    elif skip:
        what = (f"Dispatches of the run after the first {skip} of each kernel and grid (the "
                "warm-up steps)")
    else:
        what = "Every dispatch of the run, warm-up included"
    lines += [what + ", grouped by kernel and grid (grid sizes in threads).", "",
              "| kernel | grid | workgroup | calls | avg us | min us | max us |",
              "|---|---|---|---|---|---|---|"]
    rows = sorted(by_launch_shape(trace).items(), key=lambda kv: -sum(kv[1]))
    for (name, grid, wg), ds in rows:
        if "gemmf32" not in name:
            continue
        if last:
            ds = ds[-last:]
        elif len(ds) > skip:
            ds = ds[skip:]
        short = name.replace("gemmf32::(anonymous namespace)::", "").replace("void ", "")
        short = short.split("(")[0]
        lines.append(f"| `{short}` | {grid} | {wg} | {len(ds)} | {sum(ds) / len(ds) / 1e3:.2f} "
                     f"| {min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")
    if bench_log is not None:
        rec = None
        for line in Path(bench_log).read_text().splitlines():
            if line.startswith("{") and '"metric"' in line:
                rec = json.loads(line)
        if rec is not None:
            r = rec.get("roofline", {})
            lines += ["", "The same run's bench.py line (HIP events around each timed launch):", "",
                      f"- kernel `{rec['config'].get('kernel')}`, {rec['steps']} timed steps after "
                      f"{rec['warmup']} warm-up steps",
                      f"- launch_ms_mean {r.get('launch_ms_mean')}, launch_ms_min "
                      f"{r.get('launch_ms_min')}, achieved {r.get('achieved')} {r.get('unit')} "
                      f"(frac {r.get('frac')})"]
            t = rec.get("timing") or {}
            if t:
                lines.append(f"- settle {t.get('settle_s')} s ({t.get('settle_calls')} calls); "
                             f"first and last quarter of the timed launches "
                             f"{t.get('first_quarter_ms_mean')} / {t.get('last_quarter_ms_mean')} ms")
                for key in ("clock_ghz_before_settle", "clock_ghz_after_timed"):
                    c = t.get(key)
                    if c:
                        lines.append(f"- {key}: median {c.get('median')} (min {c.get('min')}, "
                                     f"max {c.get('max')})")
    Path(out).write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--bench-trace", help="summarise a bench.py --kernel-trace run instead")
    ap.add_argument("--bench-log", help="with --bench-trace: the traced run's output")
    ap.add_argument("--workload")
    ap.add_argument("--kernel", help="table name of the kernel")
    ap.add_argument("--match", help="substring of the rocprof kernel name(s)")
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--sq")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--skip", type=int, default=0,
                    help="leave out the first SKIP dispatches of each kernel from the durations")
    ap.add_argument("--last", type=int, default=0,
                    help="keep only the last LAST dispatches of each kernel (instead of --skip)")
    ap.add_argument("--algo-bytes", type=float, default=0.0)
    ap.add_argument("--flops", type=float, default=0.0)
    ap.add_argument("--mfma-cycles", type=int, default=0,
                    help="cycles one MFMA of the kernel occupies the pipe (32x32x2 f32: 64)")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--log", help="stdout of the trace run (for its clock-probe line)")
    ap.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.bench_trace:
        bench_summary(Path(args.bench_trace), args.command, Path(args.out), args.skip,
                      Path(args.bench_log) if args.bench_log else None, args.last)
        return
    if not (args.workload and args.kernel and args.match and args.trace):
        ap.error("--workload, --kernel, --match and --trace are required")

    lines = [f"# {args.kernel} on {args.workload}", ""]
    lines += ["Commands (from the repository root on the MI355X box):", ""]
    lines += [f"    {c}" for c in args.command] + [""]

    dur = durations(Path(args.trace), args.skip, args.last)
    names = pick(dur, args.match)
    which = (f"the last {args.last} dispatches of each kernel (after the run's clock-settle "
             "phase)" if args.last else
             f"leaving out the first {args.skip} dispatches of each kernel (clock warm-up)")
    lines += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              f"Durations from the trace, {which}.", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    tot_avg = 0.0
    for n in names:
        calls, avg, mn, mx = dur[n]
        tot_avg += avg
        lines.append(f"| `{n[:110]}` | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    rate = f"{args.flops / (tot_avg * 1e-9) / 1e12:.2f} TFLOP/s, " if args.flops > 0 else ""
    lines += ["", f"Sum of average durations of the matched kernels: {tot_avg / 1e3:.2f} us "
              f"-> {rate}{args.algo_bytes / (tot_avg * 1e-9) / 1e9:.1f} GB/s of algorithmic "
              "traffic", ""]
    if args.log:
        probe = [l.strip() for l in Path(args.log).read_text().splitlines()
                 if l.startswith("clock probe:")]
        if probe:
            lines += [f"Shader clock right after the traced launches, same run "
                      f"(gemm_f32_clock_probe: s_memtime over the 100 MHz s_memrealtime across "
                      f"about 1 ms of fp32 MFMA load): {probe[-1][len('clock probe: '):]}", ""]

    traffic = None
    if args.fetch and args.write:
        fc, wc = counters(Path(args.fetch)), counters(Path(args.write))
        cf = mean(fc[COPY_KERNEL]["FETCH_SIZE"]) * 1024.0
        cw = mean(wc[COPY_KERNEL]["WRITE_SIZE"]) * 1024.0
        f_scale, w_scale = args.copy_bytes / cf, args.copy_bytes / cw
        fetch = sum(mean(fc[n]["FETCH_SIZE"]) for n in pick(fc, args.match)) * 1024.0 * f_scale
        write = sum(mean(wc[n]["WRITE_SIZE"]) for n in pick(wc, args.match)) * 1024.0 * w_scale
        traffic = fetch + write
        lines += ["## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
                  f"Calibration copy of {args.copy_bytes} bytes: FETCH_SIZE reads "
                  f"{cf:.0f} B (scale {f_scale:.3f}), WRITE_SIZE reads {cw:.0f} B "
                  f"(scale {w_scale:.3f}).", "",
                  "| per launch | bytes | x algorithmic |", "|---|---|---|",
                  f"| fetched (scaled) | {fetch:.4g} | {fetch / args.algo_bytes:.3f} |",
                  f"| written (scaled) | {write:.4g} | {write / args.algo_bytes:.3f} |",
                  f"| total | {traffic:.4g} | {traffic / args.algo_bytes:.3f} |",
                  f"| algorithmic 4(MK+KN+MN) | {args.algo_bytes:.4g} | 1 |", ""]

    if args.sq:
        sc = counters(Path(args.sq))
        n = pick(sc, args.match)[0]
        c = {k: mean(v) for k, v in sc[n].items()}
        lines += ["## Core counters (first matched kernel, mean per dispatch)", "",
                  "| counter | value |", "|---|---|"]
        lines += [f"| {k} | {v:.6g} |" for k, v in sorted(c.items())]
        dur = durations(Path(args.trace), args.skip, args.last)
        long_enough = n in dur and dur[n][1] >= 200e3
        if "SQ_INSTS_MFMA" in c and args.mfma_cycles and n in dur:
            util = c["SQ_INSTS_MFMA"] * args.mfma_cycles / (dur[n][1] * 2.4 * 1024.0)
            lines += ["", f"MFMA issue over the traced duration at the 2.4 GHz peak clock = "
                      f"SQ_INSTS_MFMA x {args.mfma_cycles} cycles / (avg duration x 2.4 GHz x "
                      f"1024 SIMDs) = {100 * util:.1f}%"]
        if "GRBM_GUI_ACTIVE" in c and not long_enough:
            lines += ["", "(Clock and MFMA-occupancy figures are derived only for launches of "
                      "200 us or more: on shorter ones GRBM_GUI_ACTIVE also counts the "
                      "counter collection around the dispatch.)"]
        if "GRBM_GUI_ACTIVE" in c and long_enough:
            # Both terms of each ratio below come from the same counter run.  No
            # clock is derived here: GRBM_GUI_ACTIVE comes from the counter run
            # and the duration from the trace run, two different launches.
            xcd_cycles = c["GRBM_GUI_ACTIVE"] / 8.0     # summed over the 8 XCDs
            lines.append("")
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
            if busy is not None and busy < 2.0 ** 31 * 0.999:
                util = busy / (xcd_cycles * 1024.0)
                lines.append(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs) "
                             f"= {100 * util:.1f}%")
            elif busy is not None:
                lines.append("SQ_VALU_MFMA_BUSY_CYCLES reads 2^31 (the counter saturates on launches "
                             "this long); see the issue-based figure instead.")
            if "SQ_INSTS_MFMA" in c and args.mfma_cycles:
                util = c["SQ_INSTS_MFMA"] * args.mfma_cycles / (xcd_cycles * 1024.0)
                lines.append(f"MFMA pipe occupancy from issue = SQ_INSTS_MFMA x {args.mfma_cycles} "
                             f"cycles / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs) = {100 * util:.1f}%")
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
            lines += [f"LDS bank-conflict cycles / LDS active cycles = "
                      f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f}"]
        lines.append("")

    Path(args.out).write_text("\n".join(lines) + "\n")
    if traffic is not None:
        tf = ROOT / "profiles" / "traffic.json"
        rec = json.loads(tf.read_text()) if tf.exists() else {}
        rec[args.kernel] = {"workload": args.workload, "hbm_bytes_per_launch": round(traffic),
                            "algo_bytes": args.algo_bytes,
                            "source_sha256": source_hash(args.kernel),
                            "summary": str(Path(args.out).name)}
        tf.write_text(json.dumps(rec, indent=1, sort_keys=True) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
