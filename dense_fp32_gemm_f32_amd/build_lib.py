"""Build ``libgemm_f32.so`` for gfx950 with hipcc, in-tree.

Each source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into ``dense_fp32_gemm_f32_amd/libgemm_f32.so``.
Run as ``python -m dense_fp32_gemm_f32_amd.build_lib``.

``--sweep`` builds ``libgemm_f32_sweep.so`` instead: the same sources with
``-DGEMM_F32_SWEEP=1``, whose kernel table also holds the variants that
tuning sweeps (``tune.py --sweep``) compare the tuned kernels with.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libgemm_f32.so"
SWEEP_LIB = PKG / "libgemm_f32_sweep.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of the device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{ROOT / 'include'}"]


def sources():
    return sorted([*CSRC.glob("*.hip"), *CSRC.glob("*.cpp")])


def _compile(src: Path, extra: list[str], build_dir: Path) -> Path:
    obj = build_dir / (src.name + ".o")
    lang = ["-x", "hip"] if src.suffix == ".hip" else []
    cmd = [HIPCC, *COMMON, *extra, *lang, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip():
        # hipcc's host pass warns about the device-only target feature; keep other warnings
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l
                 and "not a recognized feature" not in l and l.strip()]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(extra: list[str] | None = None, jobs: int | None = None, sweep: bool = False) -> Path:
    """Compile every source and link the shared library (the sweep library when
    ``sweep``).  Always rebuilds."""
    extra = list(extra or [])
    lib = LIB
    build_dir = BUILD
    if sweep:
        extra.append("-DGEMM_F32_SWEEP=1")
        lib = SWEEP_LIB
        build_dir = BUILD / "sweep"
    build_dir.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    sweep = "--sweep" in args
    print(build([a for a in args if a != "--sweep"], sweep=sweep))
