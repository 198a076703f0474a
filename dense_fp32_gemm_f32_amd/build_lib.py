"""Build ``libgemm_f32.so`` for gfx950 with hipcc, in-tree.

Each source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into ``dense_fp32_gemm_f32_amd/libgemm_f32.so``.
Run as ``python -m dense_fp32_gemm_f32_amd.build_lib``.
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
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of the device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{ROOT / 'include'}"]


def sources():
    return sorted([*CSRC.glob("*.hip"), *CSRC.glob("*.cpp")])


def _compile(src: Path, extra: list[str]) -> Path:
    obj = BUILD / (src.name + ".o")
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


def build(extra: list[str] | None = None, jobs: int | None = None) -> Path:
    """Compile every source and link the shared library.  Always rebuilds."""
    extra = list(extra or [])
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
