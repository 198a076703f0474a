"""Host-sanitizer build of the C ABI, for the CPU host tests.

The argument checks of the C ABI (overflow of pitch and extent arithmetic,
aliasing ranges, the kernel table and dispatcher) run on the host.  This
builds the library with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code only (device code is unchanged) and runs
``tests/test_abi_host.py`` against it in a subprocess with the sanitizer
runtime preloaded:

    python -m dense_fp32_gemm_f32_amd.sanitize_host

It needs no GPU: the host tests call only argument checks, the dispatcher and
the kernel table.  Exit status 0 means the tests passed and no sanitizer
report was printed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

from dense_fp32_gemm_f32_amd import build_lib

BUILD = build_lib.BUILD / "asan"
LIB = BUILD / "libgemm_f32_asan.so"

# Sanitizers on the host pass only: each -fsanitize follows -Xarch_host.
SAN = ["-O1", "-g", "-fno-omit-frame-pointer",
       "-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def runtime() -> str:
    """The shared AddressSanitizer runtime of the HIP compiler."""
    r = subprocess.run([build_lib.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build() -> Path:
    BUILD.mkdir(parents=True, exist_ok=True)
    srcs = build_lib.sources()
    common = [a for a in build_lib.COMMON if a != "-O3"]
    def one(src: Path) -> Path:
        obj = BUILD / (src.name + ".o")
        lang = ["-x", "hip"] if src.suffix == ".hip" else []
        cmd = [build_lib.HIPCC, *common, *SAN, *lang, "-c", str(src), "-o", str(obj)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stderr}")
        return obj
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, srcs))
    cmd = [build_lib.HIPCC, f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC",
           "-shared-libsan", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *map(str, objs), "-o", str(LIB)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    return LIB


def run(lib: Path) -> tuple[int, str]:
    """The host tests against the sanitized library; (exit status, output)."""
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "GEMM_F32_LIB": str(lib),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        str(build_lib.ROOT / "tests" / "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=build_lib.ROOT)
    out = r.stdout + r.stderr
    reported = "ERROR: AddressSanitizer" in out or "runtime error:" in out
    return (r.returncode if not reported else 1), out


if __name__ == "__main__":
    rc, out = run(build())
    print(out[-3000:])
    sys.exit(rc)
