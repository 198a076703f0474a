"""The host-side C ABI code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library is rebuilt with both sanitizers on its host pass and
tests/test_abi_host.py runs against it in a subprocess with the sanitizer
runtime preloaded.  The argument checks do the pitch, extent and alias
arithmetic that these sanitizers watch."""
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.slow


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists(
    "/opt/rocm/bin/hipcc"), reason="needs the HIP compiler")
def test_host_tests_clean_under_sanitizers():
    from dense_fp32_gemm_f32_amd import sanitize_host
    lib = sanitize_host.build()
    syms = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report" in syms, "the host code is not instrumented"
    rc, out = sanitize_host.run(lib)
    assert rc == 0, out[-4000:]
    assert " passed" in out
