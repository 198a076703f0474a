"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (they call the HIP library
through its C ABI); everything else runs on the CPU.
"""
import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once.  Fails loudly if it is missing or no GPU
    is visible: a GPU test must never pass on a fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    from dense_fp32_gemm_f32_amd import binding
    binding.load()
    return binding
