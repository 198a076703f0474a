"""gemm_f32_noalloc, the entry point that takes its scratch from a fixed array
in the library instead of allocating, against gemm_f32 through the C ABI.

Both run the same kernel on the same inputs, so the results must agree bit for
bit; each is also held to the parity gates against the CPU oracle (bit-exact
on integer inputs, |C - C_ref| <= 1e-4 * sum|a||b| on fp32 inputs).  Two calls
in a row, the second with a smaller input, reuse the array: the exchange
slots must be left empty by the first for the second to be right.
"""
import numpy as np
import pytest
import torch

from dense_fp32_gemm_f32_amd import binding, inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# (M, N, K) pairs: a first call, then a smaller one
PAIRS = [
    # K slices added through the exchange slots (8 x 8192 x 8192: 2 slices,
    # 1 MiB of slots), then 16 waves per workgroup and 16 slices
    ((8, 8192, 8192), (5, 1000, 3001)),
    # K slices added by the combine dispatch from the partial-sum region
    # (7.3 MB), then a shorter K with fewer slices
    ((8, 28672, 4096), (4, 20480, 1000)),
    # no scratch at all (MFMA tiles), then the slots again
    ((300, 520, 260), (3, 70, 40)),
]


def _check(lib, M, N, K, dist_a, dist_b, seed, integer):
    A_cpu, B_cpu = inputs.make_ab(M, N, K, dist_a, dist_b, seed)
    A, B = A_cpu.cuda(), B_cpu.cuda()
    kname = lib.selected_kernel(A, B)
    H.say(f"noalloc {M}x{N}x{K} int={integer} kernel={kname}")
    C0 = lib.gemm(A, B)
    C1, flat = H.sentinel_output(M, N)
    lib.gemm_noalloc(A, B, C1)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1), f"{kname}: gemm_f32_noalloc differs from gemm_f32"
    H.check_outside_untouched(flat, M, N, N)
    C_ref, ABS = H.oracle_of(A_cpu, B_cpu)
    c = C1.cpu().numpy()
    if integer:
        H.assert_bitexact(c, C_ref, f"noalloc {kname}")
    else:
        H.assert_within_tol(c, C_ref, ABS, f"noalloc {kname}")


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm_f32_two_calls(gpu_lib, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        _check(gpu_lib, M, N, K, "normal", "u_inv_sqrt_k", 9100 + 10 * i + M, False)
        _check(gpu_lib, M, N, K, "int2", "int2", 9200 + 10 * i + M, True)


def test_noalloc_rejects_beyond_its_scratch(gpu_lib):
    """8 x 24576 x 65536 would need 100 MB of partial sums: refused with
    GEMM_F32_ERR_SCRATCH before anything is enqueued (C untouched)."""
    M, N, K = 8, 24576, 65536
    A = torch.zeros((M, K), device="cuda")
    B = torch.empty((K, N), device="cuda")   # never read: the call is refused
    C, flat = H.sentinel_output(M, N)
    H.say(f"noalloc refuses {M}x{N}x{K}")
    rc = binding.gemm_f32_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 11, binding.STATUS_NAMES.get(rc, rc)
    assert np.all(np.isnan(flat.cpu().numpy()))
