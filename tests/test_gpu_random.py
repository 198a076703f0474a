"""A seeded random sweep through the C ABI.

Shapes, pitches, layouts, alpha, beta, bias and ReLU are drawn from a fixed
generator. Every case runs on the dispatcher's kernel and is compared bit for
bit with the oracle. The inputs are integers, and so are alpha, beta, the
input C and the bias, so every partial sum is an exact binary32 integer
(|value| stays far below 2^24).

The mix covers the skinny-M path, mid-size grids (K split over workgroups or
over the waves of a workgroup) and many-tile grids, each in all four layouts.
A second sweep keeps M, N and the pitches multiples of 4 and K a multiple of
32, the conditions under which the dispatcher takes the kernels with direct
global-to-LDS loads, plain and transposed.  A third draws strided batches.
"""
import random

import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = 50
ALIGNED_CASES = 24
BATCH_CASES = 12


def _stored(X, trans, pad):
    S = X.t().contiguous() if trans else X.contiguous()
    return inputs.embed(S, S.shape[1] + pad)[:, :S.shape[1]]


def _draw(rng):
    kind = rng.random()
    if kind < 0.3:      # skinny M
        M, N, K = rng.randint(1, 16), rng.randint(1, 6000), rng.randint(1, 8000)
    elif kind < 0.6:    # mid-size grids
        M, N, K = rng.randint(17, 600), rng.randint(1, 600), rng.randint(1, 3000)
    else:               # many tiles
        M, N, K = rng.randint(64, 1200), rng.randint(64, 1200), rng.randint(1, 1000)
    ta, tb = rng.random() < 0.3, rng.random() < 0.3
    pads = (rng.choice([0, 0, 1, 3, 4]), rng.choice([0, 0, 1, 2, 4]), rng.choice([0, 1, 5]))
    alpha = rng.choice([1.0, 1.0, 2.0, -1.0, 0.0])
    beta = rng.choice([0.0, 0.0, 1.0, -2.0])
    bias = rng.random() < 0.3
    act = 1 if rng.random() < 0.3 else 0
    return M, N, K, ta, tb, pads, alpha, beta, bias, act


def _draw_aligned(rng):
    M, N = 4 * rng.randint(5, 400), 4 * rng.randint(5, 600)
    K = 32 * rng.randint(1, 32)
    ta, tb = rng.random() < 0.5, rng.random() < 0.5
    pads = (rng.choice([0, 4, 8]), rng.choice([0, 4, 12]), rng.choice([0, 1, 5]))
    alpha = rng.choice([1.0, 2.0, -1.0])
    beta = rng.choice([0.0, 1.0, -2.0])
    return M, N, K, ta, tb, pads, alpha, beta, rng.random() < 0.3, 1 if rng.random() < 0.3 else 0


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(gpu_lib, case):
    rng = random.Random(9100 + case)
    _check_case(gpu_lib, case, 9200 + 10 * case, *_draw(rng))


@pytest.mark.parametrize("case", range(ALIGNED_CASES))
def test_random_aligned_case(gpu_lib, case):
    rng = random.Random(9600 + case)
    kname = _check_case(gpu_lib, 1000 + case, 9700 + 10 * case, *_draw_aligned(rng))
    assert "_d6_" in kname, kname


def _check_case(gpu_lib, case, seed, M, N, K, ta, tb, pads, alpha, beta, with_bias, act):
    A, B = inputs.make_ab(M, N, K, "int2", "int2", seed)
    As, Bs = _stored(A, ta, pads[0]), _stored(B, tb, pads[1])
    ldc = N + pads[2]
    Cd, flat = H.sentinel_output(M, N, ldc)
    Cin = None
    if beta != 0:
        Cin = inputs.int_matrix(M, N, seed + 7, -5, 5)
        Cd.copy_(Cin.to("cuda"))
    bias = inputs.int_matrix(1, N, seed + 11, -9, 9).reshape(-1) if with_bias else None
    plain = not (ta or tb or with_bias or act) and alpha == 1.0 and beta == 0.0
    dA, dB = H.to_device(As), H.to_device(Bs)
    kname = (gpu_lib.selected_kernel(dA, dB, Cd) if plain else
             gpu_lib.selected_kernel_ex(dA, dB, Cd, trans_a=ta, trans_b=tb, alpha=alpha,
                                        beta=beta))
    H.say(f"random {case}: M={M} N={N} K={K} trans={int(ta)}{int(tb)} pads={pads} "
          f"alpha={alpha} beta={beta} bias={with_bias} act={act} kernel={kname}")
    if plain:
        gpu_lib.gemm(dA, dB, Cd)
    else:
        gpu_lib.gemm_fused(dA, dB, Cd, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta,
                           bias=None if bias is None else bias.cuda(), act=act)
    torch.cuda.synchronize()
    C_ref, _, _ = oracle.gemm_fused(As.numpy(), Bs.numpy(), trans_a=ta, trans_b=tb,
                                    alpha=alpha, beta=beta,
                                    C_in=None if Cin is None else Cin.numpy(),
                                    bias=None if bias is None else bias.numpy(), act=act)
    H.assert_bitexact(Cd.cpu().numpy(), C_ref, f"random case {case} ({kname})")
    H.check_outside_untouched(flat, M, N, ldc)
    return kname


@pytest.mark.parametrize("case", range(BATCH_CASES))
def test_random_batched_case(gpu_lib, case):
    rng = random.Random(9400 + case)
    batch = rng.randint(1, 40)
    M, N, K = rng.randint(1, 300), rng.randint(1, 300), rng.randint(1, 600)
    g = torch.Generator().manual_seed(9500 + case)
    A = torch.randint(-2, 3, (batch, M, K), generator=g).float()
    B = torch.randint(-2, 3, (batch, K, N), generator=g).float()
    dA, dB = A.cuda(), B.cuda()
    H.say(f"random batched {case}: batch={batch} M={M} N={N} K={K} "
          f"kernel={gpu_lib.selected_kernel_batched(dA, dB)}")
    C = gpu_lib.gemm_batched(dA, dB)
    torch.cuda.synchronize()
    C_ref, _, _ = oracle.gemm_batched(A.numpy(), B.numpy())
    H.assert_bitexact(C.cpu().numpy(), C_ref, f"random batched case {case}")
