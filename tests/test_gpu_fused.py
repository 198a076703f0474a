"""GPU parity of the fused epilogue C = act(alpha * op(A) op(B) + beta * C +
bias) (``gemm_f32_fused``) against the CPU oracle's ``gemm_fused``, through
the C ABI.

Gates as for the extended operation: bit-exact on integer inputs (integer
alpha, beta and bias), |C - C_ref| <= 1e-4 * (|alpha| sum|a||b| + |beta c| +
|bias|) on fp32 inputs (ReLU is 1-Lipschitz, so the same scale holds after
it), nothing written outside the M x N window, and with beta = 0 the input C
(NaN here) is not read.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
RELU = 1


def _stored(X, trans, pad):
    S = X.t().contiguous() if trans else X.contiguous()
    return inputs.embed(S, S.shape[1] + pad)[:, :S.shape[1]]


def _case(lib, M, N, K, ta, tb, alpha, beta, act, integer, seed, kernel=None, pads=(3, 5, 7),
          with_bias=True):
    dist = "int2" if integer else "u11"
    A, B = inputs.make_ab(M, N, K, dist, dist, seed)
    As, Bs = _stored(A, ta, pads[0]), _stored(B, tb, pads[1])
    ldc = N + pads[2]
    Cd, flat = H.sentinel_output(M, N, ldc)
    Cin = None
    if beta != 0:
        Cin = (inputs.int_matrix(M, N, seed + 7, -5, 5) if integer
               else inputs.uniform_matrix(M, N, seed + 7))
        Cd.copy_(Cin.to("cuda"))
    bias = None
    if with_bias:
        bias = (inputs.int_matrix(1, N, seed + 11, -9, 9) if integer
                else inputs.uniform_matrix(1, N, seed + 11)).reshape(-1)
    H.say(f"fused {kernel or 'dispatch'} M={M} N={N} K={K} trans={int(ta)}{int(tb)} "
          f"alpha={alpha} beta={beta} act={act} bias={with_bias} int={integer}")
    lib.gemm_fused(H.to_device(As), H.to_device(Bs), Cd, trans_a=ta, trans_b=tb, alpha=alpha,
                   beta=beta, bias=None if bias is None else bias.cuda(), act=act, kernel=kernel)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    C_ref, _, ABS = oracle.gemm_fused(As.numpy(), Bs.numpy(), trans_a=ta, trans_b=tb,
                                      alpha=alpha, beta=beta,
                                      C_in=None if Cin is None else Cin.numpy(),
                                      bias=None if bias is None else bias.numpy(), act=act)
    what = f"{kernel} {M}x{N}x{K} trans={int(ta)}{int(tb)} alpha={alpha} beta={beta} act={act}"
    if integer:
        H.assert_bitexact(C, C_ref, what)
    else:
        H.assert_within_tol(C, C_ref, ABS, what)
    H.check_outside_untouched(flat, M, N, ldc)


def _fused_kernels():
    """Every kernel that takes an epilogue: the extended-operation MFMA kernels
    and the skinny-M kernels, each in the layout it was built for."""
    try:
        from dense_fp32_gemm_f32_amd import binding
        return [n for n in binding.kernel_names()
                if n.startswith("mfmaex_") or n.startswith("skinny")]
    except Exception:  # library not built: the fixture fails the test loudly
        return ["<library missing>"]


def _layout_of(kname):
    if kname.startswith("mfmaex_") or kname.endswith(("_tn", "_nt", "_tt", "_nn")):
        lay = kname.rsplit("_", 1)[-1]
        return lay[0] == "t", lay[1] == "t"
    return False, False


def _shapes_for(kname):
    if kname.startswith("skinnyr_"):
        mr = 4 * int([t for t in kname.split("_") if t.endswith("x4")][0][1:-2])
        return [(mr - 1, 1004, 2057), (min(mr, 3), 132, 21)], (3, 4, 7)
    if kname.startswith("skinnyt_m"):
        mr = int(kname.split("_")[1][1:])
        return [(min(mr, 7), 1003, 2057), (mr, 37, 8200)], (3, 5, 7)
    if kname.startswith(("skinnytl_", "skinnytc_")):
        # B^T's pitch K + 3 a multiple of 4 (its rows are copied into LDS)
        return [(13, 1003, 2057), (16, 37, 8201)], (3, 3, 7)
    if kname.startswith("skinny"):
        return [(13, 1003, 2057), (3, 130, 777)], (3, 5, 7)
    if "_d6_" in kname:
        # direct-to-LDS loads: K a multiple of the K-tile, M, N and the pitches
        # of A and B multiples of 4
        return [(300, 268, 192), (132, 68, 64)], (4, 8, 7)
    return [(301, 263, 139), (130, 70, 333)], (3, 5, 7)


@pytest.mark.parametrize("kname", _fused_kernels())
def test_every_fused_kernel(gpu_lib, kname):
    ta, tb = _layout_of(kname)
    shapes, pads = _shapes_for(kname)
    for (M, N, K) in shapes:
        _case(gpu_lib, M, N, K, ta, tb, 2.0, -1.0, RELU, True, 7601, kernel=kname, pads=pads)
        _case(gpu_lib, M, N, K, ta, tb, 1.5, 0.5, RELU, False, 7603, kernel=kname, pads=pads)
    M, N, K = shapes[0]
    _case(gpu_lib, M, N, K, ta, tb, -1.0, 0.0, 0, True, 7605, kernel=kname, pads=pads)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(512, 512, 512), (1000, 999, 777), (8, 1024, 2048),
                                   (16, 300, 1000), (1, 1, 1), (5, 3, 2)])
def test_fused_through_dispatcher(gpu_lib, ta, tb, shape):
    M, N, K = shape
    _case(gpu_lib, M, N, K, ta, tb, -2.0, 3.0, RELU, True, 7700 + M)
    _case(gpu_lib, M, N, K, ta, tb, 0.75, 0.0, RELU, False, 7800 + M)
    _case(gpu_lib, M, N, K, ta, tb, 1.0, 0.0, 0, False, 7900 + M, with_bias=True)


@pytest.mark.parametrize("act", [0, RELU])
def test_fused_k_zero(gpu_lib, act):
    """K == 0: the epilogue of an empty sum, act(beta * C + bias)."""
    M, N = 33, 70
    H.say(f"fused K=0 act={act}")
    A = torch.zeros((M, 0), device="cuda")
    B = torch.zeros((0, N), device="cuda")
    Cin = inputs.uniform_matrix(M, N, 7950)
    bias = inputs.uniform_matrix(1, N, 7951).reshape(-1)
    C = Cin.cuda()
    gpu_lib.gemm_fused(A, B, C, alpha=3.0, beta=2.5, bias=bias.cuda(), act=act)
    torch.cuda.synchronize()
    want, _, _ = oracle.gemm_fused(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32),
                                   alpha=3.0, beta=2.5, C_in=Cin.numpy(), bias=bias.numpy(),
                                   act=act)
    # two fp32 roundings (beta * c, then + bias) against the oracle's one
    got = C.cpu().numpy()
    scale = np.abs(2.5 * Cin.numpy().astype(np.float64)) + np.abs(bias.numpy())[None, :]
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-6 * scale)


def test_fused_no_bias_no_act_is_gemm_ex(gpu_lib):
    M, N, K = 384, 320, 256
    A, B = inputs.make_ab(M, N, K, "u11", "u11", 7960)
    Cin = inputs.uniform_matrix(M, N, 7961).cuda()
    H.say("fused vs ex bitwise")
    Ad, Bd = A.cuda(), B.cuda()
    C1 = Cin.clone()
    C2 = Cin.clone()
    gpu_lib.gemm_ex(Ad, Bd, C1, alpha=1.25, beta=-0.5)
    gpu_lib.gemm_fused(Ad, Bd, C2, alpha=1.25, beta=-0.5)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_fused_full_size(gpu_lib):
    """4096^3 with alpha, beta, bias and ReLU: every element against the oracle."""
    w = inputs.WORKLOADS["square_4096"]
    A, B = inputs.workload_inputs(w)
    Cin = inputs.uniform_matrix(w.M, w.N, 7970)
    bias = inputs.uniform_matrix(1, w.N, 7971).reshape(-1)
    H.say("fused 4096^3")
    C = Cin.cuda()
    gpu_lib.gemm_fused(A.cuda(), B.cuda(), C, alpha=1.25, beta=-0.5, bias=bias.cuda(), act=RELU)
    torch.cuda.synchronize()
    C_ref, _, ABS = oracle.gemm_fused(A.numpy(), B.numpy(), alpha=1.25, beta=-0.5,
                                      C_in=Cin.numpy(), bias=bias.numpy(), act=RELU)
    ratio = H.assert_within_tol(C.cpu().numpy(), C_ref, ABS, "fused 4096^3")
    print(f"fused 4096^3: max |dC| / scale = {ratio:.3e}")


def _plain_kernels():
    """The tile kernels of the plain table (A and B as stored), whose store
    applies the epilogue (and, when K is split, the combine)."""
    try:
        from dense_fp32_gemm_f32_amd import binding
        return [n for n in binding.kernel_names() if n.startswith("mfma_")]
    except Exception:  # library not built: the fixture fails the test loudly
        return ["<library missing>"]


@pytest.mark.parametrize("kname", _plain_kernels())
def test_every_plain_kernel_with_epilogue(gpu_lib, kname):
    from tests.test_gpu_parity import _kernel_case
    M, N, K, lda, ldb = _kernel_case(kname)
    for integer, (alpha, beta, act, seed) in [(True, (2.0, -1.0, RELU, 7611)),
                                              (False, (1.5, 0.5, RELU, 7613))]:
        dist = "int2" if integer else "u11"
        A, B = inputs.make_ab(M, N, K, dist, dist, seed, lda=lda, ldb=ldb)
        ldc = N + 5
        Cd, flat = H.sentinel_output(M, N, ldc)
        Cin = (inputs.int_matrix(M, N, seed + 7, -5, 5) if integer
               else inputs.uniform_matrix(M, N, seed + 7))
        Cd.copy_(Cin.to("cuda"))
        bias = (inputs.int_matrix(1, N, seed + 11, -9, 9) if integer
                else inputs.uniform_matrix(1, N, seed + 11)).reshape(-1)
        H.say(f"fused plain kernel {kname} M={M} N={N} K={K} int={integer}")
        gpu_lib.gemm_fused(H.to_device(A), H.to_device(B), Cd, alpha=alpha, beta=beta,
                           bias=bias.cuda(), act=act, kernel=kname)
        torch.cuda.synchronize()
        C_ref, _, ABS = oracle.gemm_fused(A.numpy(), B.numpy(), alpha=alpha, beta=beta,
                                          C_in=Cin.numpy(), bias=bias.numpy(), act=act)
        if integer:
            H.assert_bitexact(Cd.cpu().numpy(), C_ref, kname)
        else:
            H.assert_within_tol(Cd.cpu().numpy(), C_ref, ABS, kname)
        H.check_outside_untouched(flat, M, N, ldc)
