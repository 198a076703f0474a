"""GPU parity of the extended operation C = alpha * op(A) op(B) + beta * C
(``gemm_f32_ex``) against the CPU oracle's ``gemm_ex``, through the C ABI.

Gates as for the plain product: bit-exact on integer inputs (with integer
alpha and beta), |C - C_ref| <= 1e-4 * (|alpha| sum|a||b| + |beta c|) on fp32
inputs, nothing written outside the M x N window, and with beta = 0 the input
C (NaN here) is not read.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _stored(X, trans, pad):
    """CPU view of the stored operand (X or X^T) with `pad` extra floats of
    NaN pitch padding."""
    S = X.t().contiguous() if trans else X.contiguous()
    return inputs.embed(S, S.shape[1] + pad)[:, :S.shape[1]]


def _case(lib, M, N, K, ta, tb, alpha, beta, integer, seed, kernel=None, pads=(3, 5, 7)):
    dist = "int2" if integer else "u11"
    A, B = inputs.make_ab(M, N, K, dist, dist, seed)
    As, Bs = _stored(A, ta, pads[0]), _stored(B, tb, pads[1])
    ldc = N + pads[2]
    Cd, flat = H.sentinel_output(M, N, ldc)
    if beta != 0:
        Cin = (inputs.int_matrix(M, N, seed + 7, -5, 5) if integer
               else inputs.uniform_matrix(M, N, seed + 7))
        Cd.copy_(Cin.to("cuda"))
    else:
        Cin = None        # C keeps its NaN sentinel: it must not be read
    H.say(f"ex {kernel or 'dispatch'} M={M} N={N} K={K} trans={int(ta)}{int(tb)} "
          f"alpha={alpha} beta={beta} int={integer}")
    lib.gemm_ex(H.to_device(As), H.to_device(Bs), Cd, trans_a=ta, trans_b=tb, alpha=alpha,
                beta=beta, kernel=kernel)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    C_ref, _, ABS = oracle.gemm_ex(As.numpy(), Bs.numpy(), trans_a=ta, trans_b=tb,
                                   alpha=alpha, beta=beta,
                                   C_in=None if Cin is None else Cin.numpy())
    what = f"{kernel} {M}x{N}x{K} trans={int(ta)}{int(tb)} alpha={alpha} beta={beta}"
    if integer:
        H.assert_bitexact(C, C_ref, what)
    else:
        H.assert_within_tol(C, C_ref, ABS, what)
    H.check_outside_untouched(flat, M, N, ldc)


def _ex_kernels():
    """The kernels built for the extended operation: the MFMA ones in every
    layout, and the skinny-M ones built for a transposed layout."""
    try:
        from dense_fp32_gemm_f32_amd import binding
        return [n for n in binding.kernel_names()
                if n.startswith("mfmaex_") or n.endswith(("_tn", "_nt", "_tt"))]
    except Exception:  # library not built: the fixture fails the test loudly
        return ["<library missing>"]


def _shapes_for(kname):
    if kname.startswith("skinnyr_"):
        # N a multiple of 4 (whole float4 row runs), ending inside a wave's
        # columns; K split into slices, then too short to split
        mr = 4 * int([t for t in kname.split("_") if t.endswith("x4")][0][1:-2])
        return [(mr - 1, 1004, 2057), (min(mr, 3), 132, 21)]
    if kname.startswith(("skinnytl_", "skinnytc_")):
        # B^T's pitch K + 3 a multiple of 4 (copies into LDS need 16-byte
        # rows); a K % 256 remainder; few columns, so K is split; a short K
        return [(16, 1003, 2057), (5, 37, 8201), (16, 4100, 333)]
    if kname.startswith("skinnytm_"):
        # ragged N and K (a K % 16 tail); few columns, so K is split over
        # workgroups; M = 16 with many columns and a short K
        return [(16, 1003, 2057), (5, 37, 8200), (16, 4100, 333)]
    if kname.startswith("skinnyt_m"):
        mr = int(kname.split("_")[1][1:])
        # ragged N and K; the second shape has few columns, so K is split
        return [(min(mr, 7), 1003, 2057), (mr, 37, 8200)]
    if kname.startswith("skinny"):
        return [(13, 1003, 2057), (3, 130, 777)]
    if "_d6_" in kname:
        # direct-to-LDS loads: K a multiple of the K-tile, M and N multiples of
        # 4; ragged edges in M and N; one K-tile, two and several
        return [(300, 268, 192), (132, 68, 32), (68, 260, 64)]
    # ragged edges in M, N and K; M, N not multiples of 4 (element-wise edge
    # loads of a transposed operand); long enough for the branch-free loop
    return [(301, 263, 139), (130, 70, 333)]


@pytest.mark.parametrize("kname", _ex_kernels())
def test_every_ex_kernel(gpu_lib, kname):
    lay = kname.rsplit("_", 1)[-1][-2:]
    ta, tb = lay[0] == "t", lay[1] == "t"
    # skinnyr kernels need B's pitch a multiple of 4; direct-to-LDS kernels
    # both pitches
    pads = ((3, 4, 7) if kname.startswith("skinnyr_") else
            (3, 3, 7) if kname.startswith(("skinnytl_", "skinnytc_")) else
            (4, 8, 7) if "_d6_" in kname else (3, 5, 7))
    for (M, N, K) in _shapes_for(kname):
        _case(gpu_lib, M, N, K, ta, tb, 2.0, -1.0, True, 7001, kernel=kname, pads=pads)
        _case(gpu_lib, M, N, K, ta, tb, 1.0, 0.0, True, 7002, kernel=kname, pads=pads)
        _case(gpu_lib, M, N, K, ta, tb, 1.5, 0.5, False, 7003, kernel=kname, pads=pads)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(512, 512, 512), (1000, 999, 777), (8, 1024, 2048),
                                   (16, 300, 1000), (1, 1, 1), (5, 3, 2), (257, 129, 64)])
def test_ex_through_dispatcher(gpu_lib, ta, tb, shape):
    M, N, K = shape
    _case(gpu_lib, M, N, K, ta, tb, -2.0, 3.0, True, 7100 + M)
    _case(gpu_lib, M, N, K, ta, tb, 0.75, 0.0, False, 7200 + M)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_ex_plain_matches_gemm_f32_bitwise(gpu_lib, ta, tb):
    """alpha = 1, beta = 0, no transpose: gemm_f32_ex runs what gemm_f32 runs;
    with a transposed operand it agrees with gemm_f32 on the transposed copy to
    the parity bar (and exactly on integers)."""
    M, N, K = 384, 320, 256
    A, B = inputs.make_ab(M, N, K, "int2", "int2", 7300)
    H.say(f"ex plain vs gemm trans={int(ta)}{int(tb)}")
    Ad, Bd = A.cuda(), B.cuda()
    C0 = gpu_lib.gemm(Ad, Bd)
    As = Ad.t().contiguous() if ta else Ad
    Bs = Bd.t().contiguous() if tb else Bd
    C1 = gpu_lib.gemm_ex(As, Bs, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)


@pytest.mark.parametrize("beta", [0.0, 2.5])
def test_ex_k_zero_scales_c(gpu_lib, beta):
    M, N = 33, 70
    H.say(f"ex K=0 beta={beta}")
    A = torch.zeros((M, 0), device="cuda")
    B = torch.zeros((0, N), device="cuda")
    Cin = inputs.uniform_matrix(M, N, 7400)
    C = Cin.cuda() if beta != 0 else torch.full((M, N), float("nan"), device="cuda")
    gpu_lib.gemm_ex(A, B, C, alpha=3.0, beta=beta)
    torch.cuda.synchronize()
    want = (np.float32(beta) * Cin.numpy()) if beta != 0 else np.zeros((M, N), np.float32)
    assert np.array_equal(C.cpu().numpy(), want)


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_ex_full_size(gpu_lib, ta, tb, integer):
    """4096^3 with an operand stored transposed (the kernels bench.py times
    for nt, tn and tt), alpha and beta: every element against the oracle.
    The oracle runs on the logical operands as stored untransposed; its pins
    show that the transposed storage gives the same bits (C, sums and
    magnitudes), and this keeps its reads sequential at this size.  Integer
    inputs with integer alpha and beta: bit-exact."""
    w = inputs.WORKLOADS["square_4096"]
    A, B = inputs.workload_inputs(w, integer=integer)
    if integer:
        Cin = inputs.int_matrix(w.M, w.N, 7502, -5, 5)
        alpha, beta = 2.0, -1.0
    else:
        Cin = inputs.uniform_matrix(w.M, w.N, 7500)
        alpha, beta = 1.25, -0.5
    H.say(f"ex 4096^3 trans={int(ta)}{int(tb)} int={integer}")
    Ad, Bd = A.cuda(), B.cuda()
    As = Ad.t().contiguous() if ta else Ad
    Bs = Bd.t().contiguous() if tb else Bd
    del Ad, Bd
    C = Cin.cuda()
    kname = gpu_lib.selected_kernel_ex(As, Bs, C, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta)
    assert "_d6_" in kname, kname   # the direct-to-LDS kernel the bench times
    gpu_lib.gemm_ex(As, Bs, C, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    del As, Bs, C
    C_ref, _, ABS = oracle.gemm_ex(A.numpy(), B.numpy(), alpha=alpha, beta=beta,
                                   C_in=Cin.numpy())
    what = f"{kname} 4096^3 trans={int(ta)}{int(tb)}"
    if integer:
        H.assert_bitexact(got, C_ref, what)
    else:
        ratio = H.assert_within_tol(got, C_ref, ABS, what)
        print(f"{what}: max |dC| / scale = {ratio:.3e}")


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("M,ta", [(8, False), (16, False), (16, True)])
def test_skinny_b_transposed_full_size(gpu_lib, M, ta, integer):
    """M x 8192 x 8192 with B stored transposed (the skinny shapes bench.py
    times, on the shared-ring kernel the dispatcher picks for K >= 8192), A
    stored as is or transposed: every element against the oracle, which runs
    on the logical operands.  Integer inputs: bit-exact."""
    N = K = 8192
    dist = "int2" if integer else "u11"
    A, B = inputs.make_ab(M, N, K, dist, dist, 7600 + M)
    H.say(f"ex skinny B^T {M}x{N}x{K} trans_a={int(ta)} int={integer}")
    Ad = A.t().contiguous().cuda() if ta else A.cuda()
    Bd = B.t().contiguous().cuda()
    C = torch.full((M, N), float("nan"), device="cuda")
    kname = gpu_lib.selected_kernel_ex(Ad, Bd, C, trans_a=ta, trans_b=True)
    assert kname.startswith("skinnytc_"), kname
    gpu_lib.gemm_ex(Ad, Bd, C, trans_a=ta, trans_b=True)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    C_ref, _, ABS = oracle.gemm_ex(A.numpy(), B.numpy())
    what = f"{kname} {M}x{N}x{K}"
    if integer:
        H.assert_bitexact(got, C_ref, what)
    else:
        ratio = H.assert_within_tol(got, C_ref, ABS, what)
        print(f"{what}: max |dC| / scale = {ratio:.3e}")


@pytest.mark.parametrize("ta", [False, True])
@pytest.mark.parametrize("shape", [(16, 1000, 8200), (5, 4100, 8448), (16, 40, 16400),
                                   (3, 8300, 8196)])
def test_skinny_b_transposed_long_k_dispatch(gpu_lib, ta, shape):
    """B stored transposed with K >= 8192 through the dispatcher (the ring
    kernels, 16 waves above N = 8192): ragged N, a K % 256 tail, few columns
    (K split into slices), with alpha and beta; pitches padded to multiples
    of 4.  8 waves for M <= 8 up to N = 8192, else 16."""
    M, N, K = shape
    A, B = inputs.make_ab(M, N, K, "int2", "int2", 7650)
    As = (A.t().contiguous() if ta else A).cuda()
    Bs = H.to_device(_stored(B, True, 4))
    kname = gpu_lib.selected_kernel_ex(As, Bs, trans_a=ta, trans_b=True)
    assert kname.startswith("skinnytc_w16" if N > 8192 or M > 8 else "skinnytc_w8"), kname
    _case(gpu_lib, M, N, K, ta, True, -2.0, 3.0, True, 7700 + M, pads=(3, 4, 7))
    _case(gpu_lib, M, N, K, ta, True, 0.75, 0.0, False, 7800 + M, pads=(3, 4, 7))
