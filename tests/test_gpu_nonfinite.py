"""NaN and Inf through every kernel of the table, through the C ABI.

The pages are silent on non-finite inputs; the reading taken is IEEE
propagation: a NaN or an infinity in row i of op(A) makes row i of C
non-finite, one in column j of op(B) makes column j non-finite, and nothing
else changes.  Several kernels read past-the-edge or padding positions at
clamped addresses, or prefetch past the end of a K range, and rely on
selecting exact zeros there; a zero chosen by multiplying instead would let a
NaN leak into a stored neighbour, and a masked element read as data would
lose one.  So each kernel runs one integer-valued product (bit-exact on
finite outputs) with:

  op(A)[M/2][K/3] = NaN     interior
  op(A)[M-1][K-1] = +Inf    last row, last k
  op(B)[0][N-1]   = NaN     last column, first k
  op(B)[K-1][N/3] = -Inf    last k

and the test asserts that exactly rows {M/2, M-1} and columns {N/3, N-1} of
C are non-finite, that the CPU oracle agrees on that set, that every other
element equals the oracle bit for bit, and that nothing outside the M x N
window of C is written.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _kernels():
    try:
        from dense_fp32_gemm_f32_amd import binding
        return binding.kernel_names()
    except Exception:  # library not built: the fixture fails the test loudly
        return ["<library missing>"]


def _layout(kname):
    """(trans_a, trans_b) a kernel is built for."""
    last = kname.rsplit("_", 1)[-1]
    if last in ("nt", "tn", "tt"):
        return last[0] == "t", last[1] == "t"
    return False, False


def _case(kname):
    """(M, N, K, pitch padding of the stored A and B) the kernel accepts, with
    ragged edges where it takes them."""
    if kname.startswith("skinnyr_"):
        return 7, 1004, 2057, (3, 4)        # B: N and pitch multiples of 4
    if kname.startswith("skinnyt_"):
        return 7, 1003, 2057, (3, 5)
    if kname.startswith(("skinnytl_", "skinnytc_")):
        return 13, 1003, 2057, (3, 3)      # B^T's pitch a multiple of 4
    if kname.startswith("skinnytm_"):
        return 13, 1003, 2057, (3, 5)
    if kname.startswith("skinnyx_"):
        return 13, 1003, 2057, (3, 5)
    if "_d6_" in kname:
        # direct-to-LDS loads: K a multiple of the K-tile, pitches multiples
        # of 4, M and N multiples of 4 (ragged against the tile)
        return 300, 264, 192, (4, 8)
    if kname.endswith("_small"):
        return 70, 50, 139, (3, 5)
    if kname == "ref_naive":
        return 45, 37, 29, (1, 3)
    return 301, 263, 139, (3, 5)            # register-staged tiles: any pitch


def _stored(X, trans, pad):
    S = X.t().contiguous() if trans else X.contiguous()
    return inputs.embed(S, S.shape[1] + pad)[:, :S.shape[1]]


@pytest.mark.parametrize("kname", _kernels())
def test_nonfinite_inputs_reach_exactly_their_rows_and_columns(gpu_lib, kname):
    ta, tb = _layout(kname)
    M, N, K, (pa, pb) = _case(kname)
    A, B = inputs.make_ab(M, N, K, "int2", "int2", 7700)
    A = A.contiguous().clone()
    B = B.contiguous().clone()
    rows = (M // 2, M - 1)
    cols = (N // 3, N - 1)
    A[M // 2, K // 3] = float("nan")
    A[M - 1, K - 1] = float("inf")
    B[0, N - 1] = float("nan")
    B[K - 1, N // 3] = float("-inf")
    As, Bs = _stored(A, ta, pa), _stored(B, tb, pb)
    ldc = N + 7
    C, flat = H.sentinel_output(M, N, ldc)
    H.say(f"nonfinite {kname} M={M} N={N} K={K} trans={int(ta)}{int(tb)}")
    if ta or tb:
        gpu_lib.gemm_ex(H.to_device(As), H.to_device(Bs), C, trans_a=ta, trans_b=tb,
                        kernel=kname)
    else:
        gpu_lib.run_kernel(kname, H.to_device(As), H.to_device(Bs), C)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    C_ref, _, _ = oracle.gemm(A.numpy(), B.numpy())

    want = np.zeros((M, N), dtype=bool)
    want[list(rows), :] = True
    want[:, list(cols)] = True
    assert np.array_equal(~np.isfinite(C_ref), want), "oracle: unexpected non-finite set"
    bad = ~np.isfinite(got) != want
    assert not bad.any(), (f"{kname}: {int(bad.sum())} elements finite where they should not "
                           f"be or the reverse, e.g. {np.argwhere(bad)[:4].tolist()}")
    H.assert_bitexact(np.where(want, 0.0, got).astype(np.float32),
                      np.where(want, 0.0, C_ref).astype(np.float32), kname)
    H.check_outside_untouched(flat, M, N, ldc)
