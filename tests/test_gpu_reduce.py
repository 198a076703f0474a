"""GPU parity of the deterministic sum (``reduce_sum_f32``) against the CPU
oracle's ``sum_f32``, through the C ABI.

Gates: bit-exact on integer inputs whose every contiguous partial sum stays
below 2^24 in magnitude (checked on the data); |s - s_ref| <= 1e-4 * sum|x|
on fp32 inputs (the kernel's summation depth bounds its error by 1.7e-5 *
sum|x| up to n = 2^26); the same bits on every rerun and at any alignment of
x; +0.0 for the empty sum; IEEE NaN / Inf propagation.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

N_FULL = 2 ** 26   # the pages' reduction size


def _vector(n, dist, seed):
    if n == 0:
        return torch.zeros(0)
    return inputs.draw_matrix(1, n, dist, seed).reshape(-1)


def _device(x, offset=0):
    """Device copy of x starting `offset` floats into a NaN-guarded buffer."""
    buf = torch.full((x.numel() + offset + 4,), float("nan"))
    buf[offset:offset + x.numel()] = x
    d = buf.cuda()
    return d[offset:offset + x.numel()]


def _gpu_sum(lib, xd):
    out = torch.full((1,), float("nan"), device="cuda")
    lib.reduce_sum(xd, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()[0]


@pytest.mark.parametrize("n", [1, 3, 4, 5, 255, 1000, 16383, 16384, 16385, 65537,
                               2 ** 20 + 3, N_FULL])
@pytest.mark.parametrize("dist", ["u11", "normal"])
def test_sum_float(gpu_lib, n, dist):
    x = _vector(n, dist, 9500 + n % 1000)
    H.say(f"reduce float n={n} dist={dist}")
    s = _gpu_sum(gpu_lib, _device(x))
    ref, sd, ab = oracle.sum_f32(x.numpy())
    assert np.isfinite(s)
    err = abs(float(s) - sd)
    assert err <= 1e-4 * ab, f"n={n}: |{s} - {sd}| = {err} > 1e-4 * {ab}"
    print(f"n={n} {dist}: |ds| / sum|x| = {err / ab:.2e}")


@pytest.mark.parametrize("n", [7, 16385, 2 ** 20 + 1, N_FULL])
def test_sum_integer_bitexact(gpu_lib, n):
    x = inputs.int_matrix(1, n, 9600 + n % 1000).reshape(-1)
    prefix = np.concatenate([[0], np.cumsum(x.numpy().astype(np.int64))])
    # Exactness holds if every intermediate sum is an integer below 2^24.  A
    # workgroup sums one contiguous chunk of at most max(16388, n / 256 + 4)
    # elements of magnitude <= 2, and the second pass adds at most 256 chunk
    # sums, each bounded by the range of the prefix sums.
    assert 2 * max(16388, n // 256 + 4) < 2 ** 24
    assert 256 * (prefix.max() - prefix.min()) < 2 ** 24, "pick another seed"
    H.say(f"reduce integer n={n}")
    s = _gpu_sum(gpu_lib, _device(x))
    ref, _, _ = oracle.sum_f32(x.numpy())
    assert s == ref, f"n={n}: gpu {s} != oracle {ref}"


@pytest.mark.parametrize("n", [1001, 2 ** 20 + 7])
def test_sum_same_bits_any_alignment_and_rerun(gpu_lib, n):
    x = _vector(n, "normal", 9700)
    H.say(f"reduce alignment n={n}")
    got = [_gpu_sum(gpu_lib, _device(x, off)) for off in (0, 1, 2, 3, 4, 0)]
    assert len({g.tobytes() for g in got}) == 1, got


def test_sum_empty_is_positive_zero(gpu_lib):
    H.say("reduce n=0")
    s = _gpu_sum(gpu_lib, torch.zeros(0, device="cuda"))
    assert s == 0 and not np.signbit(s)


def test_sum_special_values(gpu_lib):
    x = _vector(100000, "u11", 9800)
    for pos, val, want in [(77777, float("nan"), "nan"), (5, float("inf"), "inf"),
                           (99999, float("-inf"), "-inf")]:
        y = x.clone()
        y[pos] = val
        H.say(f"reduce special {want}")
        s = _gpu_sum(gpu_lib, _device(y))
        if want == "nan":
            assert np.isnan(s)
        else:
            assert s == float(want)
    y = x.clone()
    y[10], y[90000] = float("inf"), float("-inf")
    assert np.isnan(_gpu_sum(gpu_lib, _device(y)))


def _int_vector(n, seed):
    x = inputs.int_matrix(1, n, seed).reshape(-1)
    prefix = np.concatenate([[0], np.cumsum(x.numpy().astype(np.int64))])
    assert 256 * (prefix.max() - prefix.min()) < 2 ** 24, "pick another seed"
    return x


def test_sum_and_exchange_kernels_share_the_slots(gpu_lib):
    """The sum's groups hand their partials to group 0 through the per-stream
    exchange slots that the skinny kernel's K slices also use.  Sums of several
    sizes and skinny products in turn on one stream: every call must find the
    slots clear and leave them clear, so every result matches the oracle
    (integer data: bit-exact)."""
    s = torch.cuda.Stream()
    A, B = inputs.make_ab(8, 4096, 4096, "int2", "int2", 9900)
    C_ref, _, _ = oracle.gemm(A.numpy(), B.numpy())
    Ad, Bd = A.cuda(), B.cuda()
    torch.cuda.synchronize()
    for rep, n in enumerate([N_FULL, 5000, 2 ** 20 + 3, 16385, 2 ** 22]):
        x = _int_vector(n, 9910 + rep)
        xd = _device(x)
        out = torch.full((1,), float("nan"), device="cuda")
        C = torch.full((8, 4096), float("nan"), device="cuda")
        H.say(f"reduce and skinny on one stream n={n}")
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            gpu_lib.reduce_sum(xd, out)
            gpu_lib.run_kernel("skinnyx_w8_c2_u2_s0_vec", Ad, Bd, C)
            gpu_lib.reduce_sum(xd, out)
        torch.cuda.synchronize()
        ref, _, _ = oracle.sum_f32(x.numpy())
        assert out.cpu().numpy()[0] == ref, f"n={n}"
        H.assert_bitexact(C.cpu().numpy(), C_ref, f"skinny after reduce n={n}")


def test_sum_in_graph_replays(gpu_lib):
    """reduce_sum_f32 captured into a HIP graph: each replay, with new data
    copied into the captured input and eager sums of other sizes on the same
    stream between replays, gives the eager result bit for bit."""
    n = 2 ** 22
    s = torch.cuda.Stream()
    xd = torch.empty(n, device="cuda")
    out = torch.full((1,), float("nan"), device="cuda")
    other = _device(_int_vector(70000, 9930))
    other_out = torch.empty(1, device="cuda")
    xd.copy_(_int_vector(n, 9940))
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_lib.reduce_sum(xd, out)   # the stream's slots exist before capture
    torch.cuda.synchronize()
    H.say("reduce graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gpu_lib.reduce_sum(xd, out)
    torch.cuda.synchronize()
    for rep in range(3):
        x = _int_vector(n, 9950 + rep)
        xd.copy_(x)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        H.say(f"reduce graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()[0]
        ref, _, _ = oracle.sum_f32(x.numpy())
        assert got == ref, f"replay {rep}: {got} != {ref}"
        with torch.cuda.stream(s):
            gpu_lib.reduce_sum(other, other_out)
        torch.cuda.synchronize()
