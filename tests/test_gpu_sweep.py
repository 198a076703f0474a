"""GPU checks of the sweep build's measurement calls (``include/gemm_f32_sweep.h``):

- ``gemm_f32_stamped``: the instrumented tile computes bitwise what the plain
  kernel computes (and matches the oracle exactly on integer inputs), and
  every workgroup's stamps are ordered in time;
- ``gemm_f32_read_probe``: it reads exactly the elements it is meant to (the
  per-wave sums it writes, on integer data, against a host computation).

Skipped when the sweep library has not been built."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import build_lib, inputs

pytestmark = pytest.mark.gpu

i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int


@pytest.fixture(scope="module")
def sweep():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    if not build_lib.SWEEP_LIB.exists():
        pytest.skip("the sweep library is not built (python -m dense_fp32_gemm_f32_amd.build_lib --sweep)")
    lib = ctypes.CDLL(str(build_lib.SWEEP_LIB))
    lib.gemm_f32_stamped.argtypes = [ci, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.gemm_f32_stamped.restype = ci
    lib.gemm_f32_run_kernel.argtypes = [ci, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.gemm_f32_run_kernel.restype = ci
    lib.gemm_f32_read_probe.argtypes = [vp, i64, ci, vp, vp]
    lib.gemm_f32_read_probe.restype = ci
    lib.gemm_f32_kernel_count.restype = ci
    lib.gemm_f32_kernel_name.argtypes = [ci]
    lib.gemm_f32_kernel_name.restype = ctypes.c_char_p
    names = [lib.gemm_f32_kernel_name(i).decode() for i in range(lib.gemm_f32_kernel_count())]
    return lib, names


CASES = [
    ("mfma_64x64x32_w32x32_d6_vec", 1024, 1024, 1024),
    ("mfma_64x64x32_w32x32_d6_vec", 200, 328, 96),      # ragged M and N edge tiles
    ("mfma_256x256x32_w64x128_d6_vec", 512, 768, 64),
    ("mfma_128x192x32_w32x96_d6_vec", 300, 400, 128),
]


@pytest.mark.parametrize("kname,M,N,K", CASES)
def test_stamped_kernel_matches_plain_and_oracle(sweep, kname, M, N, K):
    lib, names = sweep
    idx = names.index(kname)
    a, b = inputs.make_ab(M, N, K, "int2", "int2", 8100 + M)
    A, B = a.cuda(), b.cuda()
    C = torch.full((M, N), float("nan"), device="cuda")
    C_plain = torch.full((M, N), float("nan"), device="cuda")
    bm, bn = (int(x) for x in kname.split("_")[1].split("x")[:2])
    tiles = -(-M // bm) * -(-N // bn)
    stamps = torch.zeros(6 * tiles, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    print(f"stamped {kname} {M}x{N}x{K}", flush=True)
    assert lib.gemm_f32_run_kernel(idx, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                   C_plain.data_ptr(), N, s) == 0
    assert lib.gemm_f32_stamped(idx, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                stamps.data_ptr(), 6 * tiles, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(C, C_plain)
    ref, _, _ = oracle.gemm(a.numpy(), b.numpy(), want_f64=False)
    assert np.array_equal(C.cpu().numpy(), ref)
    st = stamps.view(tiles, 6).cpu()
    rt, mt = st[:, :3], st[:, 3:]
    assert bool((rt[:, 0] > 0).all())
    assert bool((rt[:, 0] <= rt[:, 1]).all()) and bool((rt[:, 1] <= rt[:, 2]).all())
    assert bool((mt[:, 0] < mt[:, 1]).all()) and bool((mt[:, 1] <= mt[:, 2]).all())


def test_stamped_argument_errors(sweep):
    lib, names = sweep
    M = N = K = 256
    A = torch.zeros(M, K, device="cuda")
    B = torch.zeros(K, N, device="cuda")
    C = torch.zeros(M, N, device="cuda")
    stamps = torch.zeros(6 * 16, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    d6 = names.index("mfma_64x64x32_w32x32_d6_vec")   # 16 tiles at 256^2
    args = (M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)
    # not a direct-to-LDS tile entry
    other = next(i for i, n in enumerate(names) if not n.endswith("_d6_vec"))
    assert lib.gemm_f32_stamped(other, *args, stamps.data_ptr(), 96, s) == 8   # BAD_KERNEL
    assert lib.gemm_f32_stamped(-1, *args, stamps.data_ptr(), 96, s) == 8
    assert lib.gemm_f32_stamped(d6, *args, None, 96, s) == 3                  # NULL_PTR
    assert lib.gemm_f32_stamped(d6, *args, stamps.data_ptr(), 95, s) == 1     # INVALID_DIM
    assert lib.gemm_f32_stamped(d6, *args, stamps.data_ptr() + 4, 90, s) == 9 # POINTER
    # K not a multiple of the tile's K-tile: the entry does not take it
    assert lib.gemm_f32_stamped(d6, M, N, 100, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                stamps.data_ptr(), 96, s) == 8
    torch.cuda.synchronize()


@pytest.mark.parametrize("groups,pieces", [(4, 37), (256, 16), (3, 8), (1, 1)])
def test_read_probe_reads_its_pattern(sweep, groups, pieces):
    """Lane 0 of wave w in workgroup g adds floats 0..3 of 1 KiB pieces w,
    w + 8, ... of chunk g; small integers make every sum exact."""
    lib, _ = sweep
    chunk = 256 * pieces
    n = groups * chunk
    x = torch.from_numpy(np.random.default_rng(8200 + groups).integers(-8, 9, n).astype(np.float32))
    out = torch.full((8 * groups,), float("nan"), device="cuda")
    print(f"read probe {groups} groups x {pieces} pieces", flush=True)
    assert lib.gemm_f32_read_probe(x.cuda().data_ptr(), n, groups, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    xv = x.numpy().astype(np.float64).reshape(groups, pieces, 256)[:, :, :4].sum(axis=2)
    want = np.zeros((groups, 8))
    for w in range(8):
        want[:, w] = xv[:, w::8].sum(axis=1)
    assert np.array_equal(out.cpu().numpy().reshape(groups, 8), want.astype(np.float32))
