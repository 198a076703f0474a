"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.

Gates: bit-exact on integer inputs in {-2..2}; |C - C_ref| <= 1e-4 *
sum_k |a_ik||b_kj| per element on fp32 inputs; nothing written outside the
M x N window of C; reruns bitwise identical.
"""
import numpy as np
import pytest
import torch

from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# the measured workloads, and one GPU's share of two of them split 8 ways
WORKLOADS = list(inputs.WORKLOADS) + list(inputs.SHARDS)


def _workload(name):
    return inputs.WORKLOADS[name] if name in inputs.WORKLOADS else inputs.SHARDS[name]


def _run(lib, A_cpu, B_cpu, ldc=None, kernel=None, ref=False, offsets=(0, 0, 0)):
    """Copy inputs to the GPU (keeping pitches), run, return (C numpy, flat, ldc)."""
    M, K = A_cpu.shape
    N = B_cpu.shape[1]
    A = H.to_device(A_cpu, offset=offsets[0])
    B = H.to_device(B_cpu, offset=offsets[1])
    ldc = N if ldc is None else ldc
    C, flat = H.sentinel_output(M, N, ldc, offset=offsets[2])
    if ref:
        lib.gemm_ref(A, B, C)
    elif kernel is not None:
        lib.run_kernel(kernel, A, B, C)
    else:
        lib.gemm(A, B, C)
    torch.cuda.synchronize()
    return C.cpu().numpy(), flat, ldc


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_float(gpu_lib, name):
    w = _workload(name)
    A, B = inputs.workload_inputs(w)
    H.say(f"float workload {name} kernel={gpu_lib.selected_kernel(A, B)}")
    C, flat, ldc = _run(gpu_lib, A, B, ldc=w.ldc)
    C_ref, ABS = H.oracle_of(A, B)
    ratio = H.assert_within_tol(C, C_ref, ABS, name)
    H.check_outside_untouched(flat, w.M, w.N, ldc)
    print(f"{name}: max |dC|/sum|a||b| = {ratio:.3e}")


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_integer_bitexact(gpu_lib, name):
    w = _workload(name)
    A, B = inputs.workload_inputs(w, integer=True)
    H.say(f"integer workload {name}")
    C, flat, ldc = _run(gpu_lib, A, B, ldc=w.ldc)
    C_ref, _ = H.oracle_of(A, B)
    H.assert_bitexact(C, C_ref, name)
    H.check_outside_untouched(flat, w.M, w.N, ldc)


@pytest.mark.parametrize("name", ["square_4096", "skinny_8x8192x8192", "ragged_2047x3001x1531"])
def test_rerun_bitwise_identical(gpu_lib, name):
    w = inputs.WORKLOADS[name]
    A_cpu, B_cpu = inputs.workload_inputs(w)
    H.say(f"rerun {name}")
    A, B = H.to_device(A_cpu), H.to_device(B_cpu)
    C1 = gpu_lib.gemm(A, B)
    C2 = gpu_lib.gemm(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def _kernel_case(name):
    """A shape and pitches the named kernel accepts, with ragged edges."""
    suffix = name.rsplit("_", 1)[-1]
    vec_a = suffix in ("vec", "veca")
    vec_b = suffix in ("vec", "vecb")
    if name.startswith("skinnyr_"):
        # whole float4 row runs of B: N and ldb multiples of 4; M one short of
        # the rows the kernel holds, N ending inside a wave's 256 columns, K
        # ending inside a quad of rows
        return _skinnyr_rows(name) - 1, 1004, 2057, 2058, 1008
    if name.startswith("skinny"):
        M, N, K = 13, 1000 + 3, 2050 + 7
    elif "_d4_" in name:
        # single-float direct copies: odd pitches, ragged M, N and K (K % 32
        # != 0: a padded first K-tile)
        return 301, 263, 139, 141, 265
    elif "_d6_" in name:
        # direct-to-LDS loads: N, K, lda, ldb multiples of 4 (K of 64), ragged M
        # and N edges; with "_sk_", a last K slice shorter than the others
        M, N, K = 301, 264, 64 * 25 if "_sk_" in name else 192
        return M, N, K, K + 4, N + 4
    elif "_sk_" in name:
        # long enough for several K slices at BK = 16 and 32, the last one
        # shorter and ending in a partial K-tile
        M, N, K = 301, 263, 32 * 8 * 3 + 13
    elif name.startswith("mfma"):
        M, N, K = 301, 263, 139
    else:
        M, N, K = 45, 37, 29
    lda = K + (4 - K % 4) % 4 + 4 if vec_a else K + 1
    ldb = N + (4 - N % 4) % 4 + 4 if vec_b else N + 3
    if name == "ref_naive":
        lda, ldb = K + 1, N + 3
    return M, N, K, lda, ldb


def _skinnyr_rows(name):
    """Rows of A a skinnyr_..._m<q>x4_... kernel holds (4 q)."""
    tok = [t for t in name.split("_") if t.startswith("m") and t.endswith("x4")][0]
    return 4 * int(tok[1:-2])


def _all_kernel_names():
    """Every kernel of the table except those built for a transposed layout
    (and the extended-operation MFMA kernels), which test_gpu_ex.py covers."""
    try:
        from dense_fp32_gemm_f32_amd import binding
        return [n for n in binding.kernel_names()
                if not n.startswith("mfmaex_") and not n.endswith(("_tn", "_nt", "_tt"))]
    except Exception:  # library not built: the fixture fails the test loudly
        return ["<library missing>"]


@pytest.mark.parametrize("kname", _all_kernel_names())
def test_every_kernel_variant(gpu_lib, kname):
    M, N, K, lda, ldb = _kernel_case(kname)
    cases = [(M, N, K, lda, ldb)]
    if kname.startswith("skinnyr_"):
        # K too short to split: one slice, written straight to C
        cases.append((M, N, 21, 24, ldb))
    if "_d4_" in kname:
        # K a multiple of the K-tile (no padded first tile), the shortest K
        # taken (two K-tiles), odd pitches
        bk = int(kname.split("_")[1].split("x")[2])
        cases += [(130, 70, 3 * bk, 3 * bk + 1, 73), (67, 200, 2 * bk, 2 * bk + 3, 201)]
        # one row, one column: every other row / column of the tile reads the
        # clamped last one
        cases += [(1, 3, 2 * bk + 5, 2 * bk + 6, 4), (70, 1, 5 * bk + 3, 5 * bk + 4, 2)]
    for (M, N, K, lda, ldb), integer in [(c, i) for c in cases for i in (True, False)]:
        dist = "int2" if integer else "u11"
        A, B = inputs.make_ab(M, N, K, dist, dist, 3001 + integer, lda=lda, ldb=ldb)
        H.say(f"kernel {kname} M={M} N={N} K={K} lda={lda} ldb={ldb} int={integer}")
        C, flat, ldc = _run(gpu_lib, A, B, ldc=N + 5, kernel=kname)
        C_ref, ABS = H.oracle_of(A, B)
        if integer:
            H.assert_bitexact(C, C_ref, kname)
        else:
            H.assert_within_tol(C, C_ref, ABS, kname)
        H.check_outside_untouched(flat, M, N, ldc)


@pytest.mark.parametrize("shape", [(33, 129, 2000), (512, 512, 512), (1, 64, 4096),
                                   (200, 70, 1031), (1024, 1024, 1024),
                                   # very deep K, and one-column / one-row products
                                   (40, 50, 300000), (64, 64, 262144), (1000, 1, 1000),
                                   (1, 1000, 5000), (17, 1, 70000)])
def test_split_k_through_dispatcher(gpu_lib, shape):
    """Grids too small to fill the GPU take the K-split MFMA path; its slice
    partials are summed in a fixed order, so reruns are bitwise identical."""
    M, N, K = shape
    for integer in (True, False):
        dist = "int2" if integer else "u11"
        A, B = inputs.make_ab(M, N, K, dist, dist, 6100 + integer)
        kname = gpu_lib.selected_kernel(A, B)
        H.say(f"split-K {shape} int={integer} kernel={kname}")
        C, flat, ldc = _run(gpu_lib, A, B, ldc=N + 3)
        C_ref, ABS = H.oracle_of(A, B)
        if integer:
            H.assert_bitexact(C, C_ref, f"{shape} {kname}")
        else:
            H.assert_within_tol(C, C_ref, ABS, f"{shape} {kname}")
        H.check_outside_untouched(flat, M, N, ldc)
        C2, _, _ = _run(gpu_lib, A, B, ldc=N + 3)
        assert np.array_equal(C, C2)


EDGE_SIZES = [1, 2, 3, 31, 33, 64, 127, 129, 257]


@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 129, 257])
@pytest.mark.parametrize("N", [1, 3, 64, 129, 255])
@pytest.mark.parametrize("K", [1, 2, 17, 130])
def test_edge_shapes(gpu_lib, M, N, K):
    A, B = inputs.make_ab(M, N, K, "int2", "int2", 4000 + M * 7 + N * 3 + K)
    H.say(f"edge M={M} N={N} K={K} kernel={gpu_lib.selected_kernel(A, B)}")
    C, flat, ldc = _run(gpu_lib, A, B, ldc=N + 2)
    C_ref, _ = H.oracle_of(A, B)
    H.assert_bitexact(C, C_ref, f"{M}x{N}x{K}")
    H.check_outside_untouched(flat, M, N, ldc)


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 2, 0), (3, 1, 1)])
@pytest.mark.parametrize("shape", [(200, 300, 100), (8, 1000, 700)])
def test_unaligned_base_pointers(gpu_lib, offs, shape):
    M, N, K = shape
    A, B = inputs.make_ab(M, N, K, "u11", "u11", 5001)
    H.say(f"unaligned offsets={offs} shape={shape}")
    C, flat, ldc = _run(gpu_lib, A, B, offsets=offs)
    C_ref, ABS = H.oracle_of(A, B)
    H.assert_within_tol(C, C_ref, ABS, f"unaligned {offs}")
    H.check_outside_untouched(flat, M, N, ldc, offset=offs[2])


def test_k_zero_writes_positive_zeros(gpu_lib):
    M, N = 37, 45
    A = torch.empty((M, 0), device="cuda")
    B = torch.empty((0, N), device="cuda")
    C, flat = H.sentinel_output(M, N, N + 3)
    H.say("K=0")
    gpu_lib.gemm(A, B, C)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    assert np.all(c == 0) and not np.signbit(c).any()
    H.check_outside_untouched(flat, M, N, N + 3)


def test_empty_output_is_noop(gpu_lib):
    A = torch.ones((0, 5), device="cuda")
    B = torch.ones((5, 7), device="cuda")
    C = torch.empty((0, 7), device="cuda")
    gpu_lib.gemm(A, B, C)
    A = torch.ones((4, 5), device="cuda")
    B = torch.ones((5, 0), device="cuda")
    C = torch.empty((4, 0), device="cuda")
    gpu_lib.gemm(A, B, C)
    torch.cuda.synchronize()


def test_identity_and_permutation_exact(gpu_lib):
    n = 300
    X = inputs.uniform_matrix(n, n, 6001)
    I = torch.eye(n)
    p = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    P = torch.zeros(n, n)
    P[torch.arange(n), p] = 1.0
    Xd, Id, Pd = X.cuda(), I.cuda(), P.cuda()
    H.say("identity / permutation")
    assert torch.equal(gpu_lib.gemm(Id, Xd).cpu(), X)
    assert torch.equal(gpu_lib.gemm(Xd, Id).cpu(), X)
    assert torch.equal(gpu_lib.gemm(Pd, Xd).cpu(), X[p])
    assert torch.equal(gpu_lib.gemm(Xd, Pd).cpu(), X[:, torch.argsort(p)])


@pytest.mark.parametrize("shape", [(33, 47, 29), (128, 130, 257), (8, 1024, 512)])
def test_reference_kernel(gpu_lib, shape):
    M, N, K = shape
    A, B = inputs.make_ab(M, N, K, "normal", "normal", 7001, lda=K + 3, ldb=N + 1)
    H.say(f"ref kernel {shape}")
    C, flat, ldc = _run(gpu_lib, A, B, ldc=N + 4, ref=True)
    C_ref, ABS = H.oracle_of(A, B)
    H.assert_within_tol(C, C_ref, ABS, "ref")
    H.check_outside_untouched(flat, M, N, ldc)


def test_page_pattern_on_gpu(gpu_lib):
    """The integer pattern of the 'GPU compute shaders' check (32 x 24 x 16)."""
    m, n, k = 32, 24, 16
    a = torch.tensor([(i % 7) - 3 for i in range(m * k)], dtype=torch.float32).reshape(m, k)
    b = torch.tensor([(i % 5) - 2 for i in range(k * n)], dtype=torch.float32).reshape(k, n)
    C = gpu_lib.gemm(a.cuda(), b.cuda()).cpu().numpy()
    C_ref, _ = H.oracle_of(a, b)
    H.assert_bitexact(C, C_ref, "page pattern")
    assert C[0, 0] == 11 and C[0, 1] == -4


def test_errors_from_the_device_side(gpu_lib):
    b = gpu_lib
    A = torch.ones((64, 64), device="cuda")
    B = torch.ones((64, 64), device="cuda")
    C = torch.empty((64, 64), device="cuda")
    host = torch.ones((64, 64))
    s = torch.cuda.current_stream().cuda_stream
    # host memory that the device cannot reach
    rc = b.gemm_f32(64, 64, 64, host.data_ptr(), 64, B.data_ptr(), 64, C.data_ptr(), 64, s)
    assert rc == 9
    # C aliasing A
    rc = b.gemm_f32(64, 64, 64, A.data_ptr(), 64, B.data_ptr(), 64, A.data_ptr(), 64, s)
    assert rc == 4
    # unknown kernel index, and a skinny kernel with too many rows
    assert b.gemm_f32_run_kernel(10 ** 6, 64, 64, 64, A.data_ptr(), 64, B.data_ptr(), 64,
                                 C.data_ptr(), 64, s) == 8
    sk = [i for i, n in enumerate(b.kernel_names()) if n.startswith("skinny")][0]
    assert b.gemm_f32_run_kernel(sk, 64, 64, 64, A.data_ptr(), 64, B.data_ptr(), 64,
                                 C.data_ptr(), 64, s) == 8
    torch.cuda.synchronize()


SPLITK = "skinnyr_c2_r4_u4_m2x4_s0_nn"   # a kernel that combines K slices in a workspace
SPLITX = "skinnyx_w8_c2_u2_s0_vec"  # a kernel that adds K slices through exchange slots


@pytest.mark.parametrize("kname", [SPLITK, SPLITX])
def test_workspace_failure_is_reported(gpu_lib, monkeypatch, kname):
    A = torch.ones((8, 4096), device="cuda")
    B = torch.ones((4096, 4096), device="cuda")
    C = torch.empty((8, 4096), device="cuda")
    idx = gpu_lib.kernel_index(kname)
    monkeypatch.setenv("GEMM_F32_TEST_FAIL_WORKSPACE", "1")
    s = torch.cuda.current_stream().cuda_stream
    rc = gpu_lib.gemm_f32_run_kernel(idx, 8, 4096, 4096, A.data_ptr(), 4096, B.data_ptr(),
                                     4096, C.data_ptr(), 4096, s)
    assert rc == 6
    monkeypatch.delenv("GEMM_F32_TEST_FAIL_WORKSPACE")
    gpu_lib.run_kernel(kname, A, B, C)
    torch.cuda.synchronize()
    assert torch.all(C == 4096)


@pytest.mark.parametrize("kname", [SPLITK, SPLITX])
def test_two_streams_concurrently(gpu_lib, kname):
    """Split-K calls on two streams use separate workspaces and both match."""
    A1, B1 = inputs.make_ab(8, 4096, 8192, "normal", "u11", 8001)
    A2, B2 = inputs.make_ab(6, 4096, 8192, "normal", "u11", 8002)
    dA1, dB1, dA2, dB2 = (t.cuda() for t in (A1, B1, A2, B2))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    H.say(f"two streams {kname}")
    with torch.cuda.stream(s1):
        C1 = gpu_lib.run_kernel(kname, dA1, dB1)
    with torch.cuda.stream(s2):
        C2 = gpu_lib.run_kernel(kname, dA2, dB2)
    torch.cuda.synchronize()
    for (A, B, C) in ((A1, B1, C1), (A2, B2, C2)):
        C_ref, ABS = H.oracle_of(A, B)
        H.assert_within_tol(C.cpu().numpy(), C_ref, ABS, "two streams")


def test_exchange_tree_shapes_in_sequence(gpu_lib):
    """The in-kernel sum of K slices through exchange slots, over trees of
    many shapes in a row on one stream: 1, 2, 3, 4, 5, 7, 16 and 128 slices
    (odd counts leave a node without a right child), the slot buffer growing
    and then reused by smaller trees.  A slot left full by one call would make
    a later call take the wrong branch, so every call is checked bit for bit
    on integers and rerun."""
    # (M, N, K): 64-column strips and slices = ceil(256 / strips), capped by
    # the 16-row super-blocks of K
    shapes = [(8, 64 * 256, 4096), (8, 64 * 128, 2048), (5, 64 * 86, 3000), (8, 64 * 64, 4096),
              (16, 64 * 52, 1600), (3, 64 * 37, 2100), (8, 1000, 8192), (7, 100, 40000),
              (8, 64 * 64, 4096), (1, 64 * 86, 333)]
    for i, (M, N, K) in enumerate(shapes):
        A, B = inputs.make_ab(M, N, K, "int2", "int2", 8300 + i)
        H.say(f"exchange tree M={M} N={N} K={K}")
        C1, flat, ldc = _run(gpu_lib, A, B, ldc=N + 1, kernel=SPLITX)
        C2, _, _ = _run(gpu_lib, A, B, ldc=N + 1, kernel=SPLITX)
        C_ref, _ = H.oracle_of(A, B)
        H.assert_bitexact(C1, C_ref, f"exchange {M}x{N}x{K}")
        assert np.array_equal(C1, C2)
        H.check_outside_untouched(flat, M, N, ldc)
