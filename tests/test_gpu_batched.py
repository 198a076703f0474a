"""GPU parity of the strided batch (``gemm_f32_batched``) against the CPU
oracle's ``gemm_batched``, and of calls captured into a HIP graph against the
same calls run eagerly, through the C ABI.

Gates as for one product: bit-exact on integer inputs, |C - C_ref| <= 1e-4 *
sum|a||b| per element on fp32 inputs, nothing written outside the products'
M x N windows (NaN sentinels between and around them), reruns and graph
replays bitwise identical to eager calls.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_fp32_gemm_f32_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _stack(batch, rows, cols, dist, seed):
    """batch x rows x cols float32 CPU tensor of seeded draws."""
    return torch.stack([inputs.draw_matrix(rows, cols, dist, seed + b) for b in range(batch)])


def _device_batch(X, pitch, stride, shared=False):
    """Device copy of X (batch x rows x cols) with row pitch `pitch` and batch
    stride `stride` (elements) inside a NaN buffer; `shared` stores only X[0]
    and gives it batch stride 0."""
    bt, rows, cols = X.shape
    n = 1 if shared else bt
    if not shared and pitch == cols and stride == rows * cols:
        d = torch.cat([X.reshape(-1), torch.full((8,), float("nan"))]).cuda()
        return torch.as_strided(d, (bt, rows, cols), (stride, pitch, 1))
    flat = torch.full((max(n - 1, 0) * stride + rows * pitch + 8,), float("nan"))
    for b in range(n):
        for r in range(rows):
            flat[b * stride + r * pitch: b * stride + r * pitch + cols] = X[b, r]
    d = flat.cuda()
    return torch.as_strided(d, (bt, rows, cols), (0 if shared else stride, pitch, 1))


def _c_buffer(bt, M, N, ldc, sc):
    flat = torch.full(((bt - 1) * sc + M * ldc + 8,), float("nan"), device="cuda")
    return torch.as_strided(flat, (bt, M, N), (sc, ldc, 1)), flat


def _windows_mask(bt, M, N, ldc, sc, total):
    idx = (np.arange(bt)[:, None, None] * sc + np.arange(M)[None, :, None] * ldc
           + np.arange(N)[None, None, :])
    m = np.zeros(total, dtype=bool)
    m[idx.reshape(-1)] = True
    return m


def _check(lib, bt, M, N, K, integer, seed, pads=(0, 0, 0), gaps=(0, 0, 0),
           shared_a=False, shared_b=False):
    dist_a = dist_b = "int2" if integer else "u11"
    A = _stack(bt, M, K, dist_a, seed)
    B = _stack(bt, K, N, dist_b, seed + 5000)
    if shared_a:
        A = A[:1].expand(bt, M, K)
    if shared_b:
        B = B[:1].expand(bt, K, N)
    lda, ldb, ldc = K + pads[0], N + pads[1], N + pads[2]
    Ad = _device_batch(A, lda, M * lda + gaps[0], shared_a)
    Bd = _device_batch(B, ldb, K * ldb + gaps[1], shared_b)
    sc = M * ldc + gaps[2]
    Cd, flat = _c_buffer(bt, M, N, ldc, sc)
    kname = lib.selected_kernel_batched(Ad, Bd, Cd)
    H.say(f"batched {bt}x{M}x{N}x{K} int={integer} pads={pads} gaps={gaps} "
          f"shared={shared_a},{shared_b} kernel={kname}")
    lib.gemm_batched(Ad, Bd, Cd)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    C_ref, _, ABS = oracle.gemm_batched(A.numpy(), B.numpy())
    what = f"batched {bt}x{M}x{N}x{K} ({kname})"
    if integer:
        H.assert_bitexact(C, C_ref, what)
    else:
        H.assert_within_tol(C, C_ref, ABS, what)
    f = flat.cpu().numpy()
    outside = f[~_windows_mask(bt, M, N, ldc, sc, f.size)]
    assert np.all(np.isnan(outside)), f"{what}: wrote outside the products' windows"
    return kname


@pytest.mark.parametrize("shape", [(64, 512, 512, 512), (7, 33, 129, 200), (3, 300, 260, 1000),
                                   (1000, 8, 16, 24), (2, 1024, 1024, 1024), (5, 1, 1, 1)])
@pytest.mark.parametrize("integer", [True, False])
def test_batched_parity(gpu_lib, shape, integer):
    bt, M, N, K = shape
    _check(gpu_lib, bt, M, N, K, integer, 8000 + bt)


@pytest.mark.parametrize("integer", [True, False])
def test_batched_pitches_and_gaps(gpu_lib, integer):
    """Padded pitches and gaps between products (windows untouched); strides
    that are not multiples of 4 floats take the register-staged kernel."""
    k1 = _check(gpu_lib, 6, 130, 70, 333, integer, 8100, pads=(4, 8, 3), gaps=(4, 8, 5))
    k2 = _check(gpu_lib, 6, 130, 70, 333, integer, 8200, pads=(1, 3, 3), gaps=(1, 1, 2))
    assert "_d6_" not in k2, k2
    del k1


@pytest.mark.parametrize("shared", [(True, False), (False, True), (True, True)])
def test_batched_shared_operand(gpu_lib, shared):
    _check(gpu_lib, 9, 200, 96, 128, True, 8300, shared_a=shared[0], shared_b=shared[1])
    _check(gpu_lib, 9, 200, 96, 128, False, 8400, shared_a=shared[0], shared_b=shared[1])


def test_batched_more_than_one_launch(gpu_lib):
    """More products than one launch's grid takes (65535): launched in chunks."""
    _check(gpu_lib, 70001, 4, 5, 3, True, 8500)


def test_batched_k_zero_and_rerun(gpu_lib):
    bt, M, N = 5, 33, 40
    A = torch.zeros((bt, M, 0), device="cuda")
    B = torch.zeros((bt, 0, N), device="cuda")
    Cd, flat = _c_buffer(bt, M, N, N + 3, M * (N + 3) + 7)
    H.say("batched K=0")
    gpu_lib.gemm_batched(A, B, Cd)
    torch.cuda.synchronize()
    f = flat.cpu().numpy()
    inside = _windows_mask(bt, M, N, N + 3, M * (N + 3) + 7, f.size)
    assert np.all(f[inside] == 0) and not np.signbit(f[inside]).any()
    assert np.all(np.isnan(f[~inside]))
    # reruns are bitwise identical
    A, B = _stack(16, 256, 192, "u11", 8600).cuda(), _stack(16, 192, 128, "u11", 8700).cuda()
    H.say("batched rerun")
    C1 = gpu_lib.gemm_batched(A, B)
    C2 = gpu_lib.gemm_batched(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_batched_one_product_is_gemm_f32(gpu_lib):
    A, B = _stack(1, 700, 600, "u11", 8800), _stack(1, 600, 500, "u11", 8900)
    H.say("batched batch=1 vs gemm_f32")
    Ad, Bd = A.cuda(), B.cuda()
    C1 = gpu_lib.gemm_batched(Ad, Bd)
    C2 = gpu_lib.gemm(Ad[0], Bd[0])
    torch.cuda.synchronize()
    assert torch.equal(C1[0], C2)


# ---- calls captured into a HIP graph ------------------------------------------

def test_graph_capture_replays_match_eager(gpu_lib):
    """gemm_f32 (an MFMA tile kernel; the skinny kernel that adds its K slices
    through exchange slots, which each call must leave clear for the next
    replay; the skinny kernel with a partials workspace and a combine
    dispatch) and gemm_f32_batched captured into one graph; each replay, with
    fresh inputs copied in and eager work between replays, matches the eager
    calls bit for bit."""
    s = torch.cuda.Stream()
    shapes = {"tile": (1000, 999, 777), "skinny": (8, 4096, 4096),
              "skinny_combine": (8, 2048, 4096)}
    static = {k: (torch.empty((m, kk), device="cuda"), torch.empty((kk, n), device="cuda"),
                  torch.empty((m, n), device="cuda")) for k, (m, n, kk) in shapes.items()}
    bA, bB = torch.empty((16, 128, 96), device="cuda"), torch.empty((16, 96, 64), device="cuda")
    bC = torch.empty((16, 128, 64), device="cuda")

    def fill(seed):
        for i, (k, (m, n, kk)) in enumerate(shapes.items()):
            static[k][0].copy_(inputs.draw_matrix(m, kk, "u11", seed + 10 * i))
            static[k][1].copy_(inputs.draw_matrix(kk, n, "u11", seed + 10 * i + 1))
        bA.copy_(_stack(16, 128, 96, "int2", seed + 100))
        bB.copy_(_stack(16, 96, 64, "int2", seed + 200))

    def calls():
        for k, (A, B, C) in static.items():
            if k == "skinny_combine":
                gpu_lib.run_kernel("skinnyr_c2_r4_u4_m2x4_s0_nn", A, B, C)
            else:
                gpu_lib.gemm(A, B, C)
        gpu_lib.gemm_batched(bA, bB, bC)

    # warm up on the capture stream: the skinny kernel's workspace lives per stream
    fill(9000)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    H.say("graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        fill(9100 + rep)
        torch.cuda.synchronize()
        H.say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = [C.clone() for _, _, C in static.values()] + [bC.clone()]
        # eager work between replays, then the eager reference of the same inputs
        calls()
        torch.cuda.synchronize()
        want = [C.clone() for _, _, C in static.values()] + [bC.clone()]
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"
    # and the eager results agree with the oracle
    A, B, C = static["skinny"]
    C_ref, _, ABS = oracle.gemm(A.cpu().numpy(), B.cpu().numpy())
    H.assert_within_tol(C.cpu().numpy(), C_ref, ABS, "skinny in graph test")


# the refused call enqueues nothing, so the captured graph is empty by design
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_without_workspace_reports_error(gpu_lib):
    """A call that needs the workspace on a stream that has none yet cannot
    allocate while the stream is captured: it returns GEMM_F32_ERR_WORKSPACE
    and enqueues nothing."""
    from dense_fp32_gemm_f32_amd import binding
    s = torch.cuda.Stream()
    A = torch.randn(8, 2048, device="cuda")
    B = torch.randn(2048, 2048, device="cuda")
    C = torch.empty(8, 2048, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    rc = None
    H.say("capture without workspace")
    with torch.cuda.graph(g, stream=s):
        rc = binding.gemm_f32(8, 2048, 2048, A.data_ptr(), 2048, B.data_ptr(), 2048,
                              C.data_ptr(), 2048, s.cuda_stream)
    torch.cuda.synchronize()
    assert rc == 6, rc


def test_graph_replay_after_workspace_growth(gpu_lib):
    """A graph captured while a stream's workspaces were small replays
    correctly after larger eager calls on that stream have outgrown them: the
    outgrown buffers are kept, not freed, so the graph's kernels still find
    their partial sums and exchange slots."""
    from dense_fp32_gemm_f32_amd import binding
    torch.cuda.synchronize()
    assert binding.gemm_f32_release_workspaces() == 0
    s = torch.cuda.Stream()
    # small: 2 K slices each (0.5 MiB of exchange slots, 0.25 MiB of partials);
    # big: 4 and 32 slices (1.5 MiB of slots, 4 MiB of partials), both beyond
    # the 1 MiB first allocations
    kx, kc = "skinnyx_w8_c2_u2_s0_vec", "skinnyr_c2_r4_u4_m2x4_s0_nn"
    small = {kx: (8, 4096, 32), kc: (8, 4096, 128)}
    big = {kx: (8, 4096, 4096), kc: (8, 4096, 4096)}
    st = {k: (torch.empty((m, kk), device="cuda"), torch.empty((kk, n), device="cuda"),
              torch.empty((m, n), device="cuda")) for k, (m, n, kk) in small.items()}

    def fill(seed):
        for i, (k, (m, n, kk)) in enumerate(small.items()):
            st[k][0].copy_(inputs.draw_matrix(m, kk, "int2", seed + 2 * i))
            st[k][1].copy_(inputs.draw_matrix(kk, n, "int2", seed + 2 * i + 1))

    def calls():
        for k, (A, B, C) in st.items():
            gpu_lib.run_kernel(k, A, B, C)

    fill(9300)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    H.say("capture with small workspaces")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    # larger eager calls on the same stream outgrow both workspaces
    bigs = {}
    for i, (k, (m, n, kk)) in enumerate(big.items()):
        A, B = inputs.make_ab(m, n, kk, "int2", "int2", 9400 + i)
        bigs[k] = (A, B, A.cuda(), B.cuda())
    H.say("eager calls that grow the workspaces")
    with torch.cuda.stream(s):
        outs = {k: gpu_lib.run_kernel(k, dA, dB) for k, (_, _, dA, dB) in bigs.items()}
    torch.cuda.synchronize()
    for k, (A, B, _, _) in bigs.items():
        C_ref, _ = H.oracle_of(A, B)
        H.assert_bitexact(outs[k].cpu().numpy(), C_ref, f"grown {k}")
    for rep in range(2):
        fill(9500 + rep)
        torch.cuda.synchronize()
        H.say(f"replay after growth {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = {k: C.clone() for k, (_, _, C) in st.items()}
        with torch.cuda.stream(s):
            calls()
        torch.cuda.synchronize()
        for k, (A, B, C) in st.items():
            assert torch.equal(got[k], C), f"replay {rep} of {k} differs from the eager call"
            C_ref, _ = H.oracle_of(A.cpu(), B.cpu())
            H.assert_bitexact(C.cpu().numpy(), C_ref, f"replay {rep} {k}")
