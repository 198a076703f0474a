"""ctypes binding of ``libgemm_f32.so`` (the C ABI in ``include/gemm_f32.h``).

Two layers, both argument marshalling only -- every step of the product runs
in the HIP kernels:

* functions named exactly as the C entry points (``gemm_f32``,
  ``gemm_f32_ref_gpu``, ...) taking plain integers: sizes, device pointers,
  pitches and a ``hipStream_t`` as an integer (0 = default stream);
* ``gemm`` / ``gemm_ref`` / ``run_kernel``: the same calls on torch tensors,
  which read sizes, pitches and pointers from the tensors and enqueue on
  torch's current stream of the tensors' device.

There is no fallback: if the library is missing, ``load()`` raises.  The
environment variable ``GEMM_F32_LIB`` names another build of the same library
to load instead (the host-sanitizer build of ``sanitize_host.py``).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libgemm_f32.so"

GEMM_F32_OK = 0
STATUS_NAMES = {
    0: "GEMM_F32_OK", 1: "GEMM_F32_ERR_INVALID_DIM", 2: "GEMM_F32_ERR_INVALID_LD",
    3: "GEMM_F32_ERR_NULL_PTR", 4: "GEMM_F32_ERR_ALIAS", 5: "GEMM_F32_ERR_DEVICE",
    6: "GEMM_F32_ERR_WORKSPACE", 7: "GEMM_F32_ERR_LAUNCH", 8: "GEMM_F32_ERR_BAD_KERNEL",
    9: "GEMM_F32_ERR_POINTER", 10: "GEMM_F32_ERR_INVALID_ARG", 11: "GEMM_F32_ERR_SCRATCH",
}
ACT_NONE, ACT_RELU = 0, 1
EXPORTS = ["gemm_f32", "gemm_f32_ex", "gemm_f32_ref_gpu", "gemm_f32_status_string",
           "gemm_f32_selected_kernel", "gemm_f32_selected_kernel_ex", "gemm_f32_version",
           "gemm_f32_kernel_count", "gemm_f32_kernel_name", "gemm_f32_run_kernel",
           "gemm_f32_run_kernel_ex", "gemm_f32_release_workspaces", "gemm_f32_batched",
           "gemm_f32_selected_kernel_batched", "reduce_sum_f32", "gemm_f32_fused",
           "gemm_f32_run_kernel_fused", "gemm_f32_noalloc", "gemm_f32_clock_probe"]
CLOCK_PROBE_WORKGROUPS = 1024


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({gemm_f32_status_string(status)})")


_lib = None


def load(lib_path=None):
    """Load the HIP library (once; ``lib_path`` picks another build of it,
    such as the sweep library of tune.py).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        if lib_path is not None and Path(lib_path) != Path(_lib._name):
            raise RuntimeError(f"{_lib._name} is already loaded")
        return _lib
    if lib_path is None and os.environ.get("GEMM_F32_LIB"):
        lib_path = os.environ["GEMM_F32_LIB"]
    path = Path(lib_path) if lib_path is not None else LIB_PATH
    if not path.exists():
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m dense_fp32_gemm_f32_amd.build_lib` "
            "(there is no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(str(path))
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    gemm_args = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    for name in ("gemm_f32", "gemm_f32_ref_gpu", "gemm_f32_noalloc"):
        getattr(lib, name).argtypes = gemm_args
        getattr(lib, name).restype = ctypes.c_int
    lib.gemm_f32_run_kernel.argtypes = [ctypes.c_int, *gemm_args]
    lib.gemm_f32_run_kernel.restype = ctypes.c_int
    f32, ci = ctypes.c_float, ctypes.c_int
    ex_args = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.gemm_f32_ex.argtypes = ex_args
    lib.gemm_f32_ex.restype = ctypes.c_int
    lib.gemm_f32_run_kernel_ex.argtypes = [ci, *ex_args]
    lib.gemm_f32_run_kernel_ex.restype = ctypes.c_int
    fused_args = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp, ci, vp]
    lib.gemm_f32_fused.argtypes = fused_args
    lib.gemm_f32_fused.restype = ctypes.c_int
    lib.gemm_f32_run_kernel_fused.argtypes = [ci, *fused_args]
    lib.gemm_f32_run_kernel_fused.restype = ctypes.c_int
    lib.gemm_f32_selected_kernel_ex.argtypes = [ci, ci, i64, i64, i64, i64, i64, i64, f32, f32,
                                                vp, vp, vp]
    lib.gemm_f32_selected_kernel_ex.restype = ctypes.c_char_p
    lib.gemm_f32_status_string.argtypes = [ctypes.c_int]
    lib.gemm_f32_status_string.restype = ctypes.c_char_p
    lib.gemm_f32_selected_kernel.argtypes = [i64, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.gemm_f32_selected_kernel.restype = ctypes.c_char_p
    lib.gemm_f32_version.argtypes = []
    lib.gemm_f32_version.restype = ctypes.c_int
    lib.gemm_f32_kernel_count.argtypes = []
    lib.gemm_f32_kernel_count.restype = ctypes.c_int
    lib.gemm_f32_kernel_name.argtypes = [ctypes.c_int]
    lib.gemm_f32_kernel_name.restype = ctypes.c_char_p
    lib.gemm_f32_release_workspaces.argtypes = []
    lib.gemm_f32_release_workspaces.restype = ctypes.c_int
    lib.gemm_f32_clock_probe.argtypes = [i64, vp, vp, vp, vp]
    lib.gemm_f32_clock_probe.restype = ctypes.c_int
    lib.reduce_sum_f32.argtypes = [i64, vp, vp, vp]
    lib.reduce_sum_f32.restype = ctypes.c_int
    lib.gemm_f32_batched.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                     i64, vp]
    lib.gemm_f32_batched.restype = ctypes.c_int
    lib.gemm_f32_selected_kernel_batched.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64,
                                                     i64, vp, vp]
    lib.gemm_f32_selected_kernel_batched.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---- the C entry points, same names, plain integers ------------------------

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return load().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return load().gemm_f32_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f32_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                              stream)


def gemm_f32_fused(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                   stream=0) -> int:
    return load().gemm_f32_fused(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                 bias, act, stream)


def gemm_f32_run_kernel_fused(index, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                              ldc, bias, act, stream=0) -> int:
    return load().gemm_f32_run_kernel_fused(index, transA, transB, M, N, K, alpha, A, lda, B,
                                            ldb, beta, C, ldc, bias, act, stream)


def gemm_f32_run_kernel_ex(index, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                           stream=0) -> int:
    return load().gemm_f32_run_kernel_ex(index, transA, transB, M, N, K, alpha, A, lda, B, ldb,
                                         beta, C, ldc, stream)


def gemm_f32_selected_kernel_ex(transA, transB, M, N, K, lda, ldb, ldc, alpha=1.0, beta=0.0,
                                A=0, B=0, C=0) -> str:
    return load().gemm_f32_selected_kernel_ex(transA, transB, M, N, K, lda, ldb, ldc, alpha,
                                              beta, A, B, C).decode()


def gemm_f32_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch,
                     stream=0) -> int:
    return load().gemm_f32_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                                   batch, stream)


def gemm_f32_selected_kernel_batched(M, N, K, lda, strideA, ldb, strideB, ldc, batch, A=0,
                                     B=0) -> str:
    return load().gemm_f32_selected_kernel_batched(M, N, K, lda, strideA, ldb, strideB, ldc,
                                                   batch, A, B).decode()


def gemm_f32_clock_probe(iters, stamps, wall_khz=None, max_khz=None, stream=0) -> int:
    return load().gemm_f32_clock_probe(iters, stamps, wall_khz, max_khz, stream)


def reduce_sum_f32(n, x, out, stream=0) -> int:
    return load().reduce_sum_f32(n, x, out, stream)


def gemm_f32_ref_gpu(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return load().gemm_f32_ref_gpu(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_run_kernel(index, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    return load().gemm_f32_run_kernel(index, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_status_string(status: int) -> str:
    return load().gemm_f32_status_string(int(status)).decode()


def gemm_f32_selected_kernel(M, N, K, lda, ldb, ldc, A=0, B=0, C=0) -> str:
    return load().gemm_f32_selected_kernel(M, N, K, lda, ldb, ldc, A, B, C).decode()


def gemm_f32_version() -> int:
    return load().gemm_f32_version()


def gemm_f32_kernel_count() -> int:
    return load().gemm_f32_kernel_count()


def gemm_f32_kernel_name(index: int) -> str | None:
    r = load().gemm_f32_kernel_name(index)
    return None if r is None else r.decode()


def gemm_f32_release_workspaces() -> int:
    return load().gemm_f32_release_workspaces()


def kernel_names() -> list[str]:
    return [gemm_f32_kernel_name(i) for i in range(gemm_f32_kernel_count())]


def kernel_index(name: str) -> int:
    names = kernel_names()
    if name not in names:
        raise KeyError(f"no kernel named {name!r}")
    return names.index(name)


# ---- torch tensors -----------------------------------------------------------

def _pitch(t, name):
    import torch
    if t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 tensor")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on a GPU (got {t.device})")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    return max(t.stride(0), t.shape[1], 1) if t.shape[0] > 1 else max(t.shape[1], 1)


def _args(A, B, C):
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be {M}x{N}, got {tuple(C.shape)}")
    lda, ldb, ldc = _pitch(A, "A"), _pitch(B, "B"), _pitch(C, "C")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on one device")
    stream = torch.cuda.current_stream(A.device).cuda_stream
    return (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, stream), C


def gemm(A, B, C=None):
    """C = A @ B on the GPU with the dispatcher's kernel; returns C."""
    args, C = _args(A, B, C)
    with _device(A):
        rc = gemm_f32(*args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32")
    return C


def gemm_noalloc(A, B, C=None):
    """C = A @ B through gemm_f32_noalloc (the fixed scratch array, no
    allocation inside the library); returns C."""
    args, C = _args(A, B, C)
    with _device(A):
        rc = gemm_f32_noalloc(*args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_noalloc")
    return C


def gemm_ref(A, B, C=None):
    """C = A @ B with the naive reference kernel; returns C."""
    args, C = _args(A, B, C)
    with _device(A):
        rc = gemm_f32_ref_gpu(*args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_ref_gpu")
    return C


def run_kernel(index_or_name, A, B, C=None):
    """C = A @ B with one named (or indexed) kernel of the table; returns C."""
    index = kernel_index(index_or_name) if isinstance(index_or_name, str) else int(index_or_name)
    args, C = _args(A, B, C)
    with _device(A):
        rc = gemm_f32_run_kernel(index, *args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, f"gemm_f32_run_kernel({index_or_name})")
    return C


def _args_batched(A, B, C):
    """Sizes, pointers, pitches and batch strides of 3-D tensors (batch, rows,
    cols); a batch stride of 0 (an expanded tensor) shares one matrix."""
    import torch
    if A.dim() != 3 or B.dim() != 3:
        raise TypeError("A and B must be 3-D (batch, rows, cols)")
    batch, M, K = A.shape
    batch2, K2, N = B.shape
    if K != K2 or batch != batch2:
        raise ValueError(f"shapes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if C is None:
        C = torch.empty((batch, M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (batch, M, N):
        raise ValueError(f"C must be {batch}x{M}x{N}, got {tuple(C.shape)}")
    if batch == 0:
        lda, ldb, ldc = max(K, 1), max(N, 1), max(N, 1)
    else:
        lda, ldb, ldc = _pitch(A[0], "A"), _pitch(B[0], "B"), _pitch(C[0], "C")
    sa, sb, sc = A.stride(0), B.stride(0), C.stride(0)
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on one device")
    stream = torch.cuda.current_stream(A.device).cuda_stream
    return (M, N, K, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb, C.data_ptr(), ldc, sc,
            batch, stream), C


def gemm_batched(A, B, C=None):
    """C[b] = A[b] @ B[b] for every b, in as few launches as possible (3-D
    tensors; a stride of 0 along the batch shares one matrix).  Returns C."""
    args, C = _args_batched(A, B, C)
    with _device(A):
        rc = gemm_f32_batched(*args)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_batched")
    return C


def selected_kernel_batched(A, B, C=None) -> str:
    (M, N, K, a, lda, sa, b, ldb, sb, _c, ldc, _sc, batch, _s), _ = _args_batched(A, B, C)
    return gemm_f32_selected_kernel_batched(M, N, K, lda, sa, ldb, sb, ldc, batch, a, b)


def reduce_sum(x, out=None):
    """Sum of a 1-D contiguous float32 GPU tensor into a 1-element tensor
    (returned), in an order fixed by the length."""
    import torch
    if x.dtype != torch.float32 or x.dim() != 1 or (x.numel() > 1 and x.stride(0) != 1):
        raise TypeError("x must be a contiguous 1-D float32 tensor")
    if x.device.type != "cuda":
        raise TypeError(f"x must be on a GPU (got {x.device})")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with _device(x):
        rc = reduce_sum_f32(x.numel(), x.data_ptr(), out.data_ptr(), stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "reduce_sum_f32")
    return out


def clock_probe(iters=2400, device=None):
    """Run gemm_f32_clock_probe on torch's current stream of ``device`` and
    wait for it.  Returns (per-workgroup achieved shader clocks in GHz, the
    constant counter's rate in kHz, the device's peak shader clock in kHz)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    stamps = torch.zeros(4 * CLOCK_PROBE_WORKGROUPS, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    wall, peak = ctypes.c_int(0), ctypes.c_int(0)
    with _device(stamps):
        rc = gemm_f32_clock_probe(iters, stamps.data_ptr(), ctypes.byref(wall),
                                  ctypes.byref(peak), stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_clock_probe")
    torch.cuda.synchronize(dev)
    w = stamps.view(-1, 4).cpu().tolist()
    ghz = [wall.value * 1e-6 * (t1 - t0) / (r1 - r0) for t0, r0, t1, r1 in w if r1 > r0]
    return ghz, wall.value, peak.value


def _args_ex(A, B, C, trans_a, trans_b):
    import torch
    M, K = (A.shape[1], A.shape[0]) if trans_a else tuple(A.shape)
    K2, N = (B.shape[1], B.shape[0]) if trans_b else tuple(B.shape)
    if K != K2:
        raise ValueError(f"inner sizes differ: op(A) is {M}x{K}, op(B) is {K2}x{N}")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be {M}x{N}, got {tuple(C.shape)}")
    lda, ldb, ldc = _pitch(A, "A"), _pitch(B, "B"), _pitch(C, "C")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on one device")
    stream = torch.cuda.current_stream(A.device).cuda_stream
    return (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, stream), C


def gemm_ex(A, B, C=None, *, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, kernel=None):
    """C = alpha * op(A) @ op(B) + beta * C on the GPU; A and B are the stored
    matrices (A is K x M when trans_a, B is N x K when trans_b).  ``kernel``
    runs one named (or indexed) kernel of the table instead of the
    dispatcher's.  Returns C."""
    (M, N, K, a, lda, b, ldb, c, ldc, stream), C = _args_ex(A, B, C, trans_a, trans_b)
    ta, tb = int(bool(trans_a)), int(bool(trans_b))
    with _device(A):
        if kernel is None:
            rc = gemm_f32_ex(ta, tb, M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, stream)
        else:
            index = kernel_index(kernel) if isinstance(kernel, str) else int(kernel)
            rc = gemm_f32_run_kernel_ex(index, ta, tb, M, N, K, alpha, a, lda, b, ldb, beta, c,
                                        ldc, stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_ex" if kernel is None else f"gemm_f32_run_kernel_ex({kernel})")
    return C


def gemm_fused(A, B, C=None, *, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, bias=None,
               act=ACT_NONE, kernel=None):
    """C = act(alpha * op(A) @ op(B) + beta * C + bias) on the GPU; ``bias`` a
    1-D contiguous tensor of N floats (or None), ``act`` ACT_NONE or ACT_RELU.
    ``kernel`` runs one named (or indexed) kernel of the table.  Returns C."""
    (M, N, K, a, lda, b, ldb, c, ldc, stream), C = _args_ex(A, B, C, trans_a, trans_b)
    bptr = 0
    if bias is not None:
        if bias.dim() != 1 or bias.numel() != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError(f"bias must be a contiguous vector of {N} floats")
        bptr = bias.data_ptr()
    ta, tb = int(bool(trans_a)), int(bool(trans_b))
    with _device(A):
        if kernel is None:
            rc = gemm_f32_fused(ta, tb, M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, bptr,
                                int(act), stream)
        else:
            index = kernel_index(kernel) if isinstance(kernel, str) else int(kernel)
            rc = gemm_f32_run_kernel_fused(index, ta, tb, M, N, K, alpha, a, lda, b, ldb, beta,
                                           c, ldc, bptr, int(act), stream)
    if rc != GEMM_F32_OK:
        raise GemmError(rc, "gemm_f32_fused" if kernel is None else
                        f"gemm_f32_run_kernel_fused({kernel})")
    return C


def selected_kernel_ex(A, B, C=None, *, trans_a=False, trans_b=False, alpha=1.0,
                       beta=0.0) -> str:
    M, K = (A.shape[1], A.shape[0]) if trans_a else tuple(A.shape)
    N = B.shape[0] if trans_b else B.shape[1]
    lda = max(A.stride(0), A.shape[1], 1)
    ldb = max(B.stride(0), B.shape[1], 1)
    ldc = N if C is None else max(C.stride(0), N)
    return gemm_f32_selected_kernel_ex(int(bool(trans_a)), int(bool(trans_b)), M, N, K, lda,
                                       ldb, max(ldc, 1), alpha, beta, A.data_ptr(),
                                       B.data_ptr(), 0 if C is None else C.data_ptr())


def selected_kernel(A, B, C=None) -> str:
    M, K = A.shape
    N = B.shape[1]
    ldc = N if C is None else max(C.stride(0), N)
    return gemm_f32_selected_kernel(M, N, K, max(A.stride(0), K, 1), max(B.stride(0), N, 1),
                                    max(ldc, 1), A.data_ptr(), B.data_ptr(),
                                    0 if C is None else C.data_ptr())


class _device:
    """Make the tensor's device current for the call (the library uses the
    current HIP device)."""

    def __init__(self, t):
        self.idx = t.device.index

    def __enter__(self):
        import torch
        self.prev = torch.cuda.current_device()
        if self.idx is not None and self.idx != self.prev:
            torch.cuda.set_device(self.idx)

    def __exit__(self, *exc):
        import torch
        if self.idx is not None and self.idx != self.prev:
            torch.cuda.set_device(self.prev)
        return False
