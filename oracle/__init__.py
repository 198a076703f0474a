"""CPU oracle for dense row-major fp32 ``C = A x B`` and for the sum of an
fp32 array (binary64 accumulation).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library in
``dense_fp32_gemm_f32_amd``: the arithmetic lives in ``gemm_oracle.c``
(plain C, built with gcc, no HIP headers) and this module only marshals
numpy arrays into it.

Definition followed (see the header of ``gemm_oracle.c``): element (i, j) is
row i of A dotted with column j of B ("Optimizing a WebGPU Matmul Kernel
using Subgroups", section 1 Naive), summed in ascending k in binary64 and
rounded once to binary32, as the CPU triple loop of "WebGPU 行列積の限界を測る"
does with its JavaScript-number accumulator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "gemm_oracle.c"
LIB_PATH = _HERE / "libgemm_oracle.so"

# gcc, OpenMP over output rows, no -ffast-math (IEEE binary64 throughout).
_CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-fno-fast-math", "-ffp-contract=off"]

_lib = None


def build(force: bool = True) -> Path:
    """Compile ``gemm_oracle.c`` into ``libgemm_oracle.so`` with gcc."""
    if not force and LIB_PATH.exists() and LIB_PATH.stat().st_mtime >= _SRC.stat().st_mtime:
        return LIB_PATH
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = ["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        build()
    lib = ctypes.CDLL(str(LIB_PATH))
    i64, f32p, f64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_gemm_f64acc.argtypes = [i64, i64, i64, f32p, i64, f32p, i64,
                                       f32p, i64, f64p, i64, f64p, i64]
    lib.oracle_gemm_f64acc.restype = ctypes.c_int
    lib.oracle_gemm_elems.argtypes = [i64, i64, i64, f32p, i64, f32p, i64,
                                      i64, ctypes.c_void_p, ctypes.c_void_p,
                                      f32p, f64p, f64p]
    lib.oracle_gemm_elems.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.oracle_gemm_ex_f64acc.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, f32,
                                          f32p, i64, f32p, i64, f32, f32p, i64,
                                          f32p, i64, f64p, i64, f64p, i64]
    lib.oracle_gemm_ex_f64acc.restype = ctypes.c_int
    lib.oracle_gemm_fused_f64acc.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, f32,
                                             f32p, i64, f32p, i64, f32, f32p, i64,
                                             f32p, ctypes.c_int,
                                             f32p, i64, f64p, i64, f64p, i64]
    lib.oracle_gemm_fused_f64acc.restype = ctypes.c_int
    lib.oracle_sum_f64acc.argtypes = [i64, f32p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.oracle_sum_f64acc.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_int
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ld(x: np.ndarray, name: str) -> int:
    """Row pitch in elements of a 2-D float32 array whose rows are contiguous."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return max(1, x.shape[1])
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} rows must be contiguous")
    if x.shape[0] <= 1:
        return max(1, x.shape[1])
    if x.strides[0] % 4:
        raise ValueError(f"{name} row pitch must be a multiple of 4 bytes")
    return x.strides[0] // 4


def gemm(A: np.ndarray, B: np.ndarray, *, want_f64: bool = True):
    """Return ``(C, Cd, ABS)`` for ``A @ B``.

    ``A`` (M x K) and ``B`` (K x N) are float32 arrays with contiguous rows and
    any row pitch (``lda = A.strides[0] / 4`` etc.).  ``C`` is float32, ``Cd``
    (the binary64 sum before rounding) and ``ABS`` (sum of |a_ik b_kj|) are
    float64; the last two are ``None`` when ``want_f64`` is false.
    """
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    C = np.zeros((M, N), dtype=np.float32)
    Cd = np.zeros((M, N), dtype=np.float64) if want_f64 else None
    ABS = np.zeros((M, N), dtype=np.float64) if want_f64 else None
    if M == 0 or N == 0:
        return C, Cd, ABS
    ldn = max(1, N)
    rc = _load().oracle_gemm_f64acc(
        M, N, K, A.ctypes.data if A.size else None, max(lda, K),
        B.ctypes.data if B.size else None, max(ldb, N),
        C.ctypes.data, ldn,
        Cd.ctypes.data if want_f64 else None, ldn,
        ABS.ctypes.data if want_f64 else None, ldn)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_f64acc failed with status {rc}")
    return C, Cd, ABS


def gemm_elems(A: np.ndarray, B: np.ndarray, rows, cols):
    """The oracle at the listed positions only: ``(C, Cd, ABS)`` 1-D arrays."""
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    n = rows.size
    C = np.zeros(n, dtype=np.float32)
    Cd = np.zeros(n, dtype=np.float64)
    ABS = np.zeros(n, dtype=np.float64)
    if n == 0:
        return C, Cd, ABS
    rc = _load().oracle_gemm_elems(
        M, N, K, A.ctypes.data if A.size else None, max(lda, K),
        B.ctypes.data if B.size else None, max(ldb, N),
        n, rows.ctypes.data, cols.ctypes.data,
        C.ctypes.data, Cd.ctypes.data, ABS.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_elems failed with status {rc}")
    return C, Cd, ABS


def gemm_ex(A: np.ndarray, B: np.ndarray, *, trans_a: bool = False, trans_b: bool = False,
            alpha: float = 1.0, beta: float = 0.0, C_in: np.ndarray | None = None):
    """Return ``(C, Cd, ABS)`` for ``alpha * op(A) @ op(B) + beta * C_in``.

    ``A`` is stored M x K, or K x M when ``trans_a``; ``B`` is stored K x N, or
    N x K when ``trans_b`` (float32, contiguous rows, any row pitch).  ``C_in``
    (M x N float32) is read only when ``beta != 0``.  ``alpha`` and ``beta``
    are used as binary32 values.  Definition: ``oracle_gemm_ex_f64acc`` in
    ``gemm_oracle.c``.
    """
    if trans_a:
        K, M = A.shape
    else:
        M, K = A.shape
    if trans_b:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    alpha32, beta32 = float(np.float32(alpha)), float(np.float32(beta))
    C = np.zeros((M, N), dtype=np.float32)
    Cd = np.zeros((M, N), dtype=np.float64)
    ABS = np.zeros((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return C, Cd, ABS
    cin_ptr, ldcin = None, max(1, N)
    if beta32 != 0.0:
        if C_in is None or C_in.shape != (M, N):
            raise ValueError("C_in (M x N) is needed when beta != 0")
        ldcin = _ld(C_in, "C_in")
        cin_ptr = C_in.ctypes.data
    rc = _load().oracle_gemm_ex_f64acc(
        int(bool(trans_a)), int(bool(trans_b)), M, N, K, alpha32,
        A.ctypes.data if A.size else None, max(lda, M if trans_a else K),
        B.ctypes.data if B.size else None, max(ldb, K if trans_b else N),
        beta32, cin_ptr, max(ldcin, N),
        C.ctypes.data, N, Cd.ctypes.data, N, ABS.ctypes.data, N)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex_f64acc failed with status {rc}")
    return C, Cd, ABS


def gemm_batched(A: np.ndarray, B: np.ndarray, *, want_f64: bool = True):
    """Return ``(C, Cd, ABS)`` for the strided batch ``C[b] = A[b] @ B[b]``.

    ``A`` (batch x M x K) and ``B`` (batch x K x N) are float32 arrays whose
    matrices have contiguous rows; a batch stride of 0 (``np.broadcast_to``)
    shares one matrix.  Each product is ``gemm`` of its two matrices: the
    batch is a set of independent products (the batched dispatch the "GPU
    compute shaders" page times), with nothing shared between them.
    """
    if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0]:
        raise ValueError("A and B must be 3-D with equal batch sizes")
    batch, M, _ = A.shape
    N = B.shape[2]
    C = np.zeros((batch, M, N), dtype=np.float32)
    Cd = np.zeros((batch, M, N), dtype=np.float64) if want_f64 else None
    ABS = np.zeros((batch, M, N), dtype=np.float64) if want_f64 else None
    for b in range(batch):
        c, cd, ab = gemm(A[b], B[b], want_f64=want_f64)
        C[b] = c
        if want_f64:
            Cd[b] = cd
            ABS[b] = ab
    return C, Cd, ABS


def sum_f32(x: np.ndarray):
    """Return ``(s, sd, abs)`` for the sum of a 1-D float32 array: the binary32
    rounding of the ascending-order binary64 sum, that sum, and sum |x[i]|.
    Definition: ``oracle_sum_f64acc`` in ``gemm_oracle.c``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 1:
        raise ValueError("x must be 1-D")
    s = ctypes.c_float(0.0)
    sd = ctypes.c_double(0.0)
    ab = ctypes.c_double(0.0)
    rc = _load().oracle_sum_f64acc(x.size, x.ctypes.data if x.size else None,
                                   ctypes.byref(s), ctypes.byref(sd), ctypes.byref(ab))
    if rc != 0:
        raise RuntimeError(f"oracle_sum_f64acc failed with status {rc}")
    return np.float32(s.value), sd.value, ab.value


def gemm_fused(A: np.ndarray, B: np.ndarray, *, trans_a: bool = False, trans_b: bool = False,
               alpha: float = 1.0, beta: float = 0.0, C_in: np.ndarray | None = None,
               bias: np.ndarray | None = None, act: int = 0):
    """Return ``(C, Cd, ABS)`` for ``act(alpha * op(A) @ op(B) + beta * C_in +
    bias)``: ``gemm_ex`` plus a bias row vector (length N, added to every row)
    and an activation (0: none, 1: ReLU).  Definition:
    ``oracle_gemm_fused_f64acc`` in ``gemm_oracle.c``."""
    if trans_a:
        K, M = A.shape
    else:
        M, K = A.shape
    if trans_b:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    alpha32, beta32 = float(np.float32(alpha)), float(np.float32(beta))
    C = np.zeros((M, N), dtype=np.float32)
    Cd = np.zeros((M, N), dtype=np.float64)
    ABS = np.zeros((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return C, Cd, ABS
    cin_ptr, ldcin = None, max(1, N)
    if beta32 != 0.0:
        if C_in is None or C_in.shape != (M, N):
            raise ValueError("C_in (M x N) is needed when beta != 0")
        ldcin = _ld(C_in, "C_in")
        cin_ptr = C_in.ctypes.data
    bias_ptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have N elements")
        bias_ptr = bias.ctypes.data
    rc = _load().oracle_gemm_fused_f64acc(
        int(bool(trans_a)), int(bool(trans_b)), M, N, K, alpha32,
        A.ctypes.data if A.size else None, max(lda, M if trans_a else K),
        B.ctypes.data if B.size else None, max(ldb, K if trans_b else N),
        beta32, cin_ptr, max(ldcin, N), bias_ptr, int(act),
        C.ctypes.data, N, Cd.ctypes.data, N, ABS.ctypes.data, N)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_fused_f64acc failed with status {rc}")
    return C, Cd, ABS
