"""Pins for the CPU oracle: checks against facts the definition and the
mathematics fix, independent of the oracle's own code.

Each ``pin_*`` takes a GEMM function ``fn(A, B) -> (C, Cd, ABS)`` with the
oracle's contract (float32 inputs with contiguous rows and any row pitch;
float32 C, float64 Cd and ABS) and returns a list of failure messages (empty
when the pin holds).  The same pins are run against deliberately wrong
variants in ``test_oracle_pins.py`` to show that each plausible mistake is
caught by at least one of them.
"""
from __future__ import annotations

import json
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

from dense_fp32_gemm_f32_amd import inputs

GOLDEN = Path(__file__).resolve().parent / "golden"


def _np(t: torch.Tensor) -> np.ndarray:
    return t.numpy()


def _ints(rows, cols, seed, lo=-2, hi=2):
    return _np(inputs.int_matrix(rows, cols, seed, lo, hi))


def _exact_int(A, B):
    """Integer product in int64: exact, no floating point involved."""
    return A.astype(np.int64) @ B.astype(np.int64)


def _fail(name, msg):
    return [f"{name}: {msg}"]


# --- closed forms -----------------------------------------------------------

def pin_identity(fn):
    """I x B = B and A x I = A, bit for bit (one nonzero product per term)."""
    errs = []
    for (m, n, seed) in [(17, 23, 11), (64, 40, 12), (5, 1, 13)]:
        B = _np(inputs.uniform_matrix(m, n, seed))
        C, _, _ = fn(np.eye(m, dtype=np.float32), B)
        if not np.array_equal(C, B):
            errs += _fail("identity-left", f"I({m}) x B({m}x{n}) != B")
        A = _np(inputs.uniform_matrix(n, m, seed + 100))
        C, _, _ = fn(A, np.eye(m, dtype=np.float32))
        if not np.array_equal(C, A):
            errs += _fail("identity-right", f"A({n}x{m}) x I({m}) != A")
    return errs


def pin_permutation(fn):
    """P x B permutes the rows of B, A x P permutes the columns of A."""
    errs = []
    rng = np.random.default_rng(7)
    for (m, n) in [(19, 13), (32, 48), (24, 24)]:
        p = rng.permutation(m)
        P = np.zeros((m, m), dtype=np.float32)
        P[np.arange(m), p] = 1.0           # (P x B)[i] = B[p[i]]
        B = _np(inputs.uniform_matrix(m, n, 21))
        C, _, _ = fn(P, B)
        if not np.array_equal(C, B[p]):
            errs += _fail("permutation-left", f"rows not permuted at {m}x{n}")
        A = _np(inputs.uniform_matrix(n, m, 22))
        C, _, _ = fn(A, P)                 # (A x P)[:, j] = A[:, q] with p[q] = j
        q = np.argsort(p)
        if not np.array_equal(C, A[:, q]):
            errs += _fail("permutation-right", f"columns not permuted at {n}x{m}")
    return errs


def pin_all_ones(fn):
    """Ones(M x K) x Ones(K x N) = K everywhere."""
    errs = []
    for (m, n, k) in [(3, 5, 7), (16, 9, 300)]:
        C, Cd, ABS = fn(np.ones((m, k), np.float32), np.ones((k, n), np.float32))
        if not np.all(C == np.float32(k)):
            errs += _fail("all-ones", f"C != {k} at {m}x{n}x{k}")
        if ABS is not None and not np.all(ABS == float(k)):
            errs += _fail("all-ones", "ABS != K")
    return errs


def pin_rank1(fn):
    """Both readings of the rank-1 closed form, small integers, exact:
    (u v^T)(w z^T) = (v.w) u z^T  and  (u v^T) W = u (v^T W)."""
    errs = []
    m, k, n = 11, 9, 14
    u, v = _ints(m, 1, 31, -3, 3), _ints(k, 1, 32, -3, 3)
    w, z = _ints(k, 1, 33, -3, 3), _ints(n, 1, 34, -3, 3)
    A = (u @ v.T).astype(np.float32)
    B = (w @ z.T).astype(np.float32)
    dot = sum(int(v[t, 0]) * int(w[t, 0]) for t in range(k))
    want = np.array([[dot * int(u[i, 0]) * int(z[j, 0]) for j in range(n)]
                     for i in range(m)], dtype=np.float32)
    C, _, _ = fn(A, B)
    if not np.array_equal(C, want):
        errs += _fail("rank1-outer", "(u v^T)(w z^T) != (v.w) u z^T")
    W = _ints(k, n, 35, -4, 4)
    vW = [sum(int(v[t, 0]) * int(W[t, j]) for t in range(k)) for j in range(n)]
    want = np.array([[int(u[i, 0]) * vW[j] for j in range(n)] for i in range(m)],
                    dtype=np.float32)
    C, _, _ = fn(A, W)
    if not np.array_equal(C, want):
        errs += _fail("rank1-left", "(u v^T) W != u (v^T W)")
    return errs


# --- brute force --------------------------------------------------------------

def pin_integer_bruteforce(fn):
    """Random small integers against an int64 product (exact in any order),
    including padded row pitches and a 1-row / 1-column / 1-deep case."""
    errs = []
    cases = [(32, 24, 16, 0, 0), (37, 29, 53, 3, 5), (1, 50, 40, 0, 0),
             (50, 1, 40, 0, 0), (20, 30, 1, 2, 0), (64, 64, 257, 0, 7)]
    for t, (m, n, k, pa, pb) in enumerate(cases):
        A, B = inputs.make_ab(m, n, k, "int2", "int2", 500 + t, lda=k + pa, ldb=n + pb)
        A, B = _np(A), _np(B)
        C, Cd, ABS = fn(A, B)
        want = _exact_int(A, B)
        if not np.array_equal(C, want.astype(np.float32)):
            errs += _fail("int-bruteforce", f"C wrong at {m}x{n}x{k} (pads {pa},{pb})")
        if Cd is not None and not np.array_equal(Cd, want.astype(np.float64)):
            errs += _fail("int-bruteforce", f"Cd wrong at {m}x{n}x{k}")
        if ABS is not None:
            want_abs = np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))
            if not np.array_equal(ABS, want_abs.astype(np.float64)):
                errs += _fail("int-bruteforce", f"ABS != |A| |B| at {m}x{n}x{k}")
    return errs


def pin_exact_rational(fn):
    """Tiny inputs on a 2^-12 grid: every partial sum is exact in binary64,
    so the true sum is known exactly (Fraction) and C must be its single
    round-to-nearest-even rounding to binary32."""
    errs = []
    rng = np.random.default_rng(99)
    for (m, n, k) in [(3, 4, 5), (6, 2, 8), (1, 7, 3)]:
        A = (rng.integers(-4095, 4096, (m, k)) / 4096.0).astype(np.float32)
        B = (rng.integers(-4095, 4096, (k, n)) / 4096.0).astype(np.float32)
        C, Cd, _ = fn(A, B)
        for i in range(m):
            for j in range(n):
                s = sum((Fraction(float(A[i, p])) * Fraction(float(B[p, j])) for p in range(k)),
                        Fraction(0))
                exact64 = float(s)       # exact: s is a multiple of 2^-24 below 2^4
                if Fraction(exact64) != s:
                    raise AssertionError("grid assumption broken")
                if np.float32(exact64) != C[i, j]:
                    errs += _fail("exact-rational", f"C[{i},{j}] not RN-even of exact sum")
                if Cd is not None and Cd[i, j] != exact64:
                    errs += _fail("exact-rational", f"Cd[{i},{j}] != exact sum")
    return errs


def pin_golden_page_pattern(fn):
    """The integer pattern checked on the 'GPU compute shaders' page."""
    g = json.loads((GOLDEN / "gpu_compute_shaders_tiled_matmul_pattern.json").read_text())
    m, n, k = g["m"], g["n"], g["k"]
    a = np.array([(i % g["a_mod"]) + g["a_offset"] for i in range(m * k)], np.float32).reshape(m, k)
    b = np.array([(i % g["b_mod"]) + g["b_offset"] for i in range(k * n)], np.float32).reshape(k, n)
    C, _, _ = fn(a, b)
    errs = []
    for e in g["hand_derived"]:
        if C[e["row"], e["col"]] != e["value"]:
            errs += _fail("page-pattern", f"C[{e['row']},{e['col']}] = {C[e['row'], e['col']]} != {e['value']}")
    # the page's own check: each element equals the ascending-k sum (exact for integers)
    for r in range(m):
        for q in range(n):
            want = 0
            for p in range(k):
                want += int(a[r, p]) * int(b[p, q])
            if C[r, q] != want:
                return errs + _fail("page-pattern", f"C[{r},{q}] != {want}")
    return errs


# --- metamorphic relations ----------------------------------------------------

def pin_transpose(fn):
    """(B^T A^T) = (A B)^T bit for bit: same products, same ascending k."""
    A = _np(inputs.uniform_matrix(21, 34, 41))
    B = _np(inputs.uniform_matrix(34, 15, 42))
    C1, _, _ = fn(A, B)
    C2, _, _ = fn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    return [] if np.array_equal(C1, C2.T) else _fail("transpose", "(B^T A^T)^T != A B")


def pin_linearity(fn):
    """(A1 + A2) B = A1 B + A2 B on integers (exact)."""
    A1, A2 = _ints(18, 27, 51, -3, 3), _ints(18, 27, 52, -3, 3)
    B = _ints(27, 22, 53, -3, 3)
    C, _, _ = fn((A1 + A2).astype(np.float32), B)
    C1, _, _ = fn(A1, B)
    C2, _, _ = fn(A2, B)
    return [] if np.array_equal(C, C1 + C2) else _fail("linearity", "(A1+A2)B != A1 B + A2 B")


def pin_pitch_invariance(fn):
    """Same values with padded pitches (padding = NaN) give the same C."""
    A, B = inputs.make_ab(23, 31, 45, "u11", "u11", 61)
    Ap, Bp = inputs.make_ab(23, 31, 45, "u11", "u11", 61, lda=48, ldb=36)
    C1, _, _ = fn(_np(A), _np(B))
    C2, _, _ = fn(_np(Ap), _np(Bp))
    if not np.all(np.isfinite(C2)):
        return _fail("pitch", "padding leaked into C")
    return [] if np.array_equal(C1, C2) else _fail("pitch", "C depends on the row pitch")


# --- agreement with a library routine and the error bound ----------------------

def pin_float64_library(fn):
    """Random U[-1,1) and N(0,1) inputs: the binary64 sum agrees with torch's
    float64 matmul within the summation bound 2 K u64 sum|a b|, and C is within
    one binary32 rounding of the exact product."""
    errs = []
    for (m, n, k, dist, seed) in [(40, 50, 300, "u11", 71), (33, 17, 1000, "normal", 72)]:
        A, B = inputs.make_ab(m, n, k, dist, dist, seed)
        C, Cd, ABS = fn(_np(A), _np(B))
        ref = (A.double() @ B.double()).numpy()
        absref = (A.double().abs() @ B.double().abs()).numpy()
        u64 = 2.0 ** -53
        bound64 = 2 * k * u64 * absref
        if Cd is not None and not np.all(np.abs(Cd - ref) <= bound64):
            errs += _fail("float64-library", f"Cd differs from float64 matmul at {m}x{n}x{k}")
        if ABS is not None and not np.all(np.abs(ABS - absref) <= bound64):
            errs += _fail("float64-library", "ABS differs from |A| |B|")
        # binary32 rounding of the (nearly) exact value: half an ulp plus bound64
        err = np.abs(C.astype(np.float64) - ref)
        allow = np.abs(ref) * 2.0 ** -24 + 2 * bound64 + 1e-45
        if not np.all(err <= allow):
            errs += _fail("float64-library", f"C not the rounded product at {m}x{n}x{k}")
    return errs


ALL_PINS = [pin_identity, pin_permutation, pin_all_ones, pin_rank1,
            pin_integer_bruteforce, pin_exact_rational, pin_golden_page_pattern,
            pin_transpose, pin_linearity, pin_pitch_invariance, pin_float64_library]


def run_all(fn):
    errs = []
    for p in ALL_PINS:
        errs += p(fn)
    return errs


# --- the extended operation: alpha * op(A) op(B) + beta * C ---------------------
#
# Each ``pin_ex_*`` takes ``fn_ex(A, B, trans_a, trans_b, alpha, beta, C_in) ->
# (C, Cd, ABS)`` with the contract of ``oracle.gemm_ex``.

TRANS = [(False, False), (False, True), (True, False), (True, True)]


def _stored(X, trans):
    """The buffer a caller passes for op(X) = X (trans false) or X^T."""
    return np.ascontiguousarray(X.T) if trans else X


def pin_ex_integer_bruteforce(fn_ex):
    """Small integers, integer alpha and beta, every layout: C is exactly
    alpha * (A @ B) + beta * C_in, computed in int64 with no floating point."""
    errs = []
    for (m, n, k, seed) in [(13, 9, 21, 301), (16, 16, 16, 302), (1, 7, 5, 303), (6, 1, 9, 304)]:
        A, B = _ints(m, k, seed), _ints(k, n, seed + 10)
        Cin = _ints(m, n, seed + 20, -5, 5)
        for (ta, tb) in TRANS:
            for (alpha, beta) in [(1, 0), (2, 1), (-1, -3), (0, 1)]:
                C, _, _ = fn_ex(_stored(A, ta), _stored(B, tb), ta, tb, float(alpha),
                                float(beta), Cin)
                want = alpha * _exact_int(A, B) + beta * Cin.astype(np.int64)
                if not np.array_equal(C.astype(np.int64), want):
                    errs += _fail("ex-integer", f"{m}x{n}x{k} trans={ta},{tb} "
                                                f"alpha={alpha} beta={beta}")
    return errs


def pin_ex_float_layouts(fn_ex):
    """alpha = 1, beta = 0: every layout gives, bit for bit, the product of
    the explicitly transposed operands under the plain oracle contract (C, Cd
    and ABS), which the pins above fix."""
    import oracle
    errs = []
    A, B = inputs.make_ab(19, 23, 37, "normal", "u11", 311)
    A, B = _np(A), _np(B)
    C0, Cd0, ABS0 = oracle.gemm(A, B)
    for (ta, tb) in TRANS:
        C, Cd, ABS = fn_ex(_stored(A, ta), _stored(B, tb), ta, tb, 1.0, 0.0, None)
        if not (np.array_equal(C, C0) and np.array_equal(Cd, Cd0) and np.array_equal(ABS, ABS0)):
            errs += _fail("ex-layouts", f"trans={ta},{tb} differs from the plain product")
    return errs


def pin_ex_beta_zero_ignores_c(fn_ex):
    """beta = 0: the input C is not read, so NaN there does not reach C."""
    A, B = _ints(7, 11, 321), _ints(11, 5, 322)
    Cin = np.full((7, 5), np.nan, np.float32)
    C, _, _ = fn_ex(A, B, False, False, 3.0, 0.0, Cin)
    if not np.all(np.isfinite(C)):
        return _fail("ex-beta0", "NaN of the input C reached C with beta = 0")
    return [] if np.array_equal(C.astype(np.int64), 3 * _exact_int(A, B)) else \
        _fail("ex-beta0", "C != 3 A B")


def pin_ex_alpha_zero(fn_ex):
    """alpha = 0, beta = 1: C is the input C bit for bit (any A, B)."""
    A, B = inputs.make_ab(9, 8, 30, "normal", "normal", 331)
    Cin = _np(inputs.uniform_matrix(9, 8, 332))
    C, _, ABS = fn_ex(_np(A), _np(B), False, False, 0.0, 1.0, Cin)
    errs = [] if np.array_equal(C, Cin) else _fail("ex-alpha0", "C != C_in")
    if not np.array_equal(ABS, np.abs(Cin.astype(np.float64))):
        errs += _fail("ex-alpha0", "ABS != |C_in|")
    return errs


def pin_ex_pitch(fn_ex):
    """Transposed operands with padded pitches (padding = NaN) give the same C."""
    errs = []
    A, B = inputs.make_ab(21, 17, 26, "u11", "u11", 341)
    for (ta, tb) in TRANS:
        As, Bs = _stored(_np(A), ta), _stored(_np(B), tb)
        Ap = _np(inputs.embed(torch.from_numpy(As), As.shape[1] + 3))[:, :As.shape[1]]
        Bp = _np(inputs.embed(torch.from_numpy(Bs), Bs.shape[1] + 5))[:, :Bs.shape[1]]
        C1, _, _ = fn_ex(As, Bs, ta, tb, 1.5, 0.0, None)
        C2, _, _ = fn_ex(Ap, Bp, ta, tb, 1.5, 0.0, None)
        if not np.all(np.isfinite(C2)) or not np.array_equal(C1, C2):
            errs += _fail("ex-pitch", f"trans={ta},{tb}: C depends on the row pitch")
    return errs


EX_PINS = [pin_ex_integer_bruteforce, pin_ex_float_layouts, pin_ex_beta_zero_ignores_c,
           pin_ex_alpha_zero, pin_ex_pitch]


def run_all_ex(fn_ex):
    errs = []
    for p in EX_PINS:
        errs += p(fn_ex)
    return errs


# --- strided batch (gemm_batched contract: fn_b(A3, B3) -> (C, Cd, ABS)) ---------

def _ints3(batch, rows, cols, seed):
    return np.stack([_ints(rows, cols, seed + b) for b in range(batch)])


def pin_batched_integer_einsum(fn_b):
    """Integer batches against an int64 einsum (a library routine, exact):
    C, the binary64 sums and sum|a||b| all equal it exactly, for distinct
    matrices and for one A or one B shared by the batch (stride 0)."""
    errs = []
    for (bt, m, n, k, seed) in [(5, 7, 9, 11, 900), (3, 1, 33, 70, 910), (4, 16, 5, 1, 920)]:
        A, B = _ints3(bt, m, k, seed), _ints3(bt, k, n, seed + 50)
        cases = [("distinct", A, B),
                 ("shared A", np.broadcast_to(A[0], A.shape), B),
                 ("shared B", A, np.broadcast_to(B[0], B.shape))]
        for what, Aa, Bb in cases:
            want = np.einsum("bik,bkj->bij", Aa.astype(np.int64), Bb.astype(np.int64))
            mag = np.einsum("bik,bkj->bij", np.abs(Aa).astype(np.int64),
                            np.abs(Bb).astype(np.int64))
            C, Cd, ABS = fn_b(Aa, Bb)
            if C.shape != want.shape or not np.array_equal(C, want.astype(np.float32)):
                errs += _fail("batched-int", f"{what} {bt}x{m}x{n}x{k}: C != int64 einsum")
            elif not (np.array_equal(Cd, want.astype(np.float64)) and
                      np.array_equal(ABS, mag.astype(np.float64))):
                errs += _fail("batched-int", f"{what} {bt}x{m}x{n}x{k}: Cd or ABS inexact")
    return errs


def pin_batched_products_independent(fn_b):
    """A NaN in one product's A reaches only that product's rows; the others
    keep their exact values (products share nothing)."""
    A, B = _ints3(4, 6, 8, 940).astype(np.float32), _ints3(4, 8, 5, 950).astype(np.float32)
    A = A.copy()
    A[2, 3, 4] = np.nan
    C, _, _ = fn_b(A, B)
    want = np.einsum("bik,bkj->bij", A.astype(np.float64), B.astype(np.float64))
    bad = np.isnan(C)
    expect_bad = np.zeros_like(bad)
    expect_bad[2, 3, :] = True
    if not np.array_equal(bad, expect_bad):
        return _fail("batched-independent", "NaN spread beyond its product's row")
    ok = ~expect_bad
    if not np.array_equal(C[ok], want[ok].astype(np.float32)):
        return _fail("batched-independent", "products other than the NaN one changed")
    return []


BATCHED_PINS = [pin_batched_integer_einsum, pin_batched_products_independent]


# --- sum of an fp32 array (sum contract: fn_s(x) -> (s_f32, s_f64, abs_f64)) ------

def pin_sum_closed_forms(fn_s):
    """Sums with a closed form, exact in binary64 and in the binary32 result:
    0 + 1 + ... + (n-1) = n(n-1)/2, n ones = n, the empty sum = +0.0, and the
    cancellation 1e8 + 1 - 1e8 = 1 (lost by a binary32 running sum)."""
    errs = []
    for n in (1, 2, 7, 1000, 4097):
        s, sd, ab = fn_s(np.arange(n, dtype=np.float32))
        if sd != n * (n - 1) / 2 or s != np.float32(n * (n - 1) / 2) or ab != sd:
            errs += _fail("sum-arange", f"n={n}: got {sd}")
        s, sd, _ = fn_s(np.ones(n, dtype=np.float32))
        if sd != n or s != n:
            errs += _fail("sum-ones", f"n={n}: got {sd}")
    s, sd, ab = fn_s(np.zeros(0, dtype=np.float32))
    if not (s == 0 and not np.signbit(s) and sd == 0 and ab == 0):
        errs += _fail("sum-empty", f"got {s}")
    s, sd, _ = fn_s(np.array([1e8, 1.0, -1e8], dtype=np.float32))
    if sd != 1.0 or s != 1.0:
        errs += _fail("sum-cancel", f"1e8 + 1 - 1e8 gave {sd}")
    return errs


def pin_sum_integer_int64(fn_s):
    """Integer arrays against an int64 sum (a library routine, exact)."""
    errs = []
    for n, seed in [(1, 960), (3, 961), (1000, 962), (2 ** 20 + 3, 963)]:
        x = _ints(1, n, seed).reshape(-1)
        want = int(x.astype(np.int64).sum())
        s, sd, ab = fn_s(x)
        if sd != want or s != np.float32(want) or ab != float(np.abs(x).astype(np.int64).sum()):
            errs += _fail("sum-int", f"n={n}: got {sd}, want {want}")
    return errs


def pin_sum_fsum(fn_s):
    """Float arrays against math.fsum (the correctly rounded exact sum, a
    library routine): the binary64 sum within n 2^-53 sum|x| of it, and the
    binary32 result its rounding (within half an ulp plus that bound)."""
    import math
    errs = []
    for n, seed in [(10, 970), (12345, 971), (2 ** 18, 972)]:
        x = _np(inputs.draw_matrix(1, n, "normal", seed)).reshape(-1)
        exact = math.fsum(x.astype(np.float64))
        s, sd, ab = fn_s(x)
        if abs(sd - exact) > n * 2.0 ** -53 * ab:
            errs += _fail("sum-fsum", f"n={n}: binary64 sum {sd} vs fsum {exact}")
        if abs(float(s) - exact) > 2.0 ** -24 * abs(exact) + n * 2.0 ** -53 * ab:
            errs += _fail("sum-fsum", f"n={n}: binary32 result {s} vs fsum {exact}")
        if abs(ab - math.fsum(np.abs(x).astype(np.float64))) > n * 2.0 ** -53 * ab:
            errs += _fail("sum-fsum", f"n={n}: sum |x| wrong")
    return errs


def pin_sum_special_values(fn_s):
    """IEEE propagation: one NaN makes the sum NaN, Inf stays Inf, Inf - Inf is NaN."""
    x = _np(inputs.draw_matrix(1, 100, "u11", 980)).reshape(-1).copy()
    errs = []
    y = x.copy(); y[57] = np.nan
    if not np.isnan(fn_s(y)[0]):
        errs += _fail("sum-nan", "NaN did not propagate")
    y = x.copy(); y[3] = np.inf
    if fn_s(y)[0] != np.inf:
        errs += _fail("sum-inf", "Inf lost")
    y[90] = -np.inf
    if not np.isnan(fn_s(y)[0]):
        errs += _fail("sum-inf", "Inf - Inf is not NaN")
    return errs


SUM_PINS = [pin_sum_closed_forms, pin_sum_integer_int64, pin_sum_fsum, pin_sum_special_values]


# --- fused epilogue: act(alpha * op(A) op(B) + beta * C + bias) ----------------------
#
# ``fn_f(A, B, ta, tb, alpha, beta, C_in, bias, act) -> (C, Cd, ABS)`` with the
# contract of ``oracle.gemm_fused``.

def _relu64(x):
    return np.where(x < 0, 0, x)


def pin_fused_integer_bruteforce(fn_f):
    """Small integers, integer alpha, beta and bias, every layout, with and
    without ReLU: C equals the int64 computation exactly."""
    errs = []
    for (m, n, k, seed) in [(13, 9, 21, 1401), (5, 17, 3, 1402), (1, 6, 8, 1403)]:
        A, B = _ints(m, k, seed), _ints(k, n, seed + 10)
        Cin = _ints(m, n, seed + 20, -5, 5)
        bias = _ints(1, n, seed + 30, -9, 9).reshape(-1)
        for (ta, tb) in TRANS:
            for (alpha, beta, act) in [(1, 0, 1), (2, -1, 0), (-3, 2, 1), (0, 1, 1)]:
                C, _, _ = fn_f(_stored(A, ta), _stored(B, tb), ta, tb, float(alpha), float(beta),
                               Cin, bias, act)
                want = (alpha * _exact_int(A, B) + beta * Cin.astype(np.int64)
                        + bias.astype(np.int64)[None, :])
                if act == 1:
                    want = _relu64(want)
                if not np.array_equal(C.astype(np.int64), want):
                    errs += _fail("fused-integer", f"{m}x{n}x{k} trans={ta},{tb} "
                                                   f"alpha={alpha} beta={beta} act={act}")
    return errs


def pin_fused_bias_is_a_row_vector(fn_f):
    """With A = 0 the product vanishes: every row of C is act(bias) (M != N, so
    a bias indexed by row would not fit or would differ)."""
    errs = []
    m, n, k = 6, 10, 4
    A = np.zeros((m, k), np.float32)
    B = _np(inputs.uniform_matrix(k, n, 1411))
    bias = _np(inputs.uniform_matrix(1, n, 1412)).reshape(-1)
    for act in (0, 1):
        C, _, ABS = fn_f(A, B, False, False, 1.0, 0.0, None, bias, act)
        want = np.maximum(bias, 0) if act else bias
        if not np.array_equal(C, np.broadcast_to(want, (m, n))):
            errs += _fail("fused-bias", f"act={act}: rows are not act(bias)")
        if not np.array_equal(ABS, np.broadcast_to(np.abs(bias).astype(np.float64), (m, n))):
            errs += _fail("fused-bias", "ABS is not |bias|")
    return errs


def pin_fused_relu_of_identity(fn_f):
    """ReLU is applied last and keeps NaN: the ReLU result equals ReLU of the
    identity-activation result, element by element and bit for bit."""
    A, B = inputs.make_ab(12, 15, 40, "normal", "normal", 1421)
    A, B = _np(A).copy(), _np(B)
    A[3, 7] = np.nan
    bias = _np(inputs.uniform_matrix(1, 15, 1422)).reshape(-1)
    C0, _, _ = fn_f(A, B, False, False, 0.5, 0.0, None, bias, 0)
    C1, _, _ = fn_f(A, B, False, False, 0.5, 0.0, None, bias, 1)
    want = np.where(C0 < 0, np.float32(0), C0)
    same = (C1 == want) | (np.isnan(C1) & np.isnan(want))
    if not same.all():
        return _fail("fused-relu", "ReLU result != ReLU of the plain result (or NaN lost)")
    if not np.isnan(C1[3]).all():
        return _fail("fused-relu", "NaN row did not survive ReLU")
    return []


def pin_fused_reduces_to_ex(fn_f):
    """No bias, no activation: exactly gemm_ex (C, Cd and ABS), which the
    extended-operation pins fix."""
    import oracle
    A, B = inputs.make_ab(10, 9, 33, "u11", "normal", 1431)
    Cin = _np(inputs.uniform_matrix(10, 9, 1432))
    errs = []
    for (ta, tb) in TRANS:
        As, Bs = _stored(_np(A), ta), _stored(_np(B), tb)
        want = oracle.gemm_ex(As, Bs, trans_a=ta, trans_b=tb, alpha=1.5, beta=-0.5, C_in=Cin)
        got = fn_f(As, Bs, ta, tb, 1.5, -0.5, Cin, None, 0)
        if not all(np.array_equal(g, w) for g, w in zip(got, want)):
            errs += _fail("fused-ex", f"trans={ta},{tb}: differs from gemm_ex")
    return errs


FUSED_PINS = [pin_fused_integer_bruteforce, pin_fused_bias_is_a_row_vector,
              pin_fused_relu_of_identity, pin_fused_reduces_to_ex]
