"""The CPU oracle against its pins, and the pins against planted mistakes.

CPU only.  The oracle must pass every pin; each mutant below (a plausible
mistake written as a small numpy variant of the oracle's contract) must fail
at least one pin, which shows the pins can tell.
"""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def oracle_fn(A, B):
    return oracle.gemm(A, B)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    errs = pin(oracle_fn)
    assert not errs, "\n".join(errs)


# ---- planted mistakes (CPU, numpy) -----------------------------------------

def _variant(mistake):
    """Oracle-like GEMM with one planted mistake."""
    def fn(A, B):
        M, K = A.shape
        N = B.shape[1]
        acc_t = np.float32 if mistake == "fp32_accumulate" else np.float64
        acc = np.zeros((M, N), acc_t)
        mag = np.zeros((M, N), np.float64)
        ks = range(K)
        if mistake == "drop_last_k":
            ks = range(max(K - 1, 0))
        if mistake == "skip_first_k":
            ks = range(1, K)
        Aeff = A
        if mistake == "ignore_lda" and M > 1 and A.strides[0] != 4 * K:
            flat = np.lib.stride_tricks.as_strided(A, shape=(M * K,), strides=(4,))
            Aeff = flat.reshape(M, K)
        for k in ks:
            a = Aeff[:, k:k + 1].astype(acc_t)
            if mistake == "transpose_b" and B.shape[0] == B.shape[1]:
                b = B[:, k:k + 1].T.astype(acc_t)
            else:
                b = B[k:k + 1, :].astype(acc_t)
            p = a * b
            if mistake == "negate_middle" and k == K // 2:
                p = -p
            if mistake == "row_shift":
                p = np.roll(p, 1, axis=0)
            acc += p
            mag += np.abs(p.astype(np.float64))
        if mistake == "abs_of_sum":
            mag = np.abs(acc.astype(np.float64))
        Cd = acc.astype(np.float64)
        if mistake == "round_toward_zero":
            C = Cd.astype(np.float32)
            over = np.abs(C.astype(np.float64)) > np.abs(Cd)
            C[over] = np.nextafter(C[over], np.float32(0))
        else:
            C = Cd.astype(np.float32)
        if mistake == "swap_operands" and A.shape[0] == A.shape[1] == B.shape[0] == B.shape[1]:
            C = (B.astype(np.float64) @ A.astype(np.float64)).astype(np.float32)
        return C, Cd, mag
    return fn


MISTAKES = ["drop_last_k", "skip_first_k", "transpose_b", "negate_middle", "row_shift",
            "fp32_accumulate", "round_toward_zero", "ignore_lda", "abs_of_sum",
            "swap_operands"]


def test_correct_variant_passes_all_pins():
    """The mutant harness itself, with no mistake, satisfies every pin."""
    errs = pins.run_all(_variant("none"))
    assert not errs, "\n".join(errs)


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    errs = pins.run_all(_variant(mistake))
    assert errs, f"no pin caught the planted mistake {mistake!r}"


# ---- direct definitional checks of the oracle's interface -------------------

def test_empty_sum_is_positive_zero():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 4), np.float32)
    C, Cd, ABS = oracle.gemm(A, B)
    assert C.shape == (3, 4) and np.all(C == 0) and not np.any(np.signbit(C))


def test_cancelling_sum_is_positive_zero():
    A = np.array([[1.0, -1.0]], np.float32)
    B = np.array([[0.75], [0.75]], np.float32)
    C, _, _ = oracle.gemm(A, B)
    assert C[0, 0] == 0 and not np.signbit(C[0, 0])


def test_empty_output():
    C, _, _ = oracle.gemm(np.zeros((0, 5), np.float32), np.ones((5, 3), np.float32))
    assert C.shape == (0, 3)


def test_nan_propagates_along_its_row():
    A = np.ones((4, 6), np.float32)
    A[2, 3] = np.nan
    C, _, _ = oracle.gemm(A, np.ones((6, 5), np.float32))
    assert np.all(np.isnan(C[2])) and np.all(np.isfinite(np.delete(C, 2, axis=0)))


def test_elems_match_full_product():
    from dense_fp32_gemm_f32_amd import inputs
    A, B = inputs.make_ab(37, 45, 61, "normal", "normal", 81, lda=64, ldb=50)
    A, B = A.numpy(), B.numpy()
    C, Cd, ABS = oracle.gemm(A, B)
    rng = np.random.default_rng(3)
    r, c = rng.integers(0, 37, 200), rng.integers(0, 45, 200)
    Ce, Cde, ABSe = oracle.gemm_elems(A, B, r, c)
    assert np.array_equal(Ce, C[r, c]) and np.array_equal(Cde, Cd[r, c])
    assert np.array_equal(ABSe, ABS[r, c])


def test_thread_count_does_not_change_result():
    from dense_fp32_gemm_f32_amd import inputs
    A, B = inputs.make_ab(64, 70, 300, "u11", "u11", 91)
    A, B = A.numpy(), B.numpy()
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        C1, Cd1, _ = oracle.gemm(A, B)
        oracle.set_threads(max(2, n0))
        C2, Cd2, _ = oracle.gemm(A, B)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(C1, C2) and np.array_equal(Cd1, Cd2)


# ---- the extended operation: alpha * op(A) op(B) + beta * C -------------------

def oracle_ex_fn(A, B, ta, tb, alpha, beta, C_in):
    return oracle.gemm_ex(A, B, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta, C_in=C_in)


@pytest.mark.parametrize("pin", pins.EX_PINS, ids=lambda p: p.__name__)
def test_oracle_ex_passes_pin(pin):
    errs = pin(oracle_ex_fn)
    assert not errs, "\n".join(errs)


def _ex_variant(mistake):
    """gemm_ex-like numpy function with one planted mistake."""
    def fn(A, B, ta, tb, alpha, beta, C_in):
        if mistake == "ignore_trans_a":
            ta_eff = False
        elif mistake == "swap_trans":
            ta_eff = tb
        else:
            ta_eff = ta
        tb_eff = ta if mistake == "swap_trans" else tb
        opa = A.T if ta_eff else A
        opb = B.T if tb_eff else B
        if opa.shape[1] != opb.shape[0]:
            opa = A.T if ta else A
            opb = B.T if tb else B
        # binary64 sum in ascending k, as the oracle's definition has it
        M, K = opa.shape
        S = np.zeros((M, opb.shape[1]), np.float64)
        mag = np.zeros_like(S)
        for k in range(K):
            p = opa[:, k:k + 1].astype(np.float64) * opb[k:k + 1, :].astype(np.float64)
            S += p
            mag += np.abs(p)
        a = np.float64(np.float32(alpha))
        b = np.float64(np.float32(beta))
        if mistake == "alpha_ignored":
            a = 1.0
        Cd = a * S
        ABS = abs(a) * mag
        if mistake == "beta_read_when_zero" or b != 0:
            c = b * C_in.astype(np.float64) if C_in is not None else 0.0
            if mistake == "beta_times_product":
                Cd = Cd * b
            else:
                Cd = Cd + c
                ABS = ABS + np.abs(c)
        return Cd.astype(np.float32), Cd, ABS
    return fn


EX_MISTAKES = ["ignore_trans_a", "swap_trans", "alpha_ignored", "beta_read_when_zero",
               "beta_times_product"]


def test_ex_correct_variant_passes_all_pins():
    errs = pins.run_all_ex(_ex_variant("none"))
    assert not errs, "\n".join(errs)


@pytest.mark.parametrize("mistake", EX_MISTAKES)
def test_ex_pins_catch_planted_mistake(mistake):
    errs = pins.run_all_ex(_ex_variant(mistake))
    assert errs, f"no pin caught the planted mistake {mistake!r}"


# ---- strided batch ------------------------------------------------------------

def oracle_batched_fn(A, B):
    return oracle.gemm_batched(A, B)


@pytest.mark.parametrize("pin", pins.BATCHED_PINS, ids=lambda p: p.__name__)
def test_oracle_batched_passes_pin(pin):
    errs = pin(oracle_batched_fn)
    assert not errs, "\n".join(errs)


def _batched_variant(mistake):
    """Batched oracle-like function with one planted mistake."""
    def fn(A, B):
        bt = A.shape[0]
        out = [oracle.gemm(A[0] if mistake == "first_a_only" else A[b],
                           B[min(b + 1, bt - 1)] if mistake == "shifted_b" else B[b])
               for b in range(bt)]
        C = np.stack([o[0] for o in out])
        Cd = np.stack([o[1] for o in out])
        ABS = np.stack([o[2] for o in out])
        if mistake == "running_sum":
            C, Cd, ABS = (np.cumsum(C, axis=0, dtype=np.float32), np.cumsum(Cd, axis=0),
                          np.cumsum(ABS, axis=0))
        return C, Cd, ABS
    return fn


BATCHED_MISTAKES = ["first_a_only", "shifted_b", "running_sum"]


@pytest.mark.parametrize("mistake", BATCHED_MISTAKES)
def test_batched_pins_catch_planted_mistake(mistake):
    errs = []
    for pin in pins.BATCHED_PINS:
        errs += pin(_batched_variant(mistake))
    assert errs, f"no batched pin caught the planted mistake {mistake!r}"


# ---- sum of an fp32 array -------------------------------------------------------

@pytest.mark.parametrize("pin", pins.SUM_PINS, ids=lambda p: p.__name__)
def test_oracle_sum_passes_pin(pin):
    errs = pin(oracle.sum_f32)
    assert not errs, "\n".join(errs)


def _sum_variant(mistake):
    """Sum-oracle-like function with one planted mistake."""
    def fn(x):
        x = np.asarray(x, dtype=np.float32)
        if mistake == "drop_last":
            x = x[:-1]
        if mistake == "skip_first":
            x = x[1:]
        if mistake == "fp32_accumulate":
            acc = np.float32(0.0)
            for v in x:
                acc = np.float32(acc + v)
            sd = float(acc)
        else:
            sd = float(np.sum(x.astype(np.float64)))
        ab = abs(sd) if mistake == "abs_of_sum" else float(np.sum(np.abs(x).astype(np.float64)))
        if mistake == "double_first" and x.size:
            sd += float(x[0])
        return np.float32(sd), sd, ab
    return fn


SUM_MISTAKES = ["drop_last", "skip_first", "fp32_accumulate", "abs_of_sum", "double_first"]


@pytest.mark.parametrize("mistake", SUM_MISTAKES)
def test_sum_pins_catch_planted_mistake(mistake):
    errs = []
    for pin in pins.SUM_PINS:
        errs += pin(_sum_variant(mistake))
    assert errs, f"no sum pin caught the planted mistake {mistake!r}"


# ---- fused epilogue: bias and activation ----------------------------------------

def oracle_fused_fn(A, B, ta, tb, alpha, beta, C_in, bias, act):
    return oracle.gemm_fused(A, B, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta, C_in=C_in,
                             bias=bias, act=act)


@pytest.mark.parametrize("pin", pins.FUSED_PINS, ids=lambda p: p.__name__)
def test_oracle_fused_passes_pin(pin):
    errs = pin(oracle_fused_fn)
    assert not errs, "\n".join(errs)


def _fused_variant(mistake):
    """gemm_fused-like function with one planted mistake, built on gemm_ex."""
    def fn(A, B, ta, tb, alpha, beta, C_in, bias, act):
        _, Cd, ABS = oracle.gemm_ex(A, B, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta,
                                    C_in=C_in)
        Cd, ABS = Cd.copy(), ABS.copy()
        relu = (lambda x: np.abs(x)) if mistake == "relu_is_abs" else \
            (lambda x: np.where(x > 0, x, 0.0)) if mistake == "relu_drops_nan" else \
            (lambda x: np.where(x < 0, 0.0, x))
        if act == 1 and mistake == "relu_before_bias":
            Cd = relu(Cd)
        if bias is not None:
            b = bias.astype(np.float64)
            if mistake == "bias_by_row":
                m = Cd.shape[0]
                bb = np.resize(b, m)[:, None]
                Cd = Cd + bb
            else:
                Cd = Cd + b[None, :] * (2 if mistake == "bias_twice" else 1)
            ABS = ABS + np.abs(b)[None, :]
        if act == 1 and mistake != "relu_before_bias":
            Cd = relu(Cd)
        return Cd.astype(np.float32), Cd, ABS
    return fn


FUSED_MISTAKES = ["relu_is_abs", "relu_drops_nan", "relu_before_bias", "bias_by_row",
                  "bias_twice"]


def test_fused_correct_variant_passes_all_pins():
    errs = []
    for pin in pins.FUSED_PINS:
        errs += pin(_fused_variant("none"))
    assert not errs, "\n".join(errs)


@pytest.mark.parametrize("mistake", FUSED_MISTAKES)
def test_fused_pins_catch_planted_mistake(mistake):
    errs = []
    for pin in pins.FUSED_PINS:
        errs += pin(_fused_variant(mistake))
    assert errs, f"no fused pin caught the planted mistake {mistake!r}"
