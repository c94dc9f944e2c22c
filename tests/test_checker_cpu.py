"""Pins of the acceptance checker (``oracle.check_against_f64``,
``oracle.elementwise_bound``, ``oracle.check_ex_against_f64``), no GPU needed.

The checker decides every float-input parity verdict, so it is pinned on
crafted results whose verdict is fixed by hand-computed values, not by the
checker's own formula:

  * all-ones operands give C64 = K and sum_k |a*b| = K exactly, so the
    per-element bound 4*K*2^-23*S is an exact power of two (K = 64: 2^-9) and
    results one float32 step inside, exactly at, and one step past it are
    known to be accepted, accepted and rejected;
  * a row of 513 ones then 511 minus ones against all-ones B gives C64 = 2
    with S = 1024 (bound 0.5), so an error of 0.25 passes every element but
    is 12.5% in relative Frobenius norm, and 2^-16 / 2^-15 sit on either side
    of the 1e-5 limit;
  * a zero row of A makes S = 0: the exact result there is 0, so any nonzero
    value must be rejected, whatever its size;
  * NaN and Inf anywhere are rejected;
  * for the general form R = alpha*P + beta*C0, the product bound scales by
    |alpha| and one rounding of each term (2^-22 relative) is allowed; with
    alpha = 0 only the rounding of beta*C0 remains, which float32 arithmetic
    actually produces for beta = 0.1f.

The tolerance is the one the acceptance criterion states (4*K*2^-23 per
element, 1e-5 relative Frobenius); the pages fix only FP32 products summed in
an FP32 accumulator (GPU Parallel Book ch. 9, section 9.1; ratcatcher.ru
"Matrix multiplication: naive and tiled", section 1).

A mutation check then plants plausible mistakes in copies of the checker's
source (slack x10, the K factor dropped, |C64| in place of S, the Frobenius
term dropped, a strict comparison at the bound, S = 0 accepting anything,
the beta term or the rounding term of the general form dropped, alpha's sign
kept) and shows each one fails at least one pin.
"""
from __future__ import annotations

import inspect

import numpy as np
import pytest

import oracle

F32 = np.float32


def _ones_case(K=64, M=3, N=5):
    """C64 = K and S = K everywhere (exact); the bound is 4*K*K*2^-23."""
    A = np.ones((M, K), F32)
    B = np.ones((K, N), F32)
    C64, S = oracle.sgemm_f64_abs(A, B)
    assert np.all(C64 == K) and np.all(S == K)
    return C64, S


def _cancel_case():
    """Four rows of 513 ones then 511 minus ones, against ones(1024, 4):
    C64 = 2 and S = 1024 everywhere, bound 4*1024*1024*2^-23 = 0.5."""
    K = 1024
    A = np.ones((4, K), F32)
    A[:, 513:] = -1.0
    B = np.ones((K, 4), F32)
    C64, S = oracle.sgemm_f64_abs(A, B)
    assert np.all(C64 == 2.0) and np.all(S == 1024.0)
    return K, C64, S


# float32 values around 64 are spaced 2^-17 apart; the K = 64 bound 2^-9 is
# 256 of those steps
STEP64 = 2.0 ** -17


def _with(C64, i, j, value):
    C = C64.astype(F32).copy()
    C[i, j] = F32(value)
    assert float(C[i, j]) == value, "test value must be exact in float32"
    return C


# ---------------------------------------------------------------- plain form

def test_bound_of_all_ones_is_an_exact_power_of_two():
    _, S = _ones_case()
    assert np.all(oracle.elementwise_bound(64, S) == 2.0 ** -9)


@pytest.mark.parametrize("steps,accepted", [(0, True), (253, True), (256, True), (257, False),
                                            (259, False), (-256, True), (-257, False)])
def test_elementwise_bound_accepts_inside_and_rejects_past(steps, accepted):
    """One element moved by `steps` float32 steps of 2^-17 from C64 = 64:
    256 steps is exactly the bound (accepted), 257 is 1.004x it (rejected),
    253 is 0.988x; both signs. The relative Frobenius error stays near 1e-6."""
    C64, S = _ones_case()
    C = _with(C64, 1, 2, 64.0 + steps * STEP64)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, 64)
    assert ok is accepted, (steps, worst, rel)
    assert worst == pytest.approx(abs(steps) / 256.0, abs=0)
    assert rel < 1e-5


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
@pytest.mark.parametrize("where", ["interior", "zero_row"])
def test_nan_and_inf_are_rejected(bad, where):
    """A NaN or an infinity anywhere in C, including where S = 0 (a zero row
    of A), fails the check."""
    M, N, K = 4, 6, 32
    A = np.ones((M, K), F32)
    A[2] = 0.0  # S = 0 on row 2
    B = np.ones((K, N), F32)
    C64, S = oracle.sgemm_f64_abs(A, B)
    C = C64.astype(F32)
    i = 1 if where == "interior" else 2
    C[i, 3] = bad
    ok, _, _ = oracle.check_against_f64(C, C64, S, K)
    assert not ok


def test_frobenius_limit_rejects_what_every_element_allows():
    """C64 = 2 with S = 1024: an error of 0.25 is half the per-element bound
    but 12.5% in relative Frobenius norm."""
    K, C64, S = _cancel_case()
    C = (C64 + 0.25).astype(F32)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, K)
    assert worst == 0.5 and rel == 0.125
    assert not ok


@pytest.mark.parametrize("err,accepted", [(2.0 ** -20, True), (2.0 ** -16, True), (2.0 ** -15, False)])
def test_frobenius_limit_boundary(err, accepted):
    """A uniform error e on C64 = 2 is a relative Frobenius error of e/2: an
    error of 2^-16 (relative 2^-17 = 7.6e-6) passes the 1e-5 limit, 2^-15
    (relative 1.5e-5) does not; every element is far inside its bound of 0.5."""
    K, C64, S = _cancel_case()
    C = (C64 + err).astype(F32)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, K)
    assert rel == err / 2.0
    assert ok is accepted


def test_error_where_the_exact_result_is_zero_is_rejected():
    """A zero row of A gives S = 0 and the exact value 0: a nonzero result
    there fails however small it is (1e-30 passes the Frobenius limit), while
    -0.0 is the same value as +0.0 and passes."""
    M, N, K = 3, 4, 16
    A = np.full((M, K), 0.5, F32)
    A[1] = 0.0
    B = np.ones((K, N), F32)
    C64, S = oracle.sgemm_f64_abs(A, B)
    assert np.all(S[1] == 0.0) and np.all(C64[1] == 0.0)
    C = C64.astype(F32)
    C[1, 2] = F32(1e-30)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, K)
    assert not ok and worst == np.inf and rel < 1e-5
    C[1, 2] = F32(-0.0)
    assert oracle.check_against_f64(C, C64, S, K)[0]


def test_bound_counts_sum_of_absolute_products_not_the_result():
    """Row 0 all ones (C64 = S = 1024), row 1 the cancelling row (C64 = 2,
    S = 1024): an error of 2^-8 on row 1 is 1/128 of its bound 0.5, though 4
    times 4*K*2^-23*|C64|; the relative Frobenius error stays below 1e-5.
    Accepted."""
    K = 1024
    A = np.ones((2, K), F32)
    A[1, 513:] = -1.0
    B = np.ones((K, 4), F32)
    C64, S = oracle.sgemm_f64_abs(A, B)
    C = C64.astype(F32)
    C[1] += F32(2.0 ** -8)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, K)
    assert worst == 2.0 ** -7 and rel < 1e-5
    assert ok


def test_empty_result_is_accepted():
    C64 = np.zeros((0, 5))
    assert oracle.check_against_f64(np.zeros((0, 5), F32), C64, C64, 7)[0]


# ---------------------------------------------------------------- general form

def _ex(C, alpha, P, S, beta, C0, K):
    return oracle.check_ex_against_f64(np.asarray(C, F32), alpha, P, S, beta, C0, K)


def test_general_form_alpha_scales_the_product_bound():
    """alpha = 2, beta = 0 on all-ones, K = 64: R = 128, bound
    2*2^-9 + 2^-22*128 = 258 steps of 2^-16 (the float32 spacing at 128)."""
    P, S = _ones_case()
    C0 = np.zeros_like(P)
    step = 2.0 ** -16
    for steps, accepted in ((0, True), (258, True), (-258, True), (259, False), (-259, False)):
        C = np.full(P.shape, 128.0)
        C[0, 0] = 128.0 + steps * step
        assert _ex(C, 2.0, P, S, 0.0, C0, 64)[0] is accepted, steps


def test_general_form_negative_alpha():
    """alpha = -1: R = -64 and the bound is 2^-9 + 2^-22*64, that is 258 steps
    of 2^-17 (the float32 spacing just above 64 in magnitude)."""
    P, S = _ones_case()
    C0 = np.zeros_like(P)
    for steps, accepted in ((0, True), (258, True), (259, False)):
        C = np.full(P.shape, -64.0)
        C[2, 4] = -64.0 - steps * STEP64
        assert _ex(C, -1.0, P, S, 0.0, C0, 64)[0] is accepted, steps


def test_general_form_beta_term_is_part_of_the_reference():
    """alpha = 1, beta = 3, C0 = 5 on all-ones (K = 64): R = 64 + 15 = 79.
    The unscaled product 64 fails; 79 passes."""
    P, S = _ones_case()
    C0 = np.full(P.shape, 5.0)
    assert _ex(np.full(P.shape, 79.0), 1.0, P, S, 3.0, C0, 64)[0]
    assert not _ex(np.full(P.shape, 64.0), 1.0, P, S, 3.0, C0, 64)[0]


def test_general_form_allows_one_rounding_of_beta_times_c():
    """alpha = 0 (no product): R = beta*C0 exactly, and float32 beta*C0 for
    beta = 0.1f, C0 = 3 is off by 7.45e-9 (one rounding), within 2^-22*|R|;
    an error 16 times larger is not."""
    beta = float(F32(0.1))
    C0 = np.full((2, 3), 3.0)
    R = beta * 3.0
    c32 = float(F32(beta) * F32(3.0))
    assert c32 != R
    P = np.zeros((2, 3))
    S = np.zeros((2, 3))
    assert _ex(np.full((2, 3), c32), 0.0, P, S, beta, C0, 10)[0]
    far = float(F32(R + 16 * (c32 - R)))
    assert not _ex(np.full((2, 3), far), 0.0, P, S, beta, C0, 10)[0]


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_general_form_rejects_nan_and_inf(bad):
    P, S = _ones_case()
    C = np.full(P.shape, 64.0)
    C[1, 1] = bad
    assert not _ex(C, 1.0, P, S, 0.0, np.zeros_like(P), 64)[0]


def test_general_form_frobenius_limit():
    """alpha = 1, beta = 0 reduces to the plain check: the cancelling case with
    an error of 0.25 fails on the Frobenius limit alone."""
    K, P, S = _cancel_case()
    ok, worst, rel = _ex(P + 0.25, 1.0, P, S, 0.0, np.zeros_like(P), K)
    assert not ok and worst < 1.0 and rel == 0.125


# ---------------------------------------------------------------- mutation check

def _checker_source() -> str:
    return "\n\n".join(inspect.getsource(f) for f in (oracle.elementwise_bound, oracle.check_against_f64,
                                                      oracle.check_ex_against_f64))


def _load(src: str):
    ns = {"np": np}
    exec(compile(src, "<checker>", "exec"), ns)
    return ns


def _pins_pass(ns) -> bool:
    """A compact run of the pins above against a checker namespace."""
    chk, ex = ns["check_against_f64"], ns["check_ex_against_f64"]
    try:
        C64, S = _ones_case()
        for steps, want in ((253, True), (256, True), (257, False)):
            if chk(_with(C64, 1, 2, 64.0 + steps * STEP64), C64, S, 64)[0] is not want:
                return False
        K, P, Sc = _cancel_case()
        if chk((P + 0.25).astype(F32), P, Sc, K)[0] or not chk((P + 2.0 ** -16).astype(F32), P, Sc, K)[0]:
            return False
        A = np.ones((2, 1024), F32)
        A[1, 513:] = -1.0
        P2, S2 = oracle.sgemm_f64_abs(A, np.ones((1024, 4), F32))
        C2 = P2.astype(F32)
        C2[1] += F32(2.0 ** -8)
        if not chk(C2, P2, S2, 1024)[0]:
            return False
        A = np.full((3, 16), 0.5, F32)
        A[1] = 0.0
        P3, S3 = oracle.sgemm_f64_abs(A, np.ones((16, 4), F32))
        C3 = P3.astype(F32)
        C3[1, 2] = F32(1e-30)
        if chk(C3, P3, S3, 16)[0]:
            return False
        for bad in (np.nan, np.inf):
            C4 = C64.astype(F32)
            C4[0, 0] = bad
            if chk(C4, C64, S, 64)[0]:
                return False
        Z = np.zeros_like(C64)
        step = 2.0 ** -16
        for steps, want in ((258, True), (259, False)):
            C5 = np.full(C64.shape, 128.0, F32)
            C5[0, 0] = F32(128.0 + steps * step)
            if ex(C5, 2.0, C64, S, 0.0, Z, 64)[0] is not want:
                return False
        C6 = np.full(C64.shape, -64.0, F32)
        C6[0, 0] = F32(-64.0 - 100 * STEP64)
        if not ex(C6, -1.0, C64, S, 0.0, Z, 64)[0]:
            return False
        if ex((P + 0.25).astype(F32), 1.0, P, Sc, 0.0, np.zeros_like(P), K)[0]:
            return False
        C0 = np.full(C64.shape, 5.0)
        if not ex(np.full(C64.shape, 79.0, F32), 1.0, C64, S, 3.0, C0, 64)[0]:
            return False
        beta = float(F32(0.1))
        c32 = F32(beta) * F32(3.0)
        if not ex(np.full((2, 3), c32, F32), 0.0, np.zeros((2, 3)), np.zeros((2, 3)), beta,
                  np.full((2, 3), 3.0), 10)[0]:
            return False
        return True
    except Exception:
        return False


CHECKER_MUTATIONS = {
    "slack_x10": ("slack: float = 4.0", "slack: float = 40.0"),
    "slack_x2_unit_roundoff": ("return slack * K * (2.0 ** -23) * S", "return slack * K * (2.0 ** -22) * S"),
    "K_dropped": ("return slack * K * (2.0 ** -23) * S", "return slack * (2.0 ** -23) * S"),
    "result_in_place_of_S": ("bound = elementwise_bound(K, S)\n",
                             "bound = elementwise_bound(K, np.abs(C64))\n"),
    "frobenius_dropped": ("ok = bool(finite and worst <= 1.0 and rel <= frob_tol)",
                          "ok = bool(finite and worst <= 1.0)"),
    "strict_at_bound": ("ok = bool(finite and worst <= 1.0 and rel <= frob_tol)",
                        "ok = bool(finite and worst < 1.0 and rel <= frob_tol)"),
    "zero_bound_accepts_anything": (
        "ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))\n    worst = float(ratio.max()) "
        "if ratio.size else 0.0\n    denom = float(np.linalg.norm(C64))",
        "ratio = np.where(bound > 0, err / bound, 0.0)\n    worst = float(ratio.max()) "
        "if ratio.size else 0.0\n    denom = float(np.linalg.norm(C64))"),
    "ex_beta_term_dropped": ("R = alpha * P64 + bterm", "R = alpha * P64"),
    "ex_rounding_term_dropped": (
        "bound = abs(alpha) * elementwise_bound(K, S) + 2.0 ** -22 * (np.abs(alpha * P64) + np.abs(bterm))",
        "bound = abs(alpha) * elementwise_bound(K, S)"),
    "ex_alpha_sign_kept": ("bound = abs(alpha) * elementwise_bound(K, S)", "bound = alpha * elementwise_bound(K, S)"),
    "ex_frobenius_dropped": ("return bool(finite and worst <= 1.0 and rel <= frob_tol), worst, rel",
                             "return bool(finite and worst <= 1.0), worst, rel"),
}

# Mutations that change no verdict: NaN or Inf in C already makes the worst
# ratio and the Frobenius error NaN or Inf, so the explicit finiteness test
# is a third guard. The test below shows the mutated checker still rejects
# them (it is not a mistake the pins could or need to catch).
EQUIVALENT_MUTATIONS = {
    "finite_dropped": ("ok = bool(finite and worst <= 1.0 and rel <= frob_tol)",
                       "ok = bool(worst <= 1.0 and rel <= frob_tol)"),
}


def _mutate(name, table):
    src = _checker_source()
    old, new = table[name]
    assert old in src, f"mutation anchor for {name} not found"
    return _load(src.replace(old, new, 1))


def test_real_checker_passes_mutation_pins():
    assert _pins_pass(_load(_checker_source()))


@pytest.mark.parametrize("name", sorted(CHECKER_MUTATIONS))
def test_planted_checker_mistake_is_caught(name):
    assert not _pins_pass(_mutate(name, CHECKER_MUTATIONS)), f"planted mistake {name} was not caught"


def test_finite_guard_is_redundant_with_the_other_terms():
    ns = _mutate("finite_dropped", EQUIVALENT_MUTATIONS)
    C64, S = _ones_case()
    A = np.ones((3, 64), F32)
    A[1] = 0.0
    P0, S0 = oracle.sgemm_f64_abs(A, np.ones((64, 5), F32))
    for bad in (np.nan, np.inf, -np.inf):
        for (P, SS) in ((C64, S), (P0, S0)):
            C = P.astype(F32)
            C[1, 1] = bad
            assert not ns["check_against_f64"](C, P, SS, 64)[0]
    assert _pins_pass(ns)
