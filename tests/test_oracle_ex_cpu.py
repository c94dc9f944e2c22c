"""Pins of the oracle's general form C = alpha*op(A).op(B) + beta*C (no GPU).

* exact-rational brute force of the stated rounding for every op pair;
* transposed operands agree bit for bit with the (separately pinned) plain
  oracle run on transposes materialised by numpy;
* C is not read when beta == 0, A and B are not read when alpha == 0;
* the FP64 reference against exact sums and against the plain FP64 oracle;
* planted mistakes in a copy of the oracle source are each caught.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle import build as obuild
from tests._exact import exact_product, fr, sequential_f32_ex

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
SCALES = [(1.0, 0.0), (2.0, -3.0), (0.75, 0.5), (-1.5, 1.0), (0.0, 2.5), (0.0, 0.0), (1.0, 1.0)]


def stored(opX, rows, cols, seed, kind):
    """A stored array whose op is rows x cols."""
    X, _ = workloads.draw(cols if opX else rows, 1, rows if opX else cols, seed, kind)
    return workloads.as_numpy(X)


def case(opA, opB, M, N, K, seed, kind="normal"):
    A = stored(opA, M, K, seed, kind)
    B = stored(opB, K, N, seed + 1, kind)
    C0 = workloads.as_numpy(workloads.draw(M, 1, N, seed + 2, kind)[0])
    return A, B, C0


@pytest.mark.parametrize("opA,opB", OPS)
def test_bruteforce_ex_bitwise(opA, opB):
    n = 0
    for M, N, K in itertools.product((1, 2, 5), (1, 3, 4), (1, 2, 6)):
        for alpha, beta in SCALES:
            n += 1
            A, B, C0 = case(opA, opB, M, N, K, 13 * n, ("normal", "uniform", "int4")[n % 3])
            C = C0.copy()
            oracle.sgemm_ex_f32(opA, opB, alpha, A, B, beta, C)
            want = sequential_f32_ex(opA, opB, alpha, A, B, beta, C0)
            for i in range(M):
                for j in range(N):
                    assert fr(C[i, j]) == want[i][j], (opA, opB, M, N, K, alpha, beta, i, j)


@pytest.mark.parametrize("opA,opB", OPS)
def test_transposed_operands_match_plain_oracle(opA, opB):
    M, N, K = 37, 29, 53
    A, B, _ = case(opA, opB, M, N, K, 3)
    Ap = np.ascontiguousarray(A.T) if opA else A
    Bp = np.ascontiguousarray(B.T) if opB else B
    C = np.zeros((M, N), np.float32)
    oracle.sgemm_ex_f32(opA, opB, 1.0, A, B, 0.0, C)
    assert np.array_equal(C, oracle.sgemm_f32(Ap, Bp))
    P, S = oracle.sgemm_ex_f64_abs(opA, opB, A, B)
    P0, S0 = oracle.sgemm_f64_abs(Ap, Bp)
    assert np.array_equal(P, P0) and np.array_equal(S, S0)


def test_beta_zero_does_not_read_c_and_alpha_zero_does_not_read_ab():
    M, N, K = 6, 7, 5
    A, B, _ = case(0, 0, M, N, K, 5)
    C = np.full((M, N), np.nan, np.float32)
    oracle.sgemm_ex_f32(0, 0, 1.5, A, B, 0.0, C)
    assert np.isfinite(C).all()
    Anan = np.full_like(A, np.nan)
    C0 = workloads.as_numpy(workloads.draw(M, 1, N, 9, "normal")[0])
    C = C0.copy()
    oracle.sgemm_ex_f32(0, 0, 0.0, Anan, B, -2.0, C)
    assert np.array_equal(C, np.float32(-2.0) * C0)
    C = C0.copy()
    oracle.sgemm_ex_f32(0, 0, 3.0, np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), 0.5, C, K=0)
    assert np.array_equal(C, np.float32(0.5) * C0)


@pytest.mark.parametrize("opA,opB", OPS)
def test_ex_f64_exact_for_short_sums(opA, opB):
    M, N, K = 4, 5, 17
    A, B, _ = case(opA, opB, M, N, K, 21, "uniform")
    P, S = oracle.sgemm_ex_f64_abs(opA, opB, A, B)
    Cx, Sx = exact_product(np.ascontiguousarray(A.T) if opA else A, np.ascontiguousarray(B.T) if opB else B)
    for i in range(M):
        for j in range(N):
            assert Fraction(float(P[i, j])) == Cx[i][j] and Fraction(float(S[i, j])) == Sx[i][j]


def test_integer_scaled_results_are_exact():
    """Integer operands, alpha = 2, beta = -3, integer C: every intermediate is
    an integer below 2^24, so the result is the exact integer expression."""
    M, N, K = 40, 33, 300
    for opA, opB in OPS:
        A, B, C0 = case(opA, opB, M, N, K, 31, "int4")
        C = C0.copy()
        oracle.sgemm_ex_f32(opA, opB, 2.0, A, B, -3.0, C)
        Ap = A.T if opA else A
        Bp = B.T if opB else B
        exact = 2.0 * (Ap.astype(np.float64) @ Bp.astype(np.float64)) - 3.0 * C0.astype(np.float64)
        assert np.array_equal(C.astype(np.float64), exact)


EX_MUTATIONS = {
    "opA_ignored": ("return opA ? A[(size_t)k * (size_t)lda + i] : A[(size_t)i * (size_t)lda + k];",
                    "return A[(size_t)i * (size_t)lda + k];"),
    "opB_swapped": ("return opB ? B[(size_t)j * (size_t)ldb + k] : B[(size_t)k * (size_t)ldb + j];",
                    "return opB ? B[(size_t)k * (size_t)ldb + j] : B[(size_t)j * (size_t)ldb + k];"),
    "beta_term_dropped": ("                out = at + bc;", "                out = at + 0.0f * bc;"),
    "beta_read_when_zero": ("            } else if (use_ab) {\n                out = alpha * t;",
                            "            } else if (use_ab) {\n                out = alpha * t + beta * c[j];"),
    "alpha_fused": ("                float at = alpha * t;\n                float bc = beta * c[j];\n                out = at + bc;",
                    "                out = fmaf(alpha, t, beta * c[j]);"),
}


def _ex_pins_pass(lib) -> bool:
    try:
        n = 0
        for opA, opB in OPS:
            for M, N, K in [(2, 3, 4), (3, 2, 5)]:
                for alpha, beta in [(1.0, 0.0), (0.75, -0.5), (-1.5, 1.0)]:
                    n += 1
                    A, B, C0 = case(opA, opB, M, N, K, 7 * n, "normal")
                    C = C0.copy()
                    oracle.sgemm_ex_f32(opA, opB, alpha, A, B, beta, C, lib=lib)
                    want = sequential_f32_ex(opA, opB, alpha, A, B, beta, C0)
                    if any(fr(C[i, j]) != want[i][j] for i in range(M) for j in range(N)):
                        return False
        C = np.full((3, 3), np.nan, np.float32)
        A, B, _ = case(0, 0, 3, 3, 3, 99)
        oracle.sgemm_ex_f32(0, 0, 1.0, A, B, 0.0, C, lib=lib)
        return bool(np.isfinite(C).all())
    except Exception:
        return False


def test_real_oracle_passes_ex_pins():
    assert _ex_pins_pass(oracle.load())


@pytest.mark.parametrize("name", sorted(EX_MUTATIONS))
def test_planted_ex_mistake_is_caught(name, tmp_path):
    src = open(obuild.SRC).read()
    old, new = EX_MUTATIONS[name]
    assert old in src, f"mutation anchor for {name} not found"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new, 1))
    out = str(tmp_path / f"lib_{name}.so")
    obuild.compile_oracle(str(path), out, extra=("-Wno-error",))
    assert not _ex_pins_pass(oracle.load(out)), f"planted mistake {name} was not caught"
