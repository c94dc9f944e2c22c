"""Pins of the CPU oracle against facts other than itself (no GPU needed).

The pages print no numeric example of C, so the oracle is pinned by
  * brute force in exact rational arithmetic on every tiny shape,
  * closed forms (identity, all-ones = K, K = 1 single rounded product),
  * the transpose identity (AB)^T = B^T A^T, bitwise for this summation order,
  * exact small-integer products at every workload shape (BLAS FP64 matmul,
    exact for such integers in any order, supplies the expected values),
  * the classical FP32 summation error bound against the FP64 reference,
  * and a mutation check: plausible mistakes planted in a copy of the oracle's
    C source must each fail at least one of these pins.
"""
from __future__ import annotations

import itertools
import json
import os
import shutil
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle import build as obuild
from tests._exact import exact_product, fr, sequential_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def rng_mat(rows, cols, seed, kind="uniform"):
    A, _ = workloads.draw(rows, 1, cols, seed, kind)
    return workloads.as_numpy(A)


def pair(M, N, K, seed, kind="uniform"):
    A, B = workloads.draw(M, N, K, seed, kind)
    return workloads.as_numpy(A), workloads.as_numpy(B)


# ---------------------------------------------------------------- brute force

def test_bruteforce_f32_bitwise_all_tiny_shapes():
    """Every (M, N, K) in 1..8: the FP32 oracle equals the exactly-rounded
    sequential sum (separate product and add roundings, k ascending)."""
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        seed = 100 * M + 10 * N + K
        kind = ("uniform", "normal", "int4")[seed % 3]
        A, B = pair(M, N, K, seed, kind)
        C = oracle.sgemm_f32(A, B)
        want = sequential_f32(A, B)
        for i in range(M):
            for j in range(N):
                assert fr(C[i, j]) == want[i][j], (M, N, K, kind, i, j)


def test_bruteforce_f64_exact_for_short_sums():
    """Uniform inputs are multiples of 2^-23 in [-1, 1): products are exact in
    FP64 with >= 6 spare bits, so for K <= 32 the FP64 reference and the sum of
    |a*b| are the exact rational values."""
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (8, 8, 8), (4, 3, 32), (2, 9, 17)]:
        A, B = pair(M, N, K, 7 * K + M, "uniform")
        C64, S = oracle.sgemm_f64_abs(A, B)
        Cx, Sx = exact_product(A, B)
        for i in range(M):
            for j in range(N):
                assert Fraction(float(C64[i, j])) == Cx[i][j]
                assert Fraction(float(S[i, j])) == Sx[i][j]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 3), (64, 33, 129), (257, 130, 65)])
def test_identity(M, N, K):
    A, B = pair(M, N, K, 11, "normal")
    assert np.array_equal(oracle.sgemm_f32(A, np.eye(K, dtype=np.float32)), A)
    assert np.array_equal(oracle.sgemm_f32(np.eye(K, dtype=np.float32), B), B)
    C64, _ = oracle.sgemm_f64_abs(A, np.eye(K, dtype=np.float32))
    assert np.array_equal(C64, A.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 2), (17, 9, 1537), (2, 3, 8192), (4, 4, 65537)])
def test_all_ones_is_K(M, N, K):
    """ones(M,K).ones(K,N) = K in every element (exact while K < 2^24)."""
    C = oracle.sgemm_f32(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(C == K)
    C64, S = oracle.sgemm_f64_abs(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(C64 == K) and np.all(S == K)


def test_k1_is_single_rounded_product():
    """K = 1: each element is one FP32 product a_i*b_j rounded once (numpy's
    float32 multiply is IEEE round-to-nearest-even)."""
    A, B = pair(37, 53, 1, 5, "normal")
    C = oracle.sgemm_f32(A, B)
    assert np.array_equal(C, np.multiply(A[:, :1], B[:1, :], dtype=np.float32))


def test_zero_sized():
    A = np.zeros((4, 0), np.float32)
    B = np.zeros((0, 6), np.float32)
    C = np.full((4, 6), np.nan, np.float32)
    oracle.sgemm_f32(A, B, out=C)
    assert np.all(C == 0.0)
    C0 = np.full((0, 6), np.nan, np.float32)
    oracle.sgemm_f32(np.zeros((0, 3), np.float32), np.ones((3, 6), np.float32), out=C0)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("M,N,K", [(7, 5, 3), (64, 48, 80), (129, 65, 257)])
def test_transpose_identity_bitwise(M, N, K):
    """(AB)^T = B^T A^T: the same products are summed in the same k order, so
    the oracle is bitwise equal on both sides."""
    A, B = pair(M, N, K, 3, "normal")
    C = oracle.sgemm_f32(A, B)
    Ct = oracle.sgemm_f32(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct)


def test_padded_leading_dims_ignore_padding():
    M, N, K = 33, 29, 41
    A, B = workloads.draw(M, N, K, 9, "normal")
    Ap = workloads.as_numpy(workloads.embed(A, K + 7))[:, :K]
    Bp = workloads.as_numpy(workloads.embed(B, N + 3))[:, :N]
    Cbuf = np.full((M, N + 5), -7.0, np.float32)
    out = Cbuf[:, :N]
    oracle.sgemm_f32(Ap, Bp, out=out)
    assert np.array_equal(out, oracle.sgemm_f32(workloads.as_numpy(A), workloads.as_numpy(B)))
    assert np.all(Cbuf[:, N:] == -7.0)
    C64, S = oracle.sgemm_f64_abs(Ap, Bp)
    assert np.isfinite(C64).all() and np.isfinite(S).all()


def test_thread_count_does_not_change_results():
    A, B = pair(301, 203, 157, 21, "normal")
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        C1 = oracle.sgemm_f32(A, B)
        oracle.set_threads(max(2, n0))
        Cn = oracle.sgemm_f32(A, B)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(C1, Cn)


def test_f64_reference_matches_blas():
    """The FP64 reference against numpy's BLAS product (a different summation
    order; products are exact, so only FP64 rounding separates them)."""
    A, B = pair(97, 131, 523, 13, "normal")
    C64, S = oracle.sgemm_f64_abs(A, B)
    Ad, Bd = A.astype(np.float64), B.astype(np.float64)
    scale = np.abs(Ad) @ np.abs(Bd)
    assert np.all(np.abs(C64 - Ad @ Bd) <= 1e-13 * scale)
    assert np.allclose(S, scale, rtol=1e-13, atol=0)


# ------------------------------------------------ integer exactness, all shapes

def _rows_sample(M, count, seed):
    r = np.random.default_rng(seed)
    rows = set(r.choice(M, size=min(count, M), replace=False).tolist())
    rows.update({0, M - 1})
    return np.array(sorted(rows))


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_integer_variant_exact_at_workload_shapes(w):
    """Entries in {-4..4}: every partial sum is an integer of magnitude at most
    16*K < 2^24, so the FP32 oracle must equal the exact product. The exact
    values come from a BLAS FP64 product (exact for these integers in any
    order). Large shapes are checked on a sample of rows."""
    A, B = workloads.inputs(w, integer=True)
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    rows = np.arange(w.M) if w.M * w.N * w.K <= 2 ** 30 else _rows_sample(w.M, 12, w.seed)
    As = np.ascontiguousarray(A[rows])
    C = oracle.sgemm_f32(As, B)
    exact = As.astype(np.float64) @ B.astype(np.float64)
    assert np.array_equal(C.astype(np.float64), exact)


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_f32_oracle_within_classical_bound(w):
    """Recursive FP32 summation of K rounded products is within
    gamma_K * sum|a*b| of the exact value, gamma_K = K u / (1 - K u), u = 2^-24
    (the standard dot-product error bound). Against the acceptance bound
    4*K*2^-23*sum|a*b| this is a ratio of at most about 1/8."""
    A, B = workloads.inputs(w)
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    rows = np.arange(w.M) if w.M * w.N * w.K <= 2 ** 28 else _rows_sample(w.M, 6, w.seed + 1)
    As = np.ascontiguousarray(A[rows])
    C = oracle.sgemm_f32(As, B)
    C64, S = oracle.sgemm_f64_abs(As, B)
    u = 2.0 ** -24
    gamma = w.K * u / (1 - w.K * u)
    assert np.all(np.abs(C.astype(np.float64) - C64) <= gamma * S)
    ok, worst, rel = oracle.check_against_f64(C, C64, S, w.K)
    assert ok and worst <= 0.126 and rel <= 1e-5


# ---------------------------------------------------------------- page figures

def test_page_figures_fix_the_accounting():
    g = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))
    n = g["arithmetic_intensity_n4096"]["N"]
    w = workloads.Workload("sq", n, n, n, n, n, n, "uniform", 0)
    assert w.flops == 2 * n ** 3
    assert w.min_bytes == 12 * n ** 2
    assert round(w.flops / w.min_bytes) == g["arithmetic_intensity_n4096"]["value"]


# ---------------------------------------------------------------- mutation check

def _pins_pass(lib) -> bool:
    """A compact run of the pins above against a given oracle library."""
    try:
        for M, N, K in [(3, 4, 5), (2, 7, 3), (5, 2, 8)]:
            A, B = pair(M, N, K, M + N + K, "normal")
            C = oracle.sgemm_f32(A, B, lib=lib)
            want = sequential_f32(A, B)
            if any(fr(C[i, j]) != want[i][j] for i in range(M) for j in range(N)):
                return False
            A, B = pair(M, N, K, 5, "uniform")
            C64, S = oracle.sgemm_f64_abs(A, B, lib=lib)
            Cx, Sx = exact_product(A, B)
            if any(Fraction(float(C64[i, j])) != Cx[i][j] or Fraction(float(S[i, j])) != Sx[i][j]
                   for i in range(M) for j in range(N)):
                return False
        A, B = workloads.draw(9, 6, 11, 4, "normal")
        Ap = workloads.as_numpy(workloads.embed(A, 16))[:, :11]
        I = np.eye(11, dtype=np.float32)
        if not np.array_equal(oracle.sgemm_f32(Ap, I, lib=lib), workloads.as_numpy(A)):
            return False
        if not np.all(oracle.sgemm_f32(np.ones((3, 70), np.float32), np.ones((70, 2), np.float32), lib=lib) == 70):
            return False
        return True
    except Exception:
        return False


MUTATIONS = {
    "drop_last_term": ("const float aik = a[k];", "const float aik = (k + 1 < K) ? a[k] : 0.0f;"),
    "transposed_B": ("float p = aik * b[j];", "float p = aik * B[(size_t)j * (size_t)ldb + k];"),
    "sign": ("c[j] = c[j] + p;", "c[j] = c[j] - p;"),
    "fused_multiply_add": ("float p = aik * b[j];\n                c[j] = c[j] + p;",
                           "c[j] = fmaf(aik, b[j], c[j]);"),
    "lda_as_K": ("const float *a = A + (size_t)i * (size_t)lda;", "const float *a = A + (size_t)i * (size_t)K;"),
    "abs_dropped": ("s[j] = s[j] + fabs(p);", "s[j] = s[j] + p;"),
    "f64_first_term_dropped": ("double p = aik * (double)b[j];",
                               "double p = (k > 0) ? aik * (double)b[j] : 0.0;"),
}


def test_real_oracle_passes_mutation_pins():
    assert _pins_pass(oracle.load())


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(obuild.SRC).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    out = str(tmp_path / f"lib_{name}.so")
    obuild.compile_oracle(str(path), out, extra=("-Wno-error",))
    lib = oracle.load(out)
    assert not _pins_pass(lib), f"planted mistake {name} was not caught"
