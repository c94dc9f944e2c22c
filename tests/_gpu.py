"""Helpers for GPU parity tests: run the HIP library through the C ABI and
compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp32_matrix_02_amd as sg
import oracle


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X; deselect them with -m 'not gpu'")
    sg.load()  # raises if the HIP library has not been built


def dev(X: torch.Tensor) -> torch.Tensor:
    return X.to("cuda")


def gemm(A, B, *, kind="mfma", config=None, out=None) -> np.ndarray:
    """Run the GPU path on CPU tensors A, B (copied to the device) and return C."""
    print(f"[gpu] {kind} config={config} M={A.shape[0]} N={B.shape[1]} K={A.shape[1]}", flush=True)
    Ad, Bd = dev(A), dev(B)
    C = sg.matmul(Ad, Bd, out=out, kind=kind, config=config)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def band_sample(n: int, band: int, seed: int) -> np.ndarray:
    """One random index in every band of `band` consecutive indices, plus the
    first and last index: every block tile row (or column) of size >= band is
    hit, at a random position inside it."""
    r = np.random.default_rng(seed)
    idx = {0, n - 1}
    for start in range(0, n, band):
        idx.add(int(r.integers(start, min(start + band, n))))
    return np.array(sorted(idx))


def check_float(C: np.ndarray, A: np.ndarray, B: np.ndarray, rows=None, cols=None):
    """Bound (i) per element and relative Frobenius (ii) against the FP64
    reference, on all of C or on the given rows and columns."""
    K = A.shape[1]
    results = []
    if rows is None and cols is None:
        C64, S = oracle.sgemm_f64_abs(A, B)
        results.append(oracle.check_against_f64(C, C64, S, K))
    if rows is not None:
        C64, S = oracle.sgemm_f64_abs(np.ascontiguousarray(A[rows]), B)
        results.append(oracle.check_against_f64(C[rows], C64, S, K))
    if cols is not None:
        C64, S = oracle.sgemm_f64_abs(A, np.ascontiguousarray(B[:, cols]))
        results.append(oracle.check_against_f64(C[:, cols], C64, S, K))
    for ok, worst, rel in results:
        assert ok, f"bound ratio {worst:.3g} (must be <= 1), rel. Frobenius {rel:.3g} (<= 1e-5)"
    return results


def check_exact(C: np.ndarray, A: np.ndarray, B: np.ndarray, rows=None, cols=None):
    """Integer-valued inputs: every partial sum is an exact FP32 integer, so C
    must equal the FP32 oracle (itself exact) by value, on all of C or on the
    given rows and columns."""
    if rows is None and cols is None:
        want = oracle.sgemm_f32(A, B)
        np.testing.assert_array_equal(C, want)
        return
    if rows is not None:
        want = oracle.sgemm_f32(np.ascontiguousarray(A[rows]), B)
        np.testing.assert_array_equal(C[rows], want)
    if cols is not None:
        want = oracle.sgemm_f32(A, np.ascontiguousarray(B[:, cols]))
        np.testing.assert_array_equal(C[:, cols], want)


def check_exact_checksums(C: np.ndarray, A: np.ndarray, B: np.ndarray):
    """Integer-valued inputs at any size: row sums of C equal A.(B.1) and
    column sums equal (1^T A).B exactly (all values are integers far below
    2^53 in FP64), so every element of C takes part in the check."""
    Ad, Bd = A.astype(np.float64), B.astype(np.float64)
    Cd = C.astype(np.float64)
    np.testing.assert_array_equal(Cd.sum(axis=1), Ad @ Bd.sum(axis=1))
    np.testing.assert_array_equal(Cd.sum(axis=0), Ad.sum(axis=0) @ Bd)
