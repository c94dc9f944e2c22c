"""CPU oracle for C = A.B (row-major FP32) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package. The product path (``dense_fp32_matrix_02_amd``)
never imports it, and this package imports nothing from the product.

Functions follow the plain definition of the matrix product (ratcatcher.ru
"Matrix multiplication: naive and tiled", section 1; GPU Parallel Book ch. 9,
sections 9.1-9.2; CUDA Handbook section 17.3 for general M, N, K); the
arithmetic lives in ``ref_sgemm.c``, this file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I = ctypes.c_int
_LIBS: dict = {}


def load(path: str = _build.LIB) -> ctypes.CDLL:
    """Load (building first if absent) an oracle shared library."""
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        if path != _build.LIB:
            raise FileNotFoundError(path)
        _build.build()
    lib = ctypes.CDLL(path)
    lib.ref_sgemm_f32.argtypes = [_I, _I, _I, _P, _I, _P, _I, _P, _I]
    lib.ref_sgemm_f32.restype = None
    lib.ref_sgemm_f64_abs.argtypes = [_I, _I, _I, _P, _I, _P, _I, _P, _P]
    lib.ref_sgemm_f64_abs.restype = None
    lib.ref_sgemm_ex_f32.argtypes = [_I, _I, _I, _I, _I, ctypes.c_float, _P, _I, _P, _I,
                                     ctypes.c_float, _P, _I]
    lib.ref_sgemm_ex_f32.restype = None
    lib.ref_sgemm_ex_f64_abs.argtypes = [_I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P]
    lib.ref_sgemm_ex_f64_abs.restype = None
    lib.ref_max_threads.restype = _I
    lib.ref_set_threads.argtypes = [_I]
    _LIBS[path] = lib
    return lib


def _operand(X: np.ndarray, name: str):
    """Return (pointer, ld) of a 2-D float32 array whose rows may be padded."""
    if not isinstance(X, np.ndarray) or X.dtype != np.float32 or X.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 numpy array")
    if X.shape[0] and X.shape[1] and X.strides[1] != 4:
        raise ValueError(f"{name} rows must be contiguous")
    ld = X.strides[0] // 4 if X.shape[0] > 1 else max(1, X.shape[1])
    if X.shape[0] > 1 and (X.strides[0] % 4 or ld < X.shape[1]):
        raise ValueError(f"{name} has an invalid row stride")
    return X.ctypes.data, max(ld, 1)


def sgemm_f32(A: np.ndarray, B: np.ndarray, out: np.ndarray | None = None,
              lib: ctypes.CDLL | None = None) -> np.ndarray:
    """FP32 product, FP32 accumulator from +0, k ascending, no FMA.

    A (M x K) and B (K x N) are float32 arrays with contiguous (possibly
    padded) rows; ``out`` may be a padded M x N view that receives C.
    """
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = np.empty((M, N), dtype=np.float32)
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    pc, ldc = _operand(out, "C")
    lib.ref_sgemm_f32(M, N, K, pa, lda, pb, ldb, pc, ldc)
    return out


def sgemm_f64_abs(A: np.ndarray, B: np.ndarray, lib: ctypes.CDLL | None = None):
    """Return (C64, S): the FP64-accumulated product and sum_k |a_ik*b_kj|."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C64 = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    lib.ref_sgemm_f64_abs(M, N, K, pa, lda, pb, ldb, C64.ctypes.data, S.ctypes.data)
    return C64, S


def _op_shape(X: np.ndarray, op: int):
    """Rows and columns of op(X) for a stored 2-D array X."""
    return (X.shape[1], X.shape[0]) if op else X.shape


def sgemm_ex_f32(opA: int, opB: int, alpha: float, A: np.ndarray, B: np.ndarray, beta: float,
                 C: np.ndarray, K: int | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """C = alpha*op(A).op(B) + beta*C in FP32, in place on C (M x N, rows may
    be padded). op(X) = X for op 0, X^T for op 1 (row-major storage). With
    alpha == 0 or K == 0, A and B are not read (they may be empty arrays; pass
    K explicitly then)."""
    lib = lib or load()
    M, N = C.shape
    if K is None:
        Ma, K = _op_shape(A, opA)
        Kb, Nb = _op_shape(B, opB)
        if (Ma, Kb, Nb) != (M, K, N):
            raise ValueError("operand shapes do not match C")
    pa, lda = _operand(A, "A") if A.size else (0, max(1, (M if opA else K)))
    pb, ldb = _operand(B, "B") if B.size else (0, max(1, (K if opB else N)))
    pc, ldc = _operand(C, "C")
    lib.ref_sgemm_ex_f32(opA, opB, M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc)
    return C


def sgemm_ex_f64_abs(opA: int, opB: int, A: np.ndarray, B: np.ndarray,
                     lib: ctypes.CDLL | None = None):
    """Return (P64, S): op(A).op(B) accumulated in FP64 and sum_k |a*b|."""
    lib = lib or load()
    M, K = _op_shape(A, opA)
    K2, N = _op_shape(B, opB)
    if K != K2:
        raise ValueError("inner dimensions differ")
    P = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    lib.ref_sgemm_ex_f64_abs(opA, opB, M, N, K, pa, lda, pb, ldb, P.ctypes.data, S.ctypes.data)
    return P, S


def check_ex_against_f64(C: np.ndarray, alpha: float, P64: np.ndarray, S: np.ndarray,
                         beta: float, C0: np.ndarray, K: int, frob_tol: float = 1e-5):
    """Acceptance for the general form: with R = alpha*P64 + beta*C0 (FP64),
    every |C - R| <= |alpha|*4*K*2^-23*S + 2^-22*(|alpha*P64| + |beta*C0|)
    (the product bound plus one rounding each of the scaling, the beta term
    and the sum), and ||C - R||_F / ||R||_F <= frob_tol. Returns (ok, worst,
    rel)."""
    C = np.asarray(C, dtype=np.float64)
    bterm = beta * np.asarray(C0, dtype=np.float64) if beta != 0.0 else 0.0
    R = alpha * P64 + bterm
    bound = abs(alpha) * elementwise_bound(K, S) + 2.0 ** -22 * (np.abs(alpha * P64) + np.abs(bterm))
    err = np.abs(C - R)
    finite = np.isfinite(C).all()
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    denom = float(np.linalg.norm(R))
    rel = float(np.linalg.norm(C - R)) / denom if denom > 0 else float(np.linalg.norm(C))
    return bool(finite and worst <= 1.0 and rel <= frob_tol), worst, rel


def max_threads(lib: ctypes.CDLL | None = None) -> int:
    return (lib or load()).ref_max_threads()


def set_threads(n: int, lib: ctypes.CDLL | None = None) -> None:
    (lib or load()).ref_set_threads(n)


# Acceptance criteria for a computed C against the FP64 reference (the pages
# fix FP32 arithmetic with an FP32 accumulator but no error bound; the bound
# below is the standard a-priori bound for any summation order, with slack 4).

UNIT_ROUNDOFF_F32 = 2.0 ** -24


def elementwise_bound(K: int, S: np.ndarray, slack: float = 4.0) -> np.ndarray:
    """|C - C64| <= slack * K * 2^-23 * S, per element."""
    return slack * K * (2.0 ** -23) * S


def check_against_f64(C: np.ndarray, C64: np.ndarray, S: np.ndarray, K: int,
                      frob_tol: float = 1e-5):
    """Return (ok, worst_ratio, rel_frobenius) for C against the FP64 reference.

    ok requires every |C - C64| <= 4*K*2^-23*S, C free of NaN/Inf where C64 is
    finite, and ||C - C64||_F / ||C64||_F <= frob_tol.
    """
    C = np.asarray(C, dtype=np.float64)
    err = np.abs(C - C64)
    bound = elementwise_bound(K, S)
    finite = np.isfinite(C).all()
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    denom = float(np.linalg.norm(C64))
    rel = float(np.linalg.norm(C - C64)) / denom if denom > 0 else float(np.linalg.norm(C))
    ok = bool(finite and worst <= 1.0 and rel <= frob_tol)
    return ok, worst, rel
