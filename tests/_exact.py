"""Exact-arithmetic brute force for tiny matrix products (test helper).

Independent of the C oracle: it uses Python's ``fractions.Fraction`` for exact
products and sums, and its own round-to-nearest-even into IEEE binary32, so
it shares neither code nor hardware arithmetic with ``oracle/ref_sgemm.c``.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_TWO = Fraction(2)


def round_to_f32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest IEEE binary32 value (ties to even).

    Handles normal and subnormal results; raises on overflow (the inputs used
    in the tests never come near it).
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _TWO ** e > a:
        e -= 1
    if _TWO ** (e + 1) <= a:
        e += 1
    q_exp = max(e - 23, -149)          # spacing of binary32 values near a
    scaled = a / (_TWO ** q_exp)
    q, r = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * r
    if twice > scaled.denominator or (twice == scaled.denominator and q % 2 == 1):
        q += 1
    res = Fraction(q) * (_TWO ** q_exp)
    if res >= _TWO ** 128:
        raise OverflowError("binary32 overflow")
    return sign * res


def fr(v) -> Fraction:
    return Fraction(float(v))


def exact_product(A: np.ndarray, B: np.ndarray):
    """Exact C = A.B as a nested list of Fractions, plus sum |a*b| per element."""
    M, K = A.shape
    _, N = B.shape
    Af = [[fr(A[i, k]) for k in range(K)] for i in range(M)]
    Bf = [[fr(B[k, j]) for j in range(N)] for k in range(K)]
    C = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return C, S


def sequential_f32(A: np.ndarray, B: np.ndarray):
    """FP32 sum from +0 with k ascending, each product and each add rounded
    separately to binary32: the value the oracle must reproduce bit for bit."""
    M, K = A.shape
    _, N = B.shape
    Af = [[fr(A[i, k]) for k in range(K)] for i in range(M)]
    Bf = [[fr(B[k, j]) for j in range(N)] for k in range(K)]
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s = round_to_f32(s + round_to_f32(Af[i][k] * Bf[k][j]))
            out[i][j] = s
    return out


def sequential_f32_ex(opA: int, opB: int, alpha: float, A: np.ndarray, B: np.ndarray,
                      beta: float, C: np.ndarray):
    """General form, exactly rounded: t = FP32 sum (k ascending, product and
    add rounded separately), then fl(fl(alpha*t) + fl(beta*c)); the beta term
    is absent when beta == 0 and the alpha term when alpha == 0 or K == 0."""
    opa = A.T if opA else A
    opb = B.T if opB else B
    M, K = opa.shape
    N = opb.shape[1]
    al, be = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    use_ab = al != 0 and K > 0
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            t = Fraction(0)
            if use_ab:
                for k in range(K):
                    t = round_to_f32(t + round_to_f32(fr(opa[i, k]) * fr(opb[k, j])))
            c = fr(C[i, j]) if be != 0 else Fraction(0)
            if use_ab and be != 0:
                v = round_to_f32(round_to_f32(al * t) + round_to_f32(be * c))
            elif use_ab:
                v = round_to_f32(al * t)
            elif be != 0:
                v = round_to_f32(be * c)
            else:
                v = Fraction(0)
            out[i][j] = v
    return out
