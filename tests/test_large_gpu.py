"""Offsets beyond 32 bits: each case puts one matrix past 2^32 elements, so
rows near its end sit at element offsets a 32-bit index would wrap. Inputs
are small integers drawn on the GPU from a seeded generator (so the host
never holds the large matrix); the oracle computes sampled rows (or columns)
of C from copies of the matching rows (or columns) of the inputs, exactly.
Sizes: C of 66000 x 66000 (17.4 GB), A of 300000 x 16384 (19.7 GB), B of
16384 x 300000 stored transposed (19.7 GB)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp32_matrix_02_amd as sg
import oracle
from tests import _gpu as G

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 32


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()
    yield
    torch.cuda.empty_cache()


def _ints(rows, cols, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(-4, 5, (rows, cols), device="cuda", generator=g, dtype=torch.float32)


def _sample(n, seed):
    r = np.random.default_rng(seed)
    return np.array(sorted({0, 1, n // 2, n - 2, n - 1, *r.integers(0, n, 6).tolist()}))


def _host(X):
    return np.ascontiguousarray(X.cpu().numpy())


def test_c_beyond_32_bit_offsets():
    M = N = 66000
    K = 16
    assert M * N > LIMIT
    A, B = _ints(M, K, 1), _ints(K, N, 2)
    An, Bn = _host(A), _host(B)
    names = sg.config_names()
    # the selected configuration (the 256x256 direct-LDS tile) and a register-staged one
    for cid in (sg.sgemm_mi355_select_config(M, N, K), sg.config_id("mfma32_256x128x16_w4x2")):
        print(f"[gpu] {names[cid]} {M}x{N}x{K}", flush=True)
        C = sg.matmul(A, B, config=cid)
        torch.cuda.synchronize()
        rows, cols = _sample(M, 3), _sample(N, 4)
        np.testing.assert_array_equal(_host(C[rows]), oracle.sgemm_f32(np.ascontiguousarray(An[rows]), Bn))
        np.testing.assert_array_equal(_host(C[:, cols]), oracle.sgemm_f32(An, np.ascontiguousarray(Bn[:, cols])))
        del C
        torch.cuda.empty_cache()


def test_a_beyond_32_bit_offsets():
    M, N, K = 300000, 64, 16384
    assert M * K > LIMIT
    A, B = _ints(M, K, 5), _ints(K, N, 6)
    Bn = _host(B)
    print(f"[gpu] {sg.config_names()[sg.sgemm_mi355_select_config(M, N, K)]} {M}x{N}x{K}", flush=True)
    C = sg.matmul(A, B)
    torch.cuda.synchronize()
    rows = _sample(M, 7)
    np.testing.assert_array_equal(_host(C[rows]), oracle.sgemm_f32(_host(A[rows]), Bn))


def test_b_transposed_beyond_32_bit_offsets():
    M, N, K = 64, 300000, 16384
    assert N * K > LIMIT
    A, Bt = _ints(M, K, 8), _ints(N, K, 9)  # op(B) = Bt^T, Bt stored N x K
    An = _host(A)
    cid = sg.sgemm_mi355_select_config_ex(0, 1, M, N, K, 1)
    print(f"[gpu] {sg.config_names()[cid]} {M}x{N}x{K} nt", flush=True)
    C = sg.gemm(A, Bt, opB=1)
    torch.cuda.synchronize()
    cols = _sample(N, 10)
    want = oracle.sgemm_f32(An, np.ascontiguousarray(_host(Bt[cols]).T))
    np.testing.assert_array_equal(_host(C[:, cols]), want)
