"""sgemm_mi355_splitk_noalloc against sgemm_mi355_splitk (GPU).

The entry point that allocates nothing runs the same split plan and kernels
as sgemm_mi355_splitk, with its partial sums in the library's static device
scratch instead of a caller workspace, so on the same inputs the two give
the same bits. Two calls in a row, the second on a smaller problem (the
scratch keeps the first call's partial sums, which the second must not
see), each against the workspace form; then integer inputs exact against the
oracle, alpha/beta with C read, and a problem whose partial sums fill the
scratch exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp32_matrix_02_amd as sg
import oracle
import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()


def _noalloc(Ad, Bd, C, splits, alpha=1.0, beta=0.0):
    M, K = Ad.shape
    N = Bd.shape[1]
    print(f"[gpu] splitk_noalloc M={M} N={N} K={K} splits={splits}", flush=True)
    rc = sg.sgemm_mi355_splitk_noalloc(0, 0, M, N, K, alpha, Ad.data_ptr(), K, Bd.data_ptr(), N, beta,
                                       C.data_ptr(), N, splits, torch.cuda.current_stream().cuda_stream)
    assert rc == sg.OK, sg.strerror(rc)
    return C


def test_noalloc_equals_workspace_form_twice_then_smaller():
    cases = [(384, 320, 8192, 8, 41), (96, 80, 4096, 4, 42)]
    inputs = []
    for M, N, K, splits, seed in cases:
        A, B = workloads.draw(M, N, K, seed, "uniform")
        inputs.append((G.dev(A), G.dev(B), splits))
    outs = []
    for Ad, Bd, splits in inputs:  # back to back on one stream, no sync between
        C = torch.full((Ad.shape[0], Bd.shape[1]), float("nan"), device="cuda")
        outs.append(_noalloc(Ad, Bd, C, splits))
    refs = [sg.gemm_splitk(Ad, Bd, splits=splits) for Ad, Bd, splits in inputs]
    torch.cuda.synchronize()
    for (Ad, Bd, splits), C, R in zip(inputs, outs, refs):
        assert torch.equal(C, R), f"noalloc differs from sgemm_mi355_splitk at {tuple(Ad.shape)} x {tuple(Bd.shape)}"
        G.check_float(C.cpu().numpy(), Ad.cpu().numpy(), Bd.cpu().numpy())


def test_noalloc_integer_exact_and_alpha_beta():
    M, N, K = 200, 136, 5000
    A, B = workloads.draw(M, N, K, 43, "int4")
    Ad, Bd = G.dev(A), G.dev(B)
    C = torch.empty(M, N, device="cuda")
    _noalloc(Ad, Bd, C, 5)
    torch.cuda.synchronize()
    want = oracle.sgemm_f32(workloads.as_numpy(A), workloads.as_numpy(B))
    np.testing.assert_array_equal(C.cpu().numpy(), want)
    C0 = torch.randint(-3, 4, (M, N), device="cuda").float()
    C1 = C0.clone()
    _noalloc(Ad, Bd, C1, 3, alpha=2.0, beta=-1.0)
    R = sg.gemm_splitk(Ad, Bd, C0.clone(), splits=3, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    assert torch.equal(C1, R)
    np.testing.assert_array_equal(C1.cpu().numpy(), 2.0 * want - C0.cpu().numpy())


def test_noalloc_fills_scratch_exactly_and_rejects_one_more_chunk():
    # 8 chunks of 1024 x 1024 partial sums = 32 MiB, the whole scratch
    M = N = 1024
    K = 8 * 1024
    assert sg.sgemm_mi355_splitk_workspace_size(M, N, K, 8) == sg.SCRATCH_BYTES
    A, B = workloads.draw(M, N, K, 44, "int4")
    Ad, Bd = G.dev(A), G.dev(B)
    C = torch.empty(M, N, device="cuda")
    _noalloc(Ad, Bd, C, 8)
    R = sg.gemm_splitk(Ad, Bd, splits=8)
    torch.cuda.synchronize()
    assert torch.equal(C, R)
    G.check_exact_checksums(C.cpu().numpy(), workloads.as_numpy(A), workloads.as_numpy(B))
    rc = sg.sgemm_mi355_splitk_noalloc(0, 0, M, N + 4, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0,
                                       C.data_ptr(), N, 8, 0)
    assert rc == sg.ERR_LD  # ldb < N + 4: validation comes first
    Bw = torch.zeros(K, N + 4, device="cuda")
    Cw = torch.empty(M, N + 4, device="cuda")
    rc = sg.sgemm_mi355_splitk_noalloc(0, 0, M, N + 4, K, 1.0, Ad.data_ptr(), K, Bw.data_ptr(), N + 4, 0.0,
                                       Cw.data_ptr(), N + 4, 8, 0)
    assert rc == sg.ERR_SCRATCH
