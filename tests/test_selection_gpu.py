"""The tile table's recorded occupancies (workgroups per compute unit, which
the selection's fill model uses) against the HIP runtime's answer for the
kernels this library was built with: a kernel change that alters register
or LDS use without a re-measured table fails here."""
from __future__ import annotations

import pytest

import dense_fp32_matrix_02_amd as sg
from tests import _gpu as G
from tests._table import read_table

pytestmark = pytest.mark.gpu


def test_table_occupancy_matches_the_runtime():
    G.require_gpu()
    ids = {n: i for i, n in enumerate(sg.config_names())}
    stale = []
    for pair, (cands, _, _) in read_table().items():
        for name, occ in cands:
            got = sg.sgemm_mi355_config_occupancy(ids[name])
            print(f"[gpu] {name}: table {occ}, runtime {got}", flush=True)
            if got != occ:
                stale.append((name, occ, got))
    assert not stale, f"re-measure the tile table: {stale}"


# The library's own choice on shapes where the selection lands on each kind
# of kernel: off-grid single products (k-group, small and direct-LDS tiles,
# a direct tile whose last column of tiles is clamped), every op pair, and
# strided batches that pick the smallest tiles. Integer inputs in {-4..4}:
# exact against the oracle on every row and column of a band sample, plus
# exact row and column checksums of the whole result.

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

SINGLE = [
    (0, 0, 3072, 3072, 4096),
    (0, 0, 8192, 8000, 1024),
    (1, 0, 1000, 7000, 3000),
    (0, 1, 6144, 6144, 1024),
    (1, 1, 300, 260, 160),
    (1, 1, 4100, 3000, 2048),
]


def _stored(rows, cols, op, seed):
    """A rows x cols integer operand, stored transposed for op T."""
    X = workloads.as_numpy(workloads.draw(rows, 1, cols, seed, "int4")[0])
    return (np.ascontiguousarray(X.T) if op else X), X


@pytest.mark.parametrize("opA,opB,M,N,K", SINGLE, ids=lambda v: str(v))
def test_selected_config_off_grid_exact(opA, opB, M, N, K):
    G.require_gpu()
    As, A = _stored(M, K, opA, 31 + M)
    Bs, B = _stored(K, N, opB, 37 + N)
    cid = sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, 1)
    print(f"[gpu] selected {sg.config_names()[cid]} for ops {opA}{opB} {M}x{N}x{K}", flush=True)
    C = sg.gemm(torch.from_numpy(As).cuda(), torch.from_numpy(Bs).cuda(), opA=opA, opB=opB)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    G.check_exact_checksums(C, A, B)
    G.check_exact(C, A, B, rows=G.band_sample(M, 128, M), cols=G.band_sample(N, 128, N))


@pytest.mark.parametrize("batch,M,N,K", [(4096, 32, 32, 32), (256, 100, 100, 100), (64, 200, 300, 400),
                                         (16, 1024, 1024, 1024)], ids=lambda v: str(v))
def test_selected_config_batched_exact(batch, M, N, K):
    G.require_gpu()
    A = workloads.as_numpy(workloads.draw(batch * M, 1, K, 41 + batch, "int4")[0]).reshape(batch, M, K)
    B = workloads.as_numpy(workloads.draw(batch * K, 1, N, 43 + batch, "int4")[0]).reshape(batch, K, N)
    cid = sg.sgemm_mi355_select_config_ex(0, 0, M, N, K, batch)
    print(f"[gpu] selected {sg.config_names()[cid]} for {batch} x {M}x{N}x{K}", flush=True)
    C = sg.gemm_strided_batched(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    # every entry exactly (integer products and sums stay below 2^24), a spread of them via the oracle
    np.testing.assert_array_equal(C, np.matmul(A.astype(np.float64), B.astype(np.float64)).astype(np.float32))
    for b in sorted({0, batch // 3, batch // 2, batch - 1}):
        np.testing.assert_array_equal(C[b], oracle.sgemm_f32(A[b], B[b]))
