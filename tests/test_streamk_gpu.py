"""GPU parity of the stream-K form (sgemm_mi355_streamk*) against the CPU oracle.

Every configuration with a stream-K form runs, in the operand layouts it
reads, on problems that cover the schedule's cases: tiles fewer than the
slabs the grid can take (most workgroups get nothing), tiles fewer than the
grid with ranges that cross tile boundaries, whole rounds of tiles followed
by a partial round, a partial last slab on aligned rows (added in the
epilogue of each tile's last piece), a K tail and unaligned rows (the
register-staged kernel), and alpha/beta. Integer inputs in {-4..4} are exact
in any summation order, so the result must equal the oracle bit for bit;
uniform inputs are held to the standard bound and must repeat bit for bit
(the partial sums are added in a fixed order).
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

try:  # configuration ids are read from the built library at collection time
    CONFIG_NAMES = sg.config_names()
    SK_IDS = [i for i in range(len(CONFIG_NAMES)) if sg.sgemm_mi355_config_streamk(i) == 1]
except RuntimeError:  # library not built: GPU tests fail in the fixture below
    CONFIG_NAMES, SK_IDS = [], []


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()
    yield
    torch.cuda.empty_cache()


def np_(X):
    return workloads.as_numpy(X)


def _stored(X, op):
    return X.t().contiguous() if op else X


def _streamk(A, B, cid, *, C=None, alpha=1.0, beta=0.0, lda=None, ldb=None):
    """Stream-K through configuration `cid` on CPU tensors A (M x K), B (K x N),
    stored in the layout the configuration reads, optionally in padded rows."""
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    M, N, K = A.shape[0], B.shape[1], A.shape[1]
    print(f"[gpu] streamk config={CONFIG_NAMES[cid]} M={M} N={N} K={K} lda={lda} ldb={ldb}", flush=True)
    As, Bs = _stored(A, opA), _stored(B, opB)
    Ad = G.dev(As if lda is None else workloads.embed(As, lda))[:, : As.shape[1]]
    Bd = G.dev(Bs if ldb is None else workloads.embed(Bs, ldb))[:, : Bs.shape[1]]
    Cd = None if C is None else G.dev(C)
    out = sg.gemm_streamk(Ad, Bd, Cd, opA=opA, opB=opB, alpha=alpha, beta=beta, config=cid)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("cid", SK_IDS, ids=[CONFIG_NAMES[i] for i in SK_IDS])
def test_streamk_schedules_exact(cid):
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    cases = [
        (bm + 4, bn + 4, 5 * bk),            # 4 tiles, 20 slabs: most workgroups hold none
        (3 * bm - 8, 2 * bn + 36, 70 * bk),  # 9 tiles, ranges cross tile boundaries
        (bm, bn, 3 * bk),                    # one tile in three pieces
        (2 * bm + 4, bn - 4, 33 * bk + 5),   # K tail: register staging
        (1, bn + 4, 7),                      # one row, K shorter than a slab
        (bm + 4, 1, 3 * bk),                 # one column
        (64, 64, 300 * bk),                  # one tile in pieces on every workgroup of the grid
        (bm + 4, bn + 4, 5 * bk + 4),        # aligned rows, partial last slab: added in the epilogue
        (3 * bm - 8, 2 * bn + 36, 70 * bk + 12),
        (64, 64, 300 * bk + 8),
    ]
    for i, (M, N, K) in enumerate(cases):
        A, B = workloads.draw(M, N, K, 1000 + 10 * cid + i, "int4")
        C = _streamk(A, B, cid)
        G.check_exact(C, np_(A), np_(B))


@pytest.mark.parametrize("cid", SK_IDS, ids=[CONFIG_NAMES[i] for i in SK_IDS])
def test_streamk_rounds_then_split_exact(cid):
    """More tiles than any grid the device can hold at once (4 workgroups per
    CU at most for these tiles): whole rounds run first, then the last round's
    tiles are split. Checked on sampled rows and columns and on exact row and
    column checksums of all of C."""
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    side = 1
    while (-(-side * 256 // bm)) * (-(-side * 256 // bn)) <= 4 * cus:
        side += 1
    M, N = side * 256 + 4, side * 256 - 4
    for K, seed in ((4 * bk, 31), (4 * bk + 3, 32), (4 * bk + 4, 33)):  # direct; registers; direct + tail
        A, B = workloads.draw(M, N, K, 2000 + seed + cid, "int4")
        C = _streamk(A, B, cid)
        An, Bn = np_(A), np_(B)
        G.check_exact(C, An, Bn, rows=G.band_sample(M, bm, seed), cols=G.band_sample(N, bn, seed + 1))
        G.check_exact_checksums(C, An, Bn)


@pytest.mark.parametrize("cid", SK_IDS, ids=[CONFIG_NAMES[i] for i in SK_IDS])
def test_streamk_alpha_beta_unaligned_exact(cid):
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    M, N, K = 2 * bm + 36, 3 * bn - 20, 21 * bk
    A, B = workloads.draw(M, N, K, 3000 + cid, "int4")
    C0 = workloads.draw(M, 1, N, 3500 + cid, "int4")[0]  # an M x N integer matrix
    want = np_(C0).copy()  # the oracle updates it in place; C0 itself stays the input
    oracle.sgemm_ex_f32(0, 0, 2.0, np_(A), np_(B), -1.0, want)
    got = _streamk(A, B, cid, C=C0, alpha=2.0, beta=-1.0)
    np.testing.assert_array_equal(got, want)
    # rows that are not 16-byte aligned: the register-staged stream-K kernel
    lda = (M if opA else K) + 1
    ldb = (K if opB else N) + 3
    got = _streamk(A, B, cid, lda=lda, ldb=ldb)
    G.check_exact(got, np_(A), np_(B))


@pytest.mark.parametrize("cid", SK_IDS, ids=[CONFIG_NAMES[i] for i in SK_IDS])
def test_streamk_float_bound_and_repeatable(cid):
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    M, N, K = 5 * bm + 12, 4 * bn + 8, 512
    A, B = workloads.draw(M, N, K, 4000 + cid, "uniform")
    C1 = _streamk(A, B, cid)
    C2 = _streamk(A, B, cid)
    np.testing.assert_array_equal(C1, C2)
    G.check_float(C1, np_(A), np_(B))


def test_streamk_library_choice_matches_oracle():
    """Without a configuration the library picks stream-K where its model
    predicts a gain (a 5120^3 product leaves a thin last round of 256x256
    tiles) and the plain path elsewhere; both are exact here."""
    for (M, N, K) in ((5120, 5120, 256), (1000, 1000, 1000)):
        A, B = workloads.draw(M, N, K, 77, "int4")
        cid = sg.sgemm_mi355_select_streamk(0, 0, M, N, K)
        print(f"[gpu] streamk library choice {cid} M={M} N={N} K={K}", flush=True)
        C = sg.gemm_streamk(G.dev(A), G.dev(B))
        torch.cuda.synchronize()
        C = C.cpu().numpy()
        An, Bn = np_(A), np_(B)
        G.check_exact(C, An, Bn, rows=G.band_sample(M, 256, 5), cols=G.band_sample(N, 256, 6))
        G.check_exact_checksums(C, An, Bn)
    assert sg.sgemm_mi355_select_streamk(0, 0, 5120, 5120, 5120) >= 0
    assert sg.sgemm_mi355_select_streamk(0, 0, 8192, 8192, 8192) == -1


def test_streamk_errors_and_whole_rounds():
    cid = sg.config_id("mfma32_256x256x16_w4x4_lds2")
    M = N = 600
    K = 256
    A, B = workloads.draw(M, N, K, 5, "int4")
    Ad, Bd = G.dev(A), G.dev(B)
    C = torch.empty((M, N), device="cuda")
    need = sg.sgemm_mi355_streamk_workspace_size(0, 0, M, N, K, cid)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert need > 0 and need % (8 * 256 * 256 * cus) == 0
    ws = torch.empty(need // 4 + 64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, C.data_ptr(), N)
    assert sg.sgemm_mi355_streamk_with_config(*args, ws.data_ptr(), need - 4, s, cid) == sg.ERR_WORKSPACE
    assert sg.sgemm_mi355_streamk_with_config(*args, ws.data_ptr() + 4, need, s, cid) == sg.ERR_ALIGN
    assert sg.sgemm_mi355_streamk_with_config(*args, 0, need, s, cid) == sg.ERR_NULL
    assert sg.sgemm_mi355_streamk_with_config(*args, C.data_ptr(), need, s, cid) == sg.ERR_ALIAS
    plain = sg.config_id("mfma32_256x128x16_w4x2")
    assert sg.sgemm_mi355_config_streamk(plain) == 0
    assert sg.sgemm_mi355_streamk_with_config(*args, ws.data_ptr(), need, s, plain) == sg.ERR_CONFIG
    tn = sg.config_id("mfma32_256x256x16_w4x4_lds2_tn")
    assert sg.sgemm_mi355_streamk_with_config(*args, ws.data_ptr(), need, s, tn) == sg.ERR_CONFIG
    assert sg.sgemm_mi355_streamk_with_config(*args, ws.data_ptr(), need, s, cid) == sg.OK
    torch.cuda.synchronize()
    G.check_exact(C.cpu().numpy(), np_(A), np_(B))
    # whole rounds of tiles: 256 tiles of 256x256 on 256 compute units run as the
    # plain launch and need no workspace
    if cus == 256 and sg.sgemm_mi355_streamk_workspace_size(0, 0, 4096, 4096, 64, cid) == 0:
        A, B = workloads.draw(4096, 4096, 64, 6, "int4")
        Ad, Bd = G.dev(A), G.dev(B)
        C = torch.empty((4096, 4096), device="cuda")
        rc = sg.sgemm_mi355_streamk_with_config(0, 0, 4096, 4096, 64, 1.0, Ad.data_ptr(), 64, Bd.data_ptr(),
                                                4096, 0.0, C.data_ptr(), 4096, 0, 0, s, cid)
        assert rc == sg.OK
        torch.cuda.synchronize()
        G.check_exact_checksums(C.cpu().numpy(), np_(A), np_(B))


@pytest.mark.parametrize("cid", SK_IDS, ids=[CONFIG_NAMES[i] for i in SK_IDS])
def test_streamk_random_shapes_exact(cid):
    """Seeded random shapes (M, N from 1 to 1500, K from 1 to 3000, K a
    multiple of 4 or not, rows padded or not, alpha/beta or not): every
    element exact against the oracle on integer inputs."""
    import random
    rng = random.Random(7000 + cid)
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    for case in range(6):
        M, N = rng.randint(1, 1500), rng.randint(1, 1500)
        K = rng.choice([rng.randint(1, 3000), 4 * rng.randint(1, 750)])
        pad = rng.random() < 0.3
        A, B = workloads.draw(M, N, K, 9000 + 37 * cid + case, "int4")
        lda = ((M if opA else K) + rng.randint(1, 5)) if pad else None
        ldb = ((K if opB else N) + rng.randint(1, 5)) if pad else None
        if rng.random() < 0.3:
            C0 = workloads.draw(M, 1, N, 9500 + case, "int4")[0]
            want = np_(C0).copy()
            oracle.sgemm_ex_f32(0, 0, -2.0, np_(A), np_(B), 3.0, want)
            np.testing.assert_array_equal(_streamk(A, B, cid, C=C0, alpha=-2.0, beta=3.0, lda=lda, ldb=ldb), want)
        else:
            G.check_exact(_streamk(A, B, cid, lda=lda, ldb=ldb), np_(A), np_(B))
