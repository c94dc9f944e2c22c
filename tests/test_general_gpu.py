"""GPU parity of the general and batched entry points against the oracle.

C = alpha*op(A).op(B) + beta*C (sgemm_mi355_ex) and its strided batch
(sgemm_mi355_strided_batched), through the C ABI. Integer operands with
integer alpha, beta and C are exact in any order and rounding pattern, so
they are compared with the oracle's general form bit for bit; float
operands must meet |C - R| <= |alpha|*4K*2^-23*S + 2^-22*(|alpha*P| + |beta*C0|)
per element (R = alpha*P64 + beta*C0 in FP64) and the relative Frobenius
bound 1e-5.
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

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()


def stored(opX, rows, cols, seed, kind):
    X, _ = workloads.draw(cols if opX else rows, 1, rows if opX else cols, seed, kind)
    return workloads.as_numpy(X)


def case(opA, opB, M, N, K, seed, kind):
    A = stored(opA, M, K, seed, kind)
    B = stored(opB, K, N, seed + 1, kind)
    C0 = workloads.as_numpy(workloads.draw(M, 1, N, seed + 2, kind)[0])
    return A, B, C0


def run_ex(opA, opB, alpha, A, B, beta, C0, config=None):
    print(f"[gpu] ex op={opA}{opB} alpha={alpha} beta={beta} C={C0.shape} config={config}", flush=True)
    Cd = torch.from_numpy(C0.copy()).to("cuda")
    sg.gemm(torch.from_numpy(A).to("cuda"), torch.from_numpy(B).to("cuda"), Cd, opA=opA, opB=opB,
            alpha=alpha, beta=beta, config=config)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


def oracle_ex(opA, opB, alpha, A, B, beta, C0):
    C = C0.copy()
    oracle.sgemm_ex_f32(opA, opB, alpha, A, B, beta, C)
    return C


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (33, 65, 17), (300, 257, 203), (513, 129, 1537)])
def test_general_integer_exact(opA, opB, M, N, K):
    A, B, C0 = case(opA, opB, M, N, K, M + N + K, "int4")
    for alpha, beta in [(1.0, 0.0), (2.0, -3.0), (-1.0, 1.0), (3.0, 0.0)]:
        C = run_ex(opA, opB, alpha, A, B, beta, C0)
        np.testing.assert_array_equal(C, oracle_ex(opA, opB, alpha, A, B, beta, C0))


@pytest.mark.parametrize("opA,opB", OPS)
def test_general_float_within_bound(opA, opB):
    M, N, K = 419, 377, 1029
    A, B, C0 = case(opA, opB, M, N, K, 11, "normal")
    P, S = oracle.sgemm_ex_f64_abs(opA, opB, A, B)
    for alpha, beta in [(1.0, 0.0), (0.75, -0.5), (-2.5, 1.25)]:
        C = run_ex(opA, opB, alpha, A, B, beta, C0)
        ok, worst, rel = oracle.check_ex_against_f64(C, alpha, P, S, beta, C0, K)
        assert ok, f"alpha={alpha} beta={beta}: bound ratio {worst:.3g}, rel {rel:.3g}"


@pytest.mark.parametrize("opA,opB", OPS)
def test_every_config_with_scaling(opA, opB):
    """Each configuration built for this op pair, forced, with alpha = 2 and
    beta = -3 on integers (exact) around its tile edges."""
    ids = [i for i in range(sg.sgemm_mi355_num_configs()) if sg.sgemm_mi355_config_ops(i) == (opA, opB)]
    assert ids
    for cid in ids:
        bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
        for M, N, K in [(bm + 1, bn - 1, bk + 3), (2 * bm + 3, bn + 1, 3 * bk + 1), (1, 2, 1)]:
            A, B, C0 = case(opA, opB, M, N, K, cid * 7 + M, "int4")
            C = run_ex(opA, opB, 2.0, A, B, -3.0, C0, config=cid)
            np.testing.assert_array_equal(C, oracle_ex(opA, opB, 2.0, A, B, -3.0, C0))


def test_beta_zero_never_reads_c_and_alpha_zero_never_reads_ab():
    M, N, K = 129, 70, 33
    A, B, _ = case(0, 0, M, N, K, 3, "int4")
    nan_c = np.full((M, N), np.nan, np.float32)
    C = run_ex(0, 0, 2.0, A, B, 0.0, nan_c)
    np.testing.assert_array_equal(C, oracle_ex(0, 0, 2.0, A, B, 0.0, np.zeros((M, N), np.float32)))
    C0 = workloads.as_numpy(workloads.draw(M, 1, N, 4, "int4")[0])
    # alpha == 0: A and B are not read, so null pointers are accepted.
    Cd = torch.from_numpy(C0.copy()).to("cuda")
    rc = sg.sgemm_mi355_ex(0, 0, M, N, K, 0.0, 0, K, 0, N, -2.0, Cd.data_ptr(), N,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == sg.OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cd.cpu().numpy(), np.float32(-2.0) * C0)
    # K == 0 with beta: C = beta * C.
    Cd = torch.from_numpy(C0.copy()).to("cuda")
    rc = sg.sgemm_mi355_ex(0, 0, M, N, 0, 1.0, 0, 1, 0, N, 0.5, Cd.data_ptr(), N,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == sg.OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cd.cpu().numpy(), np.float32(0.5) * C0)


def test_plain_ex_matches_main_entry_bitwise():
    A, B = workloads.draw(640, 576, 700, 5, "normal")
    Ad, Bd = G.dev(A), G.dev(B)
    C1 = sg.matmul(Ad, Bd)
    C2 = sg.gemm(Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("opA,opB", OPS)
def test_strided_batched_exact(opA, opB):
    batch, M, N, K = 7, 70, 45, 61
    As = [stored(opA, M, K, 100 + b, "int4") for b in range(batch)]
    Bs = [stored(opB, K, N, 200 + b, "int4") for b in range(batch)]
    Cs = [workloads.as_numpy(workloads.draw(M, 1, N, 300 + b, "int4")[0]) for b in range(batch)]
    A3 = torch.from_numpy(np.stack(As)).to("cuda")
    B3 = torch.from_numpy(np.stack(Bs)).to("cuda")
    C3 = torch.from_numpy(np.stack(Cs)).to("cuda")
    print(f"[gpu] strided batched op={opA}{opB} batch={batch}", flush=True)
    sg.gemm_strided_batched(A3, B3, C3, opA=opA, opB=opB, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    out = C3.cpu().numpy()
    for b in range(batch):
        np.testing.assert_array_equal(out[b], oracle_ex(opA, opB, 2.0, As[b], Bs[b], -1.0, Cs[b]))


def test_strided_batched_shared_operand_and_padded_strides():
    """strideA = 0 shares one A across the batch; B and C batch strides are
    larger than one matrix (gaps filled with NaN must stay untouched)."""
    batch, M, N, K = 5, 33, 40, 29
    A = stored(0, M, K, 7, "int4")
    Bs = [stored(0, K, N, 20 + b, "int4") for b in range(batch)]
    sB, sC = K * N + 13, M * N + 7
    Bbuf = torch.full((batch * sB,), float("nan"), device="cuda")
    Cbuf = torch.full((batch * sC,), float("nan"), device="cuda")
    for b in range(batch):
        Bbuf[b * sB:b * sB + K * N] = torch.from_numpy(Bs[b].reshape(-1)).to("cuda")
    Ad = torch.from_numpy(A).to("cuda")
    print("[gpu] strided batched shared A", flush=True)
    rc = sg.sgemm_mi355_strided_batched(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, 0, Bbuf.data_ptr(), N, sB,
                                        0.0, Cbuf.data_ptr(), N, sC, batch,
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == sg.OK
    torch.cuda.synchronize()
    cb = Cbuf.cpu().numpy()
    for b in range(batch):
        np.testing.assert_array_equal(cb[b * sC:b * sC + M * N].reshape(M, N), oracle.sgemm_f32(A, Bs[b]))
        if b + 1 < batch:
            assert np.isnan(cb[b * sC + M * N:(b + 1) * sC]).all()


def test_batch_beyond_one_grid():
    """More batch entries than one launch's grid.y holds (65535): the host
    splits the batch over several launches."""
    batch, M, N, K = 70001, 2, 3, 5
    A3 = torch.randint(-4, 5, (batch, M, K), generator=torch.Generator().manual_seed(1)).float()
    B3 = torch.randint(-4, 5, (batch, K, N), generator=torch.Generator().manual_seed(2)).float()
    print(f"[gpu] batch={batch}", flush=True)
    C3 = sg.gemm_strided_batched(A3.to("cuda"), B3.to("cuda"))
    torch.cuda.synchronize()
    out = C3.cpu().numpy()
    An, Bn = A3.numpy(), B3.numpy()
    for b in list(range(0, batch, 997)) + [65534, 65535, 65536, batch - 1]:
        np.testing.assert_array_equal(out[b], oracle.sgemm_f32(An[b], Bn[b]))
    # every entry: the row sums of C_b equal A_b.(B_b.1) exactly (small integers)
    np.testing.assert_array_equal(out.sum(axis=2).astype(np.float64),
                                  np.einsum("bmk,bk->bm", An.astype(np.float64), Bn.astype(np.float64).sum(axis=2)))


# ---------------------------------------------------------------- split-K

def run_splitk(opA, opB, alpha, A, B, beta, C0, splits, config=None, poison=True):
    M, N = C0.shape
    K = A.shape[0] if opA else A.shape[1]
    need = sg.sgemm_mi355_splitk_workspace_size(M, N, K, splits)
    ws = torch.full(((need + 3) // 4 + 1,), float("nan") if poison else 0.0, device="cuda")
    print(f"[gpu] splitk op={opA}{opB} M={M} N={N} K={K} splits={splits} config={config}", flush=True)
    Cd = torch.from_numpy(C0.copy()).to("cuda")
    sg.gemm_splitk(torch.from_numpy(A).to("cuda"), torch.from_numpy(B).to("cuda"), Cd, splits=splits,
                   opA=opA, opB=opB, alpha=alpha, beta=beta, workspace=ws, config=config)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


@pytest.mark.parametrize("opA,opB", OPS)
@pytest.mark.parametrize("splits", [2, 3, 4, 8, 16])
def test_splitk_integer_exact(opA, opB, splits):
    """Chunks are multiples of 32; K = 1537 leaves a short last chunk."""
    M, N, K = 197, 131, 1537
    A, B, C0 = case(opA, opB, M, N, K, splits * 5 + opA + 2 * opB, "int4")
    for alpha, beta in [(1.0, 0.0), (2.0, -3.0)]:
        C = run_splitk(opA, opB, alpha, A, B, beta, C0, splits)
        np.testing.assert_array_equal(C, oracle_ex(opA, opB, alpha, A, B, beta, C0))


@pytest.mark.parametrize("opA,opB", OPS)
def test_splitk_float_within_bound_and_deterministic(opA, opB):
    M, N, K = 256, 320, 4100
    A, B, C0 = case(opA, opB, M, N, K, 41, "normal")
    P, S = oracle.sgemm_ex_f64_abs(opA, opB, A, B)
    C = run_splitk(opA, opB, 0.5, A, B, -1.5, C0, 8)
    ok, worst, rel = oracle.check_ex_against_f64(C, 0.5, P, S, -1.5, C0, K)
    assert ok, f"bound ratio {worst:.3g}, rel {rel:.3g}"
    for _ in range(4):
        np.testing.assert_array_equal(run_splitk(opA, opB, 0.5, A, B, -1.5, C0, 8, poison=False), C)


def test_splitk_every_plain_config_and_suggested_split():
    M, N, K = 130, 97, 2050
    A, B = workloads.draw(M, N, K, 17, "int4")
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    C0 = np.zeros((M, N), np.float32)
    want = oracle.sgemm_f32(A, B)
    for cid in range(sg.sgemm_mi355_num_configs()):
        if sg.sgemm_mi355_config_ops(cid) != (0, 0):
            continue
        np.testing.assert_array_equal(run_splitk(0, 0, 1.0, A, B, 0.0, C0, 5, config=cid), want)
    # the library's own choice of split and tile
    Cd = sg.gemm_splitk(torch.from_numpy(A).to("cuda"), torch.from_numpy(B).to("cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cd.cpu().numpy(), want)


@pytest.mark.parametrize("w", [workloads.BY_NAME["square1024"], workloads.BY_NAME["ragged3001x2047x1537"]],
                         ids=lambda w: w.name)
def test_splitk_on_workloads(w):
    A, B = workloads.inputs(w, integer=True)
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    C = run_splitk(0, 0, 1.0, A, B, 0.0, np.zeros((w.M, w.N), np.float32), 4)
    G.check_exact_checksums(C, A, B)
    G.check_exact(C, A, B, rows=G.band_sample(w.M, 128, 5), cols=G.band_sample(w.N, 128, 6))
