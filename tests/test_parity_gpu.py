"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Tolerances (the pages fix FP32 products with an FP32 accumulator but no
summation order, so any order within the standard bound is correct):
  * float inputs: |C - C64| <= 4*K*2^-23*sum_k|a_ik*b_kj| per element and
    ||C - C64||_F / ||C64||_F <= 1e-5, C64 the FP64-accumulated reference;
  * integer inputs in {-4..4}: exact (every partial sum is an integer below
    2^24, so every order gives the same FP32 value).
Full-size workloads run in the configuration the library selects (the one
the benchmark times) and are checked on one random row and one random
column in every band of 128, plus exact row/column checksums of the whole
result for the integer variant.
"""
from __future__ import annotations

import re
import numpy as np
import pytest
import torch

import dense_fp32_matrix_02_amd as sg
import oracle
import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu

KINDS = ["mfma", "valu"]

try:  # configuration ids are read from the built library at collection time
    CONFIG_NAMES = sg.config_names()
except RuntimeError:  # library not built: GPU tests fail in the fixture below
    CONFIG_NAMES = []
CONFIG_IDS = list(range(len(CONFIG_NAMES)))


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()


def np_(X):
    return workloads.as_numpy(X)


# --------------------------------------------------------------- workloads

@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_workload_float(w, kind):
    A, B = workloads.inputs(w)
    C = G.gemm(A, B, kind=kind)
    A, B = np_(A), np_(B)
    assert np.isfinite(C).all()
    if w.M * w.N * w.K <= 10 ** 10:  # every element (the ragged workload included)
        G.check_float(C, A, B)
    else:
        G.check_float(C, A, B, rows=G.band_sample(w.M, 128, w.seed),
                      cols=G.band_sample(w.N, 128, w.seed + 1))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_workload_integer_exact(w, kind):
    A, B = workloads.inputs(w, integer=True)
    C = G.gemm(A, B, kind=kind)
    A, B = np_(A), np_(B)
    G.check_exact_checksums(C, A, B)
    if w.M * w.N * w.K <= 2 ** 30:
        G.check_exact(C, A, B)
    else:
        G.check_exact(C, A, B, rows=G.band_sample(w.M, 128, w.seed + 2),
                      cols=G.band_sample(w.N, 128, w.seed + 3))


# --------------------------------------------------------------- every config, every edge

def _edge_sizes(tile):
    # tile - 1, tile + 1, tile + 2 and 2 * tile + 3 leave 3, 1, 2 and 3 values
    # of the last 4-value chunk of a line inside the matrix.
    return sorted({1, 2, 3, tile - 1, tile, tile + 1, tile + 2, 2 * tile + 3})


def _stored(X, op):
    """The array to pass for op(X) = X (op 0) or X^T (op 1)."""
    return X.t().contiguous() if op else X


def _run_config(A, B, cid):
    """C = A.B through the configuration `cid`, with A and B stored in the
    layout the configuration reads (transposed copies for its T operands)."""
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    print(f"[gpu] config={CONFIG_NAMES[cid]} M={A.shape[0]} N={B.shape[1]} K={A.shape[1]}", flush=True)
    C = sg.gemm(G.dev(_stored(A, opA)), G.dev(_stored(B, opB)), opA=opA, opB=opB, config=cid)
    torch.cuda.synchronize()
    return C.cpu().numpy()


@pytest.mark.parametrize("cid", CONFIG_IDS, ids=CONFIG_NAMES)
def test_every_config_edges_exact(cid):
    """Every compiled configuration, forced, on M, N around its block tile and
    K around its slab depth: integer inputs, bit-exact against the oracle."""
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    Ms, Ns = _edge_sizes(bm), _edge_sizes(bn)
    Ks = sorted({1, 2, 7, bk - 1, bk, bk + 1, 2 * bk + 5, 8 * bk + 3})
    seed = 0
    for M in Ms:
        for N in Ns:
            for K in (Ks if (M in (1, bm + 1) or N in (1, bn + 1)) else Ks[::3]):
                seed += 1
                A, B = workloads.draw(M, N, K, seed, "int4")
                C = _run_config(A, B, cid)
                G.check_exact(C, np_(A), np_(B))


@pytest.mark.parametrize("cid", CONFIG_IDS, ids=CONFIG_NAMES)
def test_every_config_float_ragged(cid):
    A, B = workloads.draw(301, 257, 203, 77, "normal")
    C = _run_config(A, B, cid)
    G.check_float(C, np_(A), np_(B))


# --------------------------------------------------------------- layouts

@pytest.mark.parametrize("kind", KINDS)
def test_padded_leading_dims_and_untouched_padding(kind):
    M, N, K = 197, 143, 263
    A, B = workloads.draw(M, N, K, 5, "int4")
    Ap = G.dev(workloads.embed(A, K + 5))         # NaN in the padding
    Bp = G.dev(workloads.embed(B, N + 3))
    Cbuf = torch.full((M, N + 7), 123.0, device="cuda")
    sg.matmul(Ap[:, :K], Bp[:, :N], out=Cbuf[:, :N], kind=kind)
    torch.cuda.synchronize()
    Cb = Cbuf.cpu().numpy()
    assert np.all(Cb[:, N:] == 123.0), "padding columns of C were written"
    G.check_exact(np.ascontiguousarray(Cb[:, :N]), np_(A), np_(B))


@pytest.mark.parametrize("kind", KINDS)
def test_misaligned_bases_and_odd_leading_dims(kind):
    """Bases 4 bytes past a 16-byte boundary and odd leading dimensions: the
    path needs only 4-byte alignment."""
    M, N, K = 131, 97, 77
    A, B = workloads.draw(M, N, K, 8, "int4")
    lda, ldb, ldc = K + 2, N + 4, N + 1
    abuf = torch.full((M * lda + 1,), float("nan"), device="cuda")
    bbuf = torch.full((K * ldb + 3,), float("nan"), device="cuda")
    cbuf = torch.full((M * ldc + 1,), float("nan"), device="cuda")
    Av = abuf[1:1 + M * lda].view(M, lda)
    Bv = bbuf[3:3 + K * ldb].view(K, ldb)
    Cv = cbuf[1:1 + M * ldc].view(M, ldc)
    Av[:, :K] = G.dev(A)
    Bv[:, :N] = G.dev(B)
    fn = sg.sgemm_mi355 if kind == "mfma" else sg.sgemm_mi355_valu
    rc = fn(M, N, K, Av.data_ptr(), lda, Bv.data_ptr(), ldb, Cv.data_ptr(), ldc,
            torch.cuda.current_stream().cuda_stream)
    assert rc == sg.OK
    torch.cuda.synchronize()
    C = Cv[:, :N].cpu().numpy()
    G.check_exact(np.ascontiguousarray(C), np_(A), np_(B))
    assert np.isnan(Cv[:, N:].cpu().numpy()).all()


@pytest.mark.parametrize("kind", KINDS)
def test_nan_prefilled_output_is_overwritten(kind):
    """beta = 0: C is never read, so NaN already in C cannot leak into it."""
    A, B = workloads.draw(256, 320, 96, 9, "uniform")
    out = torch.full((256, 320), float("nan"), device="cuda")
    C = G.gemm(A, B, kind=kind, out=out)
    assert np.isfinite(C).all()
    G.check_float(C, np_(A), np_(B))


# --------------------------------------------------------------- closed forms and invariants

@pytest.mark.parametrize("kind", KINDS)
def test_identity_and_all_ones(kind):
    M, N, K = 300, 260, 1537
    A, _ = workloads.draw(M, 1, K, 10, "normal")
    C = G.gemm(A, torch.eye(K), kind=kind)
    np.testing.assert_array_equal(C, np_(A))
    C = G.gemm(torch.ones(M, K), torch.ones(K, N), kind=kind)
    assert np.all(C == K)


@pytest.mark.parametrize("kind", KINDS)
def test_k1_is_single_rounded_product(kind):
    A, B = workloads.draw(130, 200, 1, 11, "normal")
    C = G.gemm(A, B, kind=kind)
    np.testing.assert_array_equal(C, np.multiply(np_(A), np_(B), dtype=np.float32))


@pytest.mark.parametrize("kind", KINDS)
def test_k0_gives_zero_and_empty_is_noop(kind):
    out = torch.full((33, 65), float("nan"), device="cuda")
    C = G.gemm(torch.zeros(33, 0), torch.zeros(0, 65), kind=kind, out=out)
    assert np.all(C == 0.0)
    out0 = torch.full((0, 5), 1.0, device="cuda")
    G.gemm(torch.zeros(0, 3), torch.ones(3, 5), kind=kind, out=out0)


@pytest.mark.parametrize("kind", KINDS)
def test_transpose_identity(kind):
    A, B = workloads.draw(213, 171, 389, 12, "int4")
    C = G.gemm(A, B, kind=kind)
    Ct = G.gemm(B.t().contiguous(), A.t().contiguous(), kind=kind)
    np.testing.assert_array_equal(C.T, Ct)
    A, B = workloads.draw(213, 171, 389, 13, "normal")
    Ct = G.gemm(B.t().contiguous(), A.t().contiguous(), kind=kind)
    G.check_float(np.ascontiguousarray(Ct.T), np_(A), np_(B))


@pytest.mark.parametrize("kind", KINDS)
def test_power_of_two_scaling_is_bitwise(kind):
    A, B = workloads.draw(384, 320, 515, 14, "normal")
    C = G.gemm(A, B, kind=kind)
    C2 = G.gemm(2.0 * A, B, kind=kind)
    Ch = G.gemm(A, 0.5 * B, kind=kind)
    np.testing.assert_array_equal(C2, 2.0 * C)
    np.testing.assert_array_equal(Ch, 0.5 * C)


EDGE_ALIGNED = workloads.Workload("edge4036x3972x4096", 4036, 3972, 4096, 4096, 3972, 3972, "uniform", 16)


@pytest.mark.parametrize("w", [workloads.BY_NAME["square1024"], workloads.BY_NAME["ragged3001x2047x1537"],
                               workloads.BY_NAME["square4096"], EDGE_ALIGNED], ids=lambda w: w.name)
def test_repeated_runs_are_bitwise_identical(w):
    """Ten more runs on the same float inputs give the same bits over all of C
    (the summation order is fixed; a race between the loads of the next slab
    and the reads of the current one would show as differences). The two
    aligned shapes run the direct-to-LDS pipeline, the second with edge tiles
    in M and N."""
    A, B = workloads.inputs(w)
    Ad, Bd = G.dev(A), G.dev(B)
    cid = sg.sgemm_mi355_selected_config(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N)
    print(f"[gpu] repeated runs {w.name} config={CONFIG_NAMES[cid]}", flush=True)
    if w.name in ("square4096", EDGE_ALIGNED.name):
        assert sg.sgemm_mi355_config_staging(cid, w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N) == 1
    first = sg.matmul(Ad, Bd)
    for _ in range(10):
        again = sg.matmul(Ad, Bd)
        assert torch.equal(first, again)
    if w is EDGE_ALIGNED:
        C = first.cpu().numpy()
        An, Bn = np_(A), np_(B)
        G.check_float(C, An, Bn, rows=G.band_sample(w.M, 128, 21), cols=G.band_sample(w.N, 128, 22))


def test_workspace_of_a_side_stream_call_outlives_the_call():
    """Split-K and stream-K on a stream that is not the current one, the
    wrapper allocating C and the workspace: right after the calls return, a
    buffer of the workspace's size is allocated and filled on the current
    stream before anything is synchronised. The workspace and C belong to the
    launch stream's pool, so that buffer cannot be carved out of them while
    the kernels still run, and the results stay exact."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    M, N, K = 96, 80, 8192
    A, B = workloads.draw(M, N, K, 31, "int4")
    Ad, Bd = G.dev(A), G.dev(B)
    side.wait_stream(cur)
    need = sg.sgemm_mi355_splitk_workspace_size(M, N, K, 8)
    C1 = sg.gemm_splitk(Ad, Bd, splits=8, stream=side)
    junk = torch.full((need // 4 + M * N,), 7.0, device="cuda")
    sk_cfg = sg.config_id("mfma32_256x256x16_w4x4_lds2")
    M2, N2, K2 = 768, 768, 2048
    A2, B2 = workloads.draw(M2, N2, K2, 32, "int4")
    A2d, B2d = G.dev(A2), G.dev(B2)
    side.wait_stream(cur)
    need2 = sg.sgemm_mi355_streamk_workspace_size(0, 0, M2, N2, K2, sk_cfg)
    assert need2 > 0
    C2 = sg.gemm_streamk(A2d, B2d, config=sk_cfg, stream=side)
    junk2 = torch.full((need2 // 4 + M2 * N2,), -3.0, device="cuda")
    side.synchronize()
    torch.cuda.synchronize()
    assert float(junk[0]) == 7.0 and float(junk2[-1]) == -3.0
    G.check_exact(C1.cpu().numpy(), np_(A), np_(B))
    G.check_exact(C2.cpu().numpy(), np_(A2), np_(B2))


def test_runs_on_a_side_stream():
    A, B = workloads.draw(512, 384, 640, 15, "int4")
    Ad, Bd = G.dev(A), G.dev(B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty(512, 384, device="cuda")
        sg.matmul(Ad, Bd, out=out, stream=s)
    s.synchronize()
    G.check_exact(out.cpu().numpy(), np_(A), np_(B))


@pytest.mark.parametrize("kind", KINDS)
def test_very_long_k_exact(kind):
    """K of about a million with a tiny ragged M x N: tens of thousands of
    slabs in one workgroup (k-group tiles on the matrix-core path), and the
    same product as 64 split-K chunks. Integer inputs in {-4..4} keep every
    partial sum below 2^24, so both are exact."""
    M, N, K = 33, 47, 1_000_003
    A, B = workloads.draw(M, N, K, 91, "int4")
    An, Bn = np_(A), np_(B)
    want = oracle.sgemm_f32(An, Bn)
    C = G.gemm(A, B, kind=kind)
    np.testing.assert_array_equal(C, want)
    if kind == "mfma":
        print(f"[gpu] split-K 64 chunks M={M} N={N} K={K}", flush=True)
        Cs = sg.gemm_splitk(G.dev(A), G.dev(B), splits=64)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Cs.cpu().numpy(), want)


DIRECT_IDS = [i for i, n in enumerate(CONFIG_NAMES) if "_lds" in n]


SCHED_IDS = [i for i, n in enumerate(CONFIG_NAMES) if n.endswith("_sched")]


@pytest.mark.parametrize("cid", SCHED_IDS, ids=[CONFIG_NAMES[i] for i in SCHED_IDS])
def test_hand_ordered_loop_repeats_bitwise(cid):
    """The one-wave-per-SIMD loop publishes each slab with a barrier two
    groups before the end of the previous one and starts the next slab's
    loads right after it: ten runs on float inputs over many slabs and edge
    tiles give the same bits over all of C, and the result is within the
    bound of the FP64 oracle."""
    M, N, K = 1100, 1020, 2048
    A, B = workloads.draw(M, N, K, 31, "uniform")
    Ad, Bd = G.dev(A), G.dev(B)
    direct = 1 if "_lds" in CONFIG_NAMES[cid] else 0  # _rs: staged through registers
    assert sg.sgemm_mi355_config_staging(cid, M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N) == direct
    print(f"[gpu] repeated runs config={CONFIG_NAMES[cid]} M={M} N={N} K={K}", flush=True)
    first = sg.gemm(Ad, Bd, config=cid)
    for _ in range(10):
        again = sg.gemm(Ad, Bd, config=cid)
        torch.cuda.synchronize()
        assert torch.equal(first, again)
    G.check_float(first.cpu().numpy(), np_(A), np_(B))



@pytest.mark.parametrize("cid", DIRECT_IDS, ids=[CONFIG_NAMES[i] for i in DIRECT_IDS])
def test_direct_lds_configs_exact(cid):
    """Configurations that stage slabs with direct global-to-LDS loads take
    that path only for 16-byte aligned operands, K of at least one slab (a
    partial last slab is staged through registers) and, for a line-contiguous
    operand (B, or A^T), its extent a multiple of 4; lines past the edge of C
    are clamped. Exercise it with ragged M and N (multiples of 4 and not),
    slab counts that leave every remainder of the stage count, a partial last
    slab, then a batch and split-K chunkings, all exact on integer inputs, in
    the operand layouts the configuration reads."""
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    seed = 500
    for M in (1, 4, bm - 1, bm + 4, 2 * bm):
        for N in (2 * bn, bn + 36, 4, bn - 3):
            for slabs in ((1, 2, 3, 7, 32) if N == 2 * bn else (1, 5)):
                seed += 1
                A, B = workloads.draw(M, N, slabs * bk, seed, "int4")
                C = _run_config(A, B, cid)
                G.check_exact(C, np_(A), np_(B))
    # strided batch of 3 entries (16-byte aligned strides)
    batch, M, N, K = 3, bm + 4, bn + 12, 9 * bk
    A = torch.stack([_stored(workloads.draw(M, N, K, 700 + b, "int4")[0], opA) for b in range(batch)])
    B = torch.stack([_stored(workloads.draw(M, N, K, 800 + b, "int4")[1], opB) for b in range(batch)])
    print(f"[gpu] config={CONFIG_NAMES[cid]} batch={batch} M={M} N={N} K={K}", flush=True)
    C = sg.gemm_strided_batched(G.dev(A), G.dev(B), opA=opA, opB=opB, config=cid)
    torch.cuda.synchronize()
    for b in range(batch):
        Ab = np_(A[b]).T if opA else np_(A[b])
        Bb = np_(B[b]).T if opB else np_(B[b])
        np.testing.assert_array_equal(C[b].cpu().numpy(),
                                      oracle.sgemm_f32(np.ascontiguousarray(Ab), np.ascontiguousarray(Bb)))
    # split-K: chunks of 32 slabs, the last one short but whole slabs
    M, N, K = bm - 8, bn, 70 * bk
    A, B = workloads.draw(M, N, K, 900, "int4")
    print(f"[gpu] config={CONFIG_NAMES[cid]} split-K M={M} N={N} K={K}", flush=True)
    Cs = sg.gemm_splitk(G.dev(_stored(A, opA)), G.dev(_stored(B, opB)), splits=3, opA=opA, opB=opB, config=cid)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cs.cpu().numpy(), oracle.sgemm_f32(np_(A), np_(B)))
    # K not a whole number of slabs (rows still 16-byte aligned): direct loads
    # for the whole slabs, the last one staged through registers; K of one
    # slab and a bit, every stage remainder, and a split-K whose chunks all end
    # in a partial slab
    for slabs in (1, 2, 3, 7):
        for r in (4, bk - 4):
            seed += 1
            M, N, K = bm + 4, bn - 4, slabs * bk + r
            A, B = workloads.draw(M, N, K, seed, "int4")
            G.check_exact(_run_config(A, B, cid), np_(A), np_(B))
    batch, M, N, K = 3, bm + 4, bn + 12, 9 * bk + 8  # a batch whose entries end in a partial slab
    A = torch.stack([_stored(workloads.draw(M, N, K, 960 + b, "int4")[0], opA) for b in range(batch)])
    B = torch.stack([_stored(workloads.draw(M, N, K, 970 + b, "int4")[1], opB) for b in range(batch)])
    print(f"[gpu] config={CONFIG_NAMES[cid]} batch={batch} M={M} N={N} K={K}", flush=True)
    C = sg.gemm_strided_batched(G.dev(A), G.dev(B), opA=opA, opB=opB, config=cid)
    torch.cuda.synchronize()
    for b in range(batch):
        Ab = np_(A[b]).T if opA else np_(A[b])
        Bb = np_(B[b]).T if opB else np_(B[b])
        np.testing.assert_array_equal(C[b].cpu().numpy(),
                                      oracle.sgemm_f32(np.ascontiguousarray(Ab), np.ascontiguousarray(Bb)))
    M, N, K = bm - 8, bn + 12, 70 * bk + 4
    A, B = workloads.draw(M, N, K, 950, "int4")
    print(f"[gpu] config={CONFIG_NAMES[cid]} split-K, partial slabs M={M} N={N} K={K}", flush=True)
    Cs = sg.gemm_splitk(G.dev(_stored(A, opA)), G.dev(_stored(B, opB)), splits=3, opA=opA, opB=opB, config=cid)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Cs.cpu().numpy(), oracle.sgemm_f32(np_(A), np_(B)))


# the register-staged configurations, and the direct ones, whose misaligned
# operands run the same hand-ordered loop staged through registers
SCHED_IDS = [i for i, n in enumerate(CONFIG_NAMES) if n.endswith("_sched") or "_sched_" in n]


@pytest.mark.parametrize("cid", SCHED_IDS, ids=[CONFIG_NAMES[i] for i in SCHED_IDS])
def test_register_staged_hand_ordered_any_alignment(cid):
    """The hand-ordered loop staged through registers takes bases at any
    4-byte offset, odd leading dimensions and extents that are not multiples
    of 4, in the operand layouts the configuration reads: lines past the edge
    of C repeat the last line, a chunk that crosses the end of a
    line-contiguous operand's lines is read as the line's last whole chunk and
    its lines are found at an offset in their slot (also where the last tile
    holds only 1 to 3 of them), a K that is not a whole number of slabs ends
    in a slab staged on its own, and problems under one slab deep, or with
    fewer than 4 lines where the lines are contiguous, take the plain register
    loop. Exact on integer inputs, with NaN around every operand and in C's
    padding, which must stay."""
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    cases = [  # M, N, K, lda pad, ldb pad, ldc pad, A offset, B offset, C offset (floats)
        (bm + 1, bn - 3, 4 * bk, 1, 3, 1, 1, 2, 3),
        (2 * bm + 5, 2 * bn + 7, 9 * bk + 3, 0, 0, 0, 3, 1, 1),
        (1, 1, bk, 0, 0, 0, 1, 1, 1),
        (3, bn + 1, 5 * bk + 1, 2, 1, 2, 2, 3, 0),
        (bm - 1, 2, 2 * bk + 31, 1, 0, 1, 0, 1, 2),
        (bm + 7, 5, 3 * bk, 3, 2, 0, 1, 3, 1),
        (bm + 2, bn + 2, 3 * bk + 5, 1, 1, 0, 2, 1, 0),  # 2 lines in the last tile of each
        (2 * bm + 3, 2 * bn + 3, 2 * bk, 0, 2, 1, 1, 0, 2),  # 3 lines in the last tile of each
        (2 * bm, 2 * bn, bk - 1, 1, 1, 1, 2, 1, 3),
        (3001 % bm + bm, 2047 % bn + bn, 1537, 0, 0, 0, 0, 0, 0),
    ]
    for seed, (M, N, K, pa, pb, pc, oa, ob, oc) in enumerate(cases, start=2500):
        A, B = workloads.draw(M, N, K, seed, "int4")
        As, Bs = _stored(A, opA), _stored(B, opB)
        ra, ca = As.shape
        rb, cb = Bs.shape
        lda, ldb, ldc = ca + pa, cb + pb, N + pc
        abuf = torch.full((oa + ra * lda + 5,), float("nan"), device="cuda")
        bbuf = torch.full((ob + rb * ldb + 5,), float("nan"), device="cuda")
        cbuf = torch.full((oc + M * ldc + 5,), float("nan"), device="cuda")
        Av = abuf[oa:oa + ra * lda].view(ra, lda)
        Bv = bbuf[ob:ob + rb * ldb].view(rb, ldb)
        Cv = cbuf[oc:oc + M * ldc].view(M, ldc)
        Av[:, :ca] = G.dev(As)
        Bv[:, :cb] = G.dev(Bs)
        assert sg.sgemm_mi355_config_staging(cid, M, N, K, Av.data_ptr(), lda, Bv.data_ptr(), ldb) == 0
        print(f"[gpu] config={CONFIG_NAMES[cid]} M={M} N={N} K={K} lda={lda} ldb={ldb} "
              f"offsets={oa},{ob},{oc}", flush=True)
        rc = sg.sgemm_mi355_strided_batched_with_config(
            opA, opB, M, N, K, 1.0, Av.data_ptr(), lda, 0, Bv.data_ptr(), ldb, 0, 0.0, Cv.data_ptr(), ldc, 0, 1,
            torch.cuda.current_stream().cuda_stream, cid)
        assert rc == sg.OK
        torch.cuda.synchronize()
        G.check_exact(np.ascontiguousarray(Cv[:, :N].cpu().numpy()), np_(A), np_(B))
        assert np.isnan(Cv[:, N:].cpu().numpy()).all()
        assert np.isnan(cbuf[:oc].cpu().numpy()).all() and np.isnan(cbuf[oc + M * ldc:].cpu().numpy()).all()


@pytest.mark.parametrize("cid", DIRECT_IDS, ids=[CONFIG_NAMES[i] for i in DIRECT_IDS])
def test_direct_lds_partial_last_slab_any_remainder(cid):
    """K = whole slabs plus 1 or 3 values (odd K) with the stored rows padded
    to multiples of 4 floats, so the operands stay 16-byte aligned and the
    configuration takes its direct path with a register-staged last slab
    (checked through sgemm_mi355_config_staging); the element-wise tail of the
    register loader then runs on the k-contiguous operands. Exact on integer
    inputs, in the operand layouts the configuration reads."""
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    opA, opB = sg.sgemm_mi355_config_ops(cid)
    seed = 1500
    for slabs, r in ((1, 1), (2, 3), (3, 1), (5, 3)):
        seed += 1
        M, N, K = bm + 4, bn - 4, slabs * bk + r
        A, B = workloads.draw(M, N, K, seed, "int4")
        As, Bs = _stored(A, opA), _stored(B, opB)
        lda = -(-As.shape[1] // 4) * 4
        ldb = -(-Bs.shape[1] // 4) * 4
        Ad = G.dev(workloads.embed(As, lda))[:, :As.shape[1]]
        Bd = G.dev(workloads.embed(Bs, ldb))[:, :Bs.shape[1]]
        assert sg.sgemm_mi355_config_staging(cid, M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb) == 2
        print(f"[gpu] config={CONFIG_NAMES[cid]} M={M} N={N} K={K} lda={lda} ldb={ldb}", flush=True)
        C = sg.gemm(Ad, Bd, opA=opA, opB=opB, config=cid)
        torch.cuda.synchronize()
        G.check_exact(C.cpu().numpy(), np_(A), np_(B))
