"""The entry points under HIP graph capture: every launch the library makes
(the GEMM kernels, the split-K reduction, the stream-K kernel and its fixup,
the C = beta*C kernel for K == 0)
is an ordinary kernel node, with no memset node, so a captured call can be
replayed. Each case captures one call, then replays it several times with
unrelated eager work and synchronisations between the replays, refilling C
before each replay, and checks every replay against the oracle exactly
(integer-valued inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_fp32_matrix_02_amd as sg
import oracle
import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    G.require_gpu()


def _ints(rows, cols, seed):
    return workloads.as_numpy(workloads.draw(rows, 1, cols, seed, "int4")[0])


def _eager_noise(seed):
    """Unrelated eager work between replays: another product on other data."""
    A, B = workloads.draw(300, 200, 100, seed, "int4")
    C = sg.matmul(A.to("cuda"), B.to("cuda"))
    torch.cuda.synchronize()
    G.check_exact(C.cpu().numpy(), workloads.as_numpy(A), workloads.as_numpy(B))


def _capture(fn):
    """Capture fn() into a graph after one eager warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _replay_and_check(graph, C, C_init, want, label):
    for r in range(REPLAYS):
        print(f"[gpu] graph {label} replay {r}", flush=True)
        C.copy_(C_init)  # eager refill, outside the graph
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(C.cpu().numpy(), want, err_msg=f"{label}, replay {r}")
        _eager_noise(100 + r)


def test_graph_plain_product():
    M, N, K = 700, 500, 300
    A, B = _ints(M, K, 1), _ints(K, N, 2)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((M, N), device="cuda")
    graph = _capture(lambda: sg.matmul(Ad, Bd, out=C))
    nan = torch.full((M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, oracle.sgemm_f32(A, B), "plain")


def test_graph_general_form_reads_c():
    M, N, K = 257, 333, 129
    A, B, C0 = _ints(K, M, 3), _ints(K, N, 4), _ints(M, N, 5)  # op(A) = A^T
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C0d = torch.from_numpy(C0).cuda()
    C = C0d.clone()
    graph = _capture(lambda: sg.gemm(Ad, Bd, C, opA=1, alpha=2.0, beta=-1.0))
    want = C0.copy()
    oracle.sgemm_ex_f32(1, 0, 2.0, A, B, -1.0, want)
    _replay_and_check(graph, C, C0d, want, "general")


def test_graph_splitk_two_kernels():
    M, N, K = 96, 80, 4100
    A, B = _ints(M, K, 6), _ints(K, N, 7)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((M, N), device="cuda")
    splits = 4
    need = sg.sgemm_mi355_splitk_workspace_size(M, N, K, splits)
    ws = torch.empty((need + 3) // 4, device="cuda")
    graph = _capture(lambda: sg.gemm_splitk(Ad, Bd, C, splits=splits, workspace=ws))
    nan = torch.full((M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, oracle.sgemm_f32(A, B), "split-K")


def test_graph_streamk_two_kernels():
    """Stream-K in 256x256 tiles: 25 tiles whose slabs are dealt to the whole
    grid, then the fixup kernel adds the partial sums (alpha 2, beta -1)."""
    M, N, K = 1280, 1280, 2048
    A, B = _ints(M, K, 8), _ints(K, N, 9)
    C0 = _ints(M, N, 10)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((M, N), device="cuda")
    cid = sg.config_id("mfma32_256x256x16_w4x4_lds2")
    need = sg.sgemm_mi355_streamk_workspace_size(0, 0, M, N, K, cid)
    assert need > 0
    ws = torch.empty((need + 3) // 4, device="cuda")
    C.copy_(torch.from_numpy(C0))
    graph = _capture(lambda: sg.gemm_streamk(Ad, Bd, C, alpha=2.0, beta=-1.0, workspace=ws, config=cid))
    want = C0.copy()
    oracle.sgemm_ex_f32(0, 0, 2.0, A, B, -1.0, want)
    _replay_and_check(graph, C, torch.from_numpy(C0).cuda(), want, "stream-K")


def test_graph_k_zero_fills_c():
    M, N = 130, 77
    Ad = torch.empty((M, 0), device="cuda")
    Bd = torch.empty((0, N), device="cuda")
    C = torch.empty((M, N), device="cuda")
    graph = _capture(lambda: sg.gemm(Ad, Bd, C))
    nan = torch.full((M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, np.zeros((M, N), np.float32), "K=0")


def test_graph_strided_batch():
    batch, M, N, K = 6, 70, 90, 50
    A = np.stack([_ints(M, K, 10 + b) for b in range(batch)])
    B = np.stack([_ints(K, N, 30 + b) for b in range(batch)])
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((batch, M, N), device="cuda")
    graph = _capture(lambda: sg.gemm_strided_batched(Ad, Bd, C))
    nan = torch.full((batch, M, N), float("nan"), device="cuda")
    want = np.stack([oracle.sgemm_f32(A[b], B[b]) for b in range(batch)])
    _replay_and_check(graph, C, nan, want, "batched")


def test_graph_direct_lds_kernels():
    """Direct global-to-LDS kernels under capture: a batch the selection runs
    in the 256x256 direct tile, and a transposed product it runs in the 32x32
    direct tile whose k groups add their sums through LDS."""
    batch, M, N, K = 16, 1024, 1024, 1024
    A = np.stack([_ints(M, K, 50 + b) for b in range(batch)])
    B = np.stack([_ints(K, N, 70 + b) for b in range(batch)])
    print(f"[gpu] graph batched selects {sg.config_names()[sg.sgemm_mi355_select_config_ex(0, 0, M, N, K, batch)]}",
          flush=True)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((batch, M, N), device="cuda")
    graph = _capture(lambda: sg.gemm_strided_batched(Ad, Bd, C))
    want = np.matmul(A.astype(np.float64), B.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(want[3], oracle.sgemm_f32(A[3], B[3]))
    nan = torch.full((batch, M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, want, "direct 256x256 batch")

    M, N, K = 512, 512, 4096
    At, Bt = _ints(K, M, 91), _ints(N, K, 92)  # stored transposed: op(A) = At^T, op(B) = Bt^T
    print(f"[gpu] graph tt selects {sg.config_names()[sg.sgemm_mi355_select_config_ex(1, 1, M, N, K, 1)]}",
          flush=True)
    Ad, Bd = torch.from_numpy(At).cuda(), torch.from_numpy(Bt).cuda()
    C = torch.empty((M, N), device="cuda")
    graph = _capture(lambda: sg.gemm(Ad, Bd, C, opA=1, opB=1))
    want = oracle.sgemm_f32(np.ascontiguousarray(At.T), np.ascontiguousarray(Bt.T))
    nan = torch.full((M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, want, "direct k-group tt")


def test_graph_hand_ordered_tile():
    """The one-wave-per-SIMD tile under capture, plain and with both operands
    transposed: its loads, fragment reads and barrier are ordered by hand,
    and every replay must still give the oracle's bits."""
    M, N, K = 768, 520, 1024
    A, B = _ints(M, K, 93), _ints(K, N, 94)
    cid = sg.config_id("mfma32_256x256x32_w2x2_lds2_sched")
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.empty((M, N), device="cuda")
    print(f"[gpu] graph hand-ordered tile M={M} N={N} K={K}", flush=True)
    graph = _capture(lambda: sg.gemm(Ad, Bd, C, config=cid))
    nan = torch.full((M, N), float("nan"), device="cuda")
    _replay_and_check(graph, C, nan, oracle.sgemm_f32(A, B), "hand-ordered tile")

    cid = sg.config_id("mfma32_256x256x32_w2x2_lds2_sched_tt")
    At, Bt = _ints(K, M, 95), _ints(N, K, 96)
    Ad, Bd = torch.from_numpy(At).cuda(), torch.from_numpy(Bt).cuda()
    graph = _capture(lambda: sg.gemm(Ad, Bd, C, opA=1, opB=1, config=cid))
    want = oracle.sgemm_f32(np.ascontiguousarray(At.T), np.ascontiguousarray(Bt.T))
    _replay_and_check(graph, C, nan, want, "hand-ordered tile tt")
