"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* the library loads and exports every function include/*.h declares;
* argument validation returns the documented codes before any HIP call;
* configuration metadata and the tile table are consistent;
* the workgroup -> tile map is a bijection for many grid shapes.
"""
from __future__ import annotations

import glob
import os
import re

import pytest

import dense_fp32_matrix_02_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(sg.LIB_PATH):
        from dense_fp32_matrix_02_amd import build
        build.build()
    return sg.load()


def header_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(sgemm_mi355\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert "sgemm_mi355" in names and len(names) >= 10
    lib = sg.load()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_error_codes_match_header():
    text = open(os.path.join(ROOT, "include", "sgemm_mi355.h")).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"#define SGEMM_MI355_(\w+) \(?(-?\d+)\)?", text))
    assert codes["OK"] == sg.OK
    for name in ("DIM", "LD", "NULL", "ALIAS", "EXTENT", "LAUNCH", "CONFIG", "ALIGN", "STRIDE", "OP",
                 "WORKSPACE", "SCRATCH"):
        assert codes["ERR_" + name] == getattr(sg, "ERR_" + name)
        assert sg.strerror(codes["ERR_" + name]) != sg.strerror(12345)
    assert sg.strerror(0) == "success"


# Fake, never-dereferenced device addresses (validation is pure host code).
A0, B0, C0 = 0x10000000, 0x20000000, 0x30000000


VALIDATION_CASES = [
    ((-1, 4, 4, A0, 4, B0, 4, C0, 4), sg.ERR_DIM),
    ((4, -1, 4, A0, 4, B0, 4, C0, 4), sg.ERR_DIM),
    ((4, 4, -1, A0, 4, B0, 4, C0, 4), sg.ERR_DIM),
    ((4, 4, 5, A0, 4, B0, 4, C0, 4), sg.ERR_LD),       # lda < K
    ((4, 5, 4, A0, 4, B0, 4, C0, 5), sg.ERR_LD),       # ldb < N
    ((4, 5, 4, A0, 4, B0, 5, C0, 4), sg.ERR_LD),       # ldc < N
    ((4, 4, 0, A0, 0, B0, 4, C0, 4), sg.ERR_LD),       # lda < max(1, K)
    ((0, 4, 4, 0, 4, 0, 4, 0, 4), sg.OK),              # M == 0: nothing referenced
    ((4, 0, 4, 0, 4, 0, 1, 0, 1), sg.OK),              # N == 0
    ((4, 4, 4, A0, 4, B0, 4, 0, 4), sg.ERR_NULL),
    ((4, 4, 4, 0, 4, B0, 4, C0, 4), sg.ERR_NULL),
    ((4, 4, 4, A0, 4, 0, 4, C0, 4), sg.ERR_NULL),
    ((4, 4, 0, 0, 1, 0, 4, C0, 4), sg.OK),             # K == 0: A and B unused
    ((4, 4, 4, A0 + 2, 4, B0, 4, C0, 4), sg.ERR_ALIGN),
    ((4, 4, 4, A0, 4, B0 + 1, 4, C0, 4), sg.ERR_ALIGN),
    ((4, 4, 4, A0, 4, B0, 4, C0 + 3, 4), sg.ERR_ALIGN),
    ((4, 4, 4, A0 + 4, 4, B0, 4, C0, 4), sg.OK),       # 4-byte alignment is enough
    ((4, 4, 4, A0, 4, B0, 4, A0 + 60, 4), sg.ERR_ALIAS),   # C starts inside A
    ((4, 4, 4, A0, 4, B0, 4, B0 - 60, 4), sg.ERR_ALIAS),   # C ends inside B
    ((4, 4, 4, A0, 4, B0, 4, A0 + 64, 4), sg.OK),          # C right after A
    ((4, 4, 4, A0, 5, B0, 4, A0 + 4 * 19, 4), sg.OK),      # A extent = 3*5+4 = 19 floats
    ((4, 4, 4, A0, 5, B0, 4, A0 + 4 * 18, 4), sg.ERR_ALIAS),
    ((2 ** 31 - 1, 4, 4, A0, 4, B0, 4, C0, 4), sg.ERR_EXTENT),
]


@pytest.mark.parametrize("args,code", VALIDATION_CASES)
def test_validation_codes(args, code):
    assert sg.sgemm_mi355_validate(*args) == code


@pytest.mark.parametrize("fn", ["sgemm_mi355", "sgemm_mi355_valu"])
def test_entry_points_reject_before_any_hip_call(fn):
    f = getattr(sg, fn)
    assert f(-1, 4, 4, A0, 4, B0, 4, C0, 4, 0) == sg.ERR_DIM
    assert f(4, 4, 5, A0, 4, B0, 4, C0, 4, 0) == sg.ERR_LD
    assert f(4, 4, 4, A0, 4, B0, 4, A0 + 8, 4, 0) == sg.ERR_ALIAS
    assert f(0, 4, 4, 0, 4, 0, 4, 0, 4, 0) == sg.OK   # quick return, nothing enqueued


def test_splitk_noalloc_rejects_before_any_hip_call():
    """Validation, then the size check against the static scratch, both on
    the host: 4 chunks of 2048 x 2048 partial sums are 64 MiB."""
    assert int(re.search(r"#define SGEMM_MI355_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                         open(os.path.join(ROOT, "include", "sgemm_mi355.h")).read()).group(1)) << 20 \
        == sg.SCRATCH_BYTES
    f = sg.sgemm_mi355_splitk_noalloc
    assert f(0, 0, -1, 4, 4, 1.0, A0, 4, B0, 4, 0.0, C0, 4, 2, 0) == sg.ERR_DIM
    assert f(0, 0, 4, 4, 4, 1.0, A0, 4, B0, 4, 0.0, C0, 4, 0, 0) == sg.ERR_DIM
    assert f(0, 0, 4, 4, 4, 1.0, A0, 4, B0, 4, 0.0, A0 + 8, 4, 2, 0) == sg.ERR_ALIAS
    M = N = 2048
    K = 8192
    assert sg.sgemm_mi355_splitk_workspace_size(M, N, K, 4) == 2 * sg.SCRATCH_BYTES
    assert f(0, 0, M, N, K, 1.0, A0, K, B0, N, 0.0, C0 + 2 ** 30, N, 4, 0) == sg.ERR_SCRATCH
    assert "scratch" in sg.strerror(sg.ERR_SCRATCH)


def test_with_config_rejects_unknown_ids():
    n = sg.sgemm_mi355_num_configs()
    for bad in (-1, n, n + 7):
        assert sg.sgemm_mi355_with_config(4, 4, 4, A0, 4, B0, 4, C0, 4, 0, bad) == sg.ERR_CONFIG
        assert sg.sgemm_mi355_config_name(bad) is None
        with pytest.raises(sg.SgemmError):
            sg.sgemm_mi355_config_info(bad)


def test_config_metadata():
    names = sg.config_names()
    assert len(names) == len(set(names)) >= 4
    for i, name in enumerate(names):
        bm, bn, bk, threads = sg.sgemm_mi355_config_info(i)
        assert f"{bm}x{bn}x{bk}" in name
        assert threads % 64 == 0 and 64 <= threads <= 1024
        assert name.startswith(("mfma32_", "valu"))
        if name.startswith("valu"):
            tm = int(name[4:name.index("x")])
            assert threads == (bm // tm) * (bn // 8)
        else:
            w = re.search(r"_w(\d+)x(\d+)", name)
            kg = re.search(r"_kg(\d+)", name)
            assert threads == 64 * int(w[1]) * int(w[2]) * (int(kg[1]) if kg else 1)
    assert sg.sgemm_mi355_version().count(".") == 2


def test_selection_picks_matrix_core_configs_for_every_workload():
    import workloads
    for w in workloads.WORKLOADS:
        cid = sg.sgemm_mi355_select_config(w.M, w.N, w.K)
        assert sg.sgemm_mi355_config_name(cid).startswith("mfma32_")
    for shape in [(1, 1, 1), (7, 3, 9000), (100000, 16, 64), (16, 100000, 64)]:
        cid = sg.sgemm_mi355_select_config(*shape)
        assert 0 <= cid < sg.sgemm_mi355_num_configs()
    assert sg.sgemm_mi355_select_config(-1, 1, 1) == sg.ERR_DIM


def test_selected_config_sees_the_alignment():
    """With 16-byte aligned operands and leading dimensions that are multiples
    of 4, sgemm_mi355_selected_config agrees with the shape-only selection;
    with a misaligned leading dimension it never names a direct-to-LDS
    configuration (their direct loads need 16-byte chunks)."""
    import workloads
    for w in workloads.WORKLOADS:
        sel = sg.sgemm_mi355_select_config(w.M, w.N, w.K)
        got = sg.sgemm_mi355_selected_config(w.M, w.N, w.K, A0, w.lda, B0, w.ldb)
        if w.lda % 4 == 0 and w.ldb % 4 == 0:
            assert got == sel
        else:
            assert "_lds" not in sg.sgemm_mi355_config_name(got)
    for (M, N, K) in [(4096, 4096, 4096), (8192, 8192, 8192), (1024, 1024, 1024)]:
        aligned = sg.sgemm_mi355_selected_config(M, N, K, A0, K, B0, N)
        assert aligned == sg.sgemm_mi355_select_config(M, N, K)
        for a, lda in ((A0 + 4, K), (A0, K + 1)):
            got = sg.sgemm_mi355_selected_config(M, N, K, a, lda, B0, N)
            assert "_lds" not in sg.sgemm_mi355_config_name(got)
    assert sg.sgemm_mi355_selected_config(-1, 1, 1, A0, 1, B0, 1) == sg.ERR_DIM


def test_config_staging_follows_the_direct_load_rules():
    """Direct loads for 16-byte aligned operands with leading dimensions that
    are multiples of 4 and K of at least one slab (2 when K ends in a partial
    slab); registers otherwise, and always for register-staged configurations."""
    names = sg.config_names()
    direct = [i for i, n in enumerate(names) if "_lds" in n]
    assert direct
    for cid in direct:
        bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
        opA, opB = sg.sgemm_mi355_config_ops(cid)
        M, N = bm + 4, bn + 8
        lda = M if opA else 4 * bk
        ldb = 4 * bk if opB else N
        st = sg.sgemm_mi355_config_staging
        assert st(cid, M, N, 4 * bk, A0, lda, B0, ldb) == 1
        assert st(cid, M, N, 3 * bk + 1, A0, lda + 4, B0, ldb + 4) == 2
        assert st(cid, M, N, bk - 1, A0, lda, B0, ldb) == 0          # less than one slab
        assert st(cid, M, N, 4 * bk, A0 + 4, lda, B0, ldb) == 0      # 4-byte aligned base
        assert st(cid, M, N, 4 * bk, A0, lda + 1, B0, ldb) == 0      # odd leading dimension
        if opA:
            assert st(cid, M + 1, N, 4 * bk, A0, lda + 4, B0, ldb) == 0  # A^T rows of M not whole chunks
        if not opB:
            assert st(cid, M, N + 1, 4 * bk, A0, lda, B0, ldb + 4) == 0  # B rows of N not whole chunks
    plain = [i for i, n in enumerate(names) if "_lds" not in n]
    assert sg.sgemm_mi355_config_staging(plain[0], 256, 256, 256, A0, 256, B0, 256) == 0
    assert sg.sgemm_mi355_config_staging(len(names), 4, 4, 4, A0, 4, B0, 4) == sg.ERR_CONFIG
    assert sg.sgemm_mi355_config_staging(direct[0], -1, 4, 4, A0, 4, B0, 4) == sg.ERR_DIM


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [
    (1, 1, 4), (1, 7, 4), (7, 1, 4), (3, 5, 2), (16, 16, 4), (32, 32, 4), (24, 16, 4),
    (13, 29, 8), (8, 8, 1), (64, 3, 16), (5, 64, 3)])
def test_tile_map_is_a_bijection(tiles_m, tiles_n, group_m):
    seen = set()
    for bid in range(tiles_m * tiles_n):
        tm, tn = sg.sgemm_mi355_tile_map(bid, tiles_m, tiles_n, group_m)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n


def test_tile_map_keeps_concurrent_tiles_on_one_xcd_compact():
    """On a 32 x 32 tile grid each XCD (workgroups b with b % 8 equal) gets
    consecutive logical tiles; its first 32 resident tiles span 4 tile rows
    and 8 tile columns instead of a full row of 32."""
    for xcd in range(8):
        tiles = [sg.sgemm_mi355_tile_map(8 * s + xcd, 32, 32, 4) for s in range(32)]
        assert len({tm for tm, _ in tiles}) == 4
        assert len({tn for _, tn in tiles}) == 8


# ---- general form and strided batch: validation only (no kernel runs) -------

def vex(opA=0, opB=0, M=4, N=4, K=4, alpha=1.0, A=A0, lda=None, sA=0, B=B0, ldb=None, sB=0,
        beta=0.0, C=C0, ldc=None, sC=0, batch=1):
    lda = lda if lda is not None else max(1, M if opA else K)
    ldb = ldb if ldb is not None else max(1, K if opB else N)
    ldc = ldc if ldc is not None else max(1, N)
    return sg.sgemm_mi355_validate_ex(opA, opB, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc,
                                      sC, batch)


def test_validate_ex_ops_and_leading_dims():
    assert vex() == sg.OK
    assert vex(opA=2) == sg.ERR_OP and vex(opB=-1) == sg.ERR_OP
    # opA = T: A is K x M, so lda >= M; opB = T: B is N x K, so ldb >= K
    assert vex(opA=1, M=9, K=3, lda=9) == sg.OK
    assert vex(opA=1, M=9, K=3, lda=8) == sg.ERR_LD
    assert vex(opA=0, M=9, K=3, lda=3) == sg.OK
    assert vex(opB=1, N=7, K=5, ldb=5) == sg.OK
    assert vex(opB=1, N=7, K=5, ldb=4) == sg.ERR_LD
    assert vex(opB=0, N=7, K=5, ldb=6) == sg.ERR_LD


def test_validate_ex_batch_and_strides():
    assert vex(batch=-1) == sg.ERR_DIM
    assert vex(batch=0, A=0, B=0, C=0) == sg.OK            # nothing to do
    assert vex(sA=-1) == sg.ERR_STRIDE
    assert vex(batch=3, sC=15) == sg.ERR_STRIDE            # C_b overlap: extent is 16
    assert vex(batch=3, sC=16, sA=0, sB=0, B=B0 + 10 ** 6) == sg.OK   # shared A and B
    assert vex(batch=1, sC=0) == sg.OK
    # C's batched range [C0, C0 + 4*(2*100 + 16)) reaches into a B placed after it
    assert vex(batch=3, sC=100, B=C0 + 4 * 200) == sg.ERR_ALIAS
    assert vex(batch=3, sC=100, B=C0 + 4 * 216) == sg.OK


def test_validate_ex_alpha_zero_and_k_zero_skip_a_and_b():
    assert vex(alpha=0.0, A=0, B=0, beta=2.0) == sg.OK
    assert vex(K=0, lda=1, A=0, B=0, beta=0.5) == sg.OK
    assert vex(alpha=1.0, A=0) == sg.ERR_NULL
    assert vex(alpha=0.0, A=0, B=0, C=0) == sg.ERR_NULL


def test_general_entry_points_reject_before_any_hip_call():
    assert sg.sgemm_mi355_ex(3, 0, 4, 4, 4, 1.0, A0, 4, B0, 4, 0.0, C0, 4, 0) == sg.ERR_OP
    assert sg.sgemm_mi355_strided_batched(0, 0, 4, 4, 4, 1.0, A0, 4, 0, B0, 4, 0, 0.0, C0, 4, 1, 2, 0) \
        == sg.ERR_STRIDE
    assert sg.sgemm_mi355_strided_batched(0, 0, 4, 4, 4, 1.0, A0, 4, 0, B0, 4, 0, 0.0, C0, 4, 16, 0, 0) \
        == sg.OK


def test_config_ops_and_config_op_mismatch():
    n = sg.sgemm_mi355_num_configs()
    seen = set()
    for cid in range(n):
        ops = sg.sgemm_mi355_config_ops(cid)
        seen.add(ops)
        name = sg.sgemm_mi355_config_name(cid)
        suffix = {(0, 0): "", (1, 0): "_tn", (0, 1): "_nt", (1, 1): "_tt"}[ops]
        assert name.endswith(suffix) if suffix else not name.endswith(("_tn", "_nt", "_tt"))
        other = (1 - ops[0], ops[1])
        assert sg.sgemm_mi355_strided_batched_with_config(other[0], other[1], 4, 4, 4, 1.0, A0, 4, 0, B0, 4, 0,
                                                          0.0, C0, 4, 0, 1, 0, cid) == sg.ERR_CONFIG
    assert seen == {(0, 0), (0, 1), (1, 0), (1, 1)}


def test_select_config_ex_matches_ops():
    for opA, opB in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        for shape in [(1, 1, 1, 1), (4096, 4096, 4096, 1), (64, 64, 64, 1000), (3001, 2047, 1537, 3)]:
            cid = sg.sgemm_mi355_select_config_ex(opA, opB, *shape)
            assert sg.sgemm_mi355_config_ops(cid) == (opA, opB)
    assert sg.sgemm_mi355_select_config_ex(2, 0, 1, 1, 1, 1) == sg.ERR_OP
    assert sg.sgemm_mi355_select_config_ex(0, 0, 1, 1, 1, -1) == sg.ERR_DIM
    # many small products: the batch fills the chip, so a large tile is fine
    big = sg.sgemm_mi355_select_config_ex(0, 0, 256, 256, 256, 64)
    small = sg.sgemm_mi355_select_config_ex(0, 0, 256, 256, 256, 1)
    assert sg.sgemm_mi355_config_info(big)[0] >= sg.sgemm_mi355_config_info(small)[0]


def test_config_occupancy_errors_and_values():
    """Unknown ids and null outputs are rejected before any HIP call. Without
    a device the runtime query reports a launch error; with one, every
    configuration holds at least one workgroup per compute unit."""
    import ctypes
    lib = sg.load()
    n = ctypes.c_int(-1)
    assert lib.sgemm_mi355_config_occupancy(-1, ctypes.byref(n)) == sg.ERR_CONFIG
    assert lib.sgemm_mi355_config_occupancy(sg.sgemm_mi355_num_configs(), ctypes.byref(n)) == sg.ERR_CONFIG
    assert lib.sgemm_mi355_config_occupancy(0, None) == sg.ERR_NULL
    rc = lib.sgemm_mi355_config_occupancy(0, ctypes.byref(n))
    assert rc in (sg.OK, sg.ERR_LAUNCH)
    if rc == sg.OK:
        assert n.value >= 1


def test_binding_leading_dimension_of_torch_tensors():
    """Row stride read from torch tensors: padded rows keep their stride, and
    a size-1 dimension's stride (arbitrary in torch) is ignored."""
    import torch
    from dense_fp32_matrix_02_amd._binding import _ld
    assert _ld(torch.zeros(1, 2).t().contiguous(), "x") == 1      # (2, 1) with strides (1, 2)
    assert _ld(torch.zeros(3, 1), "x") == 1
    assert _ld(torch.zeros(1, 5), "x") == 5
    assert _ld(torch.zeros(4, 8)[:, :5], "x") == 8
    with pytest.raises(ValueError):
        _ld(torch.zeros(4, 8).t(), "x")
    with pytest.raises(ValueError):
        _ld(torch.zeros(2, 3, 4), "x")



# ---- split-K: sizing and validation (no kernel runs) -------------------------

def test_splitk_workspace_size():
    ws = sg.sgemm_mi355_splitk_workspace_size
    assert ws(100, 50, 1000, 1) == 0                 # no split
    assert ws(100, 50, 1000, 4) == 4 * 4 * 100 * 50  # chunks of 256 -> 4 partials
    assert ws(100, 50, 64, 8) == 2 * 4 * 100 * 50    # chunks of at least 32 -> 2 partials
    assert ws(100, 50, 20, 8) == 0                   # K below one chunk: no split
    assert ws(0, 50, 1000, 4) == 0 and ws(100, 50, 1000, 0) == 0 and ws(100, 50, 1000, 257) == 0


def test_splitk_rejects_bad_arguments_before_any_hip_call():
    W = 0x40000000
    f = sg.sgemm_mi355_splitk
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 0, W, 10 ** 7, 0) == sg.ERR_DIM
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 300, W, 10 ** 7, 0) == sg.ERR_DIM
    need = sg.sgemm_mi355_splitk_workspace_size(100, 50, 1000, 4)
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 4, W, need - 4, 0) == sg.ERR_WORKSPACE
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 4, 0, need, 0) == sg.ERR_NULL
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 4, W + 2, need, 0) == sg.ERR_ALIGN
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 4, C0 + 400, need, 0) == sg.ERR_ALIAS
    assert f(0, 0, 100, 50, 1000, 1.0, A0, 1000, B0, 50, 0.0, C0, 50, 4, A0 + 4000, need, 0) == sg.ERR_ALIAS


def _plan_splits(K, s):
    """Effective split count: chunks of ceil(K/s) rounded up to 32."""
    s = max(s, 1)
    if K <= 0:
        return 1
    kc = -(-K // s)
    kc = -(-kc // 32) * 32
    eff = -(-K // kc)
    return 1 if eff <= 1 else eff


def _rule_splits(opA, opB, M, N, K):
    """Outside the measured split-K grid: split only when the unsplit grid has
    fewer than 512 workgroups, into the largest power-of-two count whose
    chunks keep at least 1024 values of k."""
    import math
    bm, bn, _, _ = sg.sgemm_mi355_config_info(sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, 1))
    s = 1
    if math.ceil(M / bm) * math.ceil(N / bn) < 512:
        while 2 * s <= 256 and K >= 2 * s * 1024:
            s *= 2
    return _plan_splits(K, s)


def test_select_splitk_matches_its_definition():
    """Near the measured split-K grid: the fastest split count at the nearest
    grid shape (then chunked as the entry point does); elsewhere the rule."""
    import random
    from tests._table import nearest, read_split_table
    table = read_split_table()
    assert len(table) > 200 and all(s in (1, 2, 4, 8, 16, 32, 64) for *_, s in table)
    rng = random.Random(5)
    cases = [(m, n, k) for m, n, k, _ in table[::7]]
    cases += [(rng.randint(1, 5000), rng.randint(1, 5000), rng.randint(1, 140000)) for _ in range(300)]
    cases += [(rng.randint(6200, 30000), rng.randint(1, 30000), rng.randint(1, 140000)) for _ in range(80)]
    cases += [(8192, 8192, 8192), (768, 768, 65536), (3000, 100, 100000), (33, 47, 1_000_003), (1, 1, 1)]
    near_seen = rule_seen = 0
    for M, N, K in cases:
        near = nearest(table, M, N, K)
        for opA, opB in [(0, 0), (1, 1)]:
            want = _plan_splits(K, table[near][3]) if near is not None else _rule_splits(opA, opB, M, N, K)
            sp, cid = sg.sgemm_mi355_select_splitk(opA, opB, M, N, K)
            assert sp == want, (opA, opB, M, N, K)
            assert sg.sgemm_mi355_config_ops(cid) == (opA, opB)
        near_seen += near is not None
        rule_seen += near is None
    assert near_seen > 100 and rule_seen > 50
    assert sg.sgemm_mi355_select_splitk(0, 0, 8192, 8192, 8192)[0] == 1   # fills the chip: no split
    with pytest.raises(sg.SgemmError):
        sg.sgemm_mi355_select_splitk(2, 0, 1, 1, 1)


# ---- configuration selection, written out from its definition ---------------

from tests._table import OP_PAIRS, read_table as _table  # noqa: E402

SAT_CHAINS = 8         # resident 32x32 accumulator blocks per compute unit for full rate
STORE_DEPTH = 40.0     # the store of a C tile, in steps of k at full rate


_IDS = {}


def _id(name):
    if not _IDS:
        _IDS.update({n: i for i, n in enumerate(sg.config_names())})
    return _IDS[name]


def _busy(cid, occ, M, N, K, batch=1):
    """Busy time of the busiest compute unit: n = ceil(workgroups / 256)
    workgroups, run occ at a time, stretched by SAT_CHAINS / resident
    accumulator blocks while fewer are resident (a workgroup holds
    k-groups * BM/32 * BN/32 blocks of 32x32), times ceil(K / BK) plus
    STORE_DEPTH / BK for the store of C."""
    import math
    bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
    kg = re.search(r"_kg(\d+)", sg.sgemm_mi355_config_name(cid))
    blocks = (int(kg.group(1)) if kg else 1) * (bm // 32) * (bn // 32)
    wgs = math.ceil(M / bm) * math.ceil(N / bn) * min(batch, 65535)
    n = math.ceil(wgs / 256)
    resident = min(n, occ) * blocks
    stretch = 1.0 if resident >= SAT_CHAINS else SAT_CHAINS / resident
    return n * stretch * (math.ceil(K / bk) + STORE_DEPTH / bk)


def _direct_path(name, M, N, K):
    """A direct-to-LDS configuration takes its direct path (aligned operands):
    K of at least one slab (a partial last slab is staged through registers)
    and a line-contiguous operand's extent a multiple of 4."""
    bk = sg.sgemm_mi355_config_info(_id(name))[2]
    opA, opB = sg.sgemm_mi355_config_ops(_id(name))
    return M > 0 and N > 0 and K >= bk and (not opA or M % 4 == 0) and (opB or N % 4 == 0)


def _model_predict(blocks, opA, opB, M, N, K):
    """The measured shape nearest (M, N, K) in summed |log2| distance among
    those within a factor of two in each dimension (first on a tie), then the
    candidate whose time there, scaled by the busy-time ratio, is least
    (first on a tie): (predicted microseconds, name), or None when no
    measured shape qualifies."""
    import math
    cands, shapes, times = blocks[(opA, opB)]
    near = None
    for s, (m, n, k) in enumerate(shapes):
        if M > 2 * m or m > 2 * M or N > 2 * n or n > 2 * N or K > 2 * k or k > 2 * K:
            continue
        d = abs(math.log2(M / m)) + abs(math.log2(N / n)) + abs(math.log2(K / k))
        if near is None or d < near[0]:
            near = (d, s)
    if near is None:
        return None
    s = near[1]
    m, n, k = shapes[s]
    best = None
    for c, (name, occ) in enumerate(cands):
        t = times[s][c]
        if t <= 0:
            continue
        if "_lds" in name and not _direct_path(name, M, N, K):
            continue
        cid = _id(name)
        pred = t / _busy(cid, occ, m, n, k) * _busy(cid, occ, M, N, K)
        if best is None or pred < best[0]:
            best = (pred, name)
    return best


def _model_select(blocks, opA, opB, M, N, K):
    best = _model_predict(blocks, opA, opB, M, N, K)
    return best[1] if best else None


def test_tile_table_is_consistent():
    blocks = _table()
    assert set(blocks) == set(OP_PAIRS.values())
    names = set(sg.config_names())
    for pair, (cands, shapes, times) in blocks.items():
        assert 0 < len(cands) <= 64 and len(shapes) > 100
        for name, occ in cands:
            assert name in names and occ >= 1
            assert sg.sgemm_mi355_config_ops(_id(name)) == pair
        for s, row in enumerate(times):
            assert all(t >= 0 for t in row) and max(row) > 0, (pair, shapes[s])
            # the shape's best is stored, and nothing beyond 2x it (times have 5 significant digits)
            b = min(t for t in row if t > 0)
            assert all(t == 0 or t <= 2.0 * b * (1 + 1e-4) for t in row)
        # every candidate is the fastest on at least one shape, overall or among
        # the configurations without direct loads
        winners = {cands[min((t, c) for c, t in enumerate(row) if t > 0)[1]][0] for row in times}
        staged = {cands[min((t, c) for c, t in enumerate(row) if t > 0 and "_lds" not in cands[c][0])[1]][0]
                  for row in times}
        assert winners | staged == {n for n, _ in cands}, pair


def test_model_selection_matches_its_definition():
    """Single products inside the measured range: the library's choice is the
    model's, written out above, for every op pair."""
    import random
    blocks = _table()
    names = sg.config_names()
    rng = random.Random(7)
    checked = 0
    for (opA, opB), (_, shapes, _) in blocks.items():
        cases = list(shapes[:30])
        cases += [(rng.randint(64, 16384), rng.randint(64, 16384), rng.randint(128, 32768)) for _ in range(150)]
        cases += [(3072, 3072, 4096), (6144, 6144, 1024), (8192, 8000, 4096), (1536, 1536, 4096), (8191, 8193, 8190)]
        for M, N, K in cases:
            want = _model_select(blocks, opA, opB, M, N, K)
            got = names[sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, 1)]
            if want is None:
                continue
            assert got == want, (opA, opB, M, N, K)
            checked += 1
    assert checked > 500


def _global_predict(norms, opA, opB, M, N, K, batch):
    """Every configuration of the op pair, predicted as its median time per
    busy unit times the busy time of this problem (batch entries included);
    the least wins (first on a tie): (predicted microseconds, name).
    Direct-to-LDS configurations count only on their direct path."""
    best = None
    for name, occ, us in norms[(opA, opB)]:
        if "_lds" in name and not _direct_path(name, M, N, K):
            continue
        t = us * _busy(_id(name), occ, M, N, K, batch)
        if best is None or t < best[0]:
            best = (t, name)
    return best


def _global_select(norms, opA, opB, M, N, K, batch):
    return _global_predict(norms, opA, opB, M, N, K, batch)[1]


def test_median_model_selection_matches_its_definition():
    """Batches, and single products with no measured shape within a factor of
    two, take the median-time model over every configuration of the op pair."""
    import random
    from tests._table import read_norms
    norms = read_norms()
    assert set(norms) == set(OP_PAIRS.values())
    names = sg.config_names()
    for pair, rows in norms.items():
        assert len(rows) >= 10
        for name, occ, us in rows:
            assert name in names and occ >= 1 and us > 0
            assert sg.sgemm_mi355_config_ops(_id(name)) == pair
    blocks = _table()
    rng = random.Random(11)
    cases = [(32, 32, 32, 4096), (16, 16, 64, 4096), (100, 100, 100, 256), (200, 300, 400, 64),
             (1536, 1536, 512, 8), (2048, 2048, 2048, 2), (20000, 20000, 4096, 1), (16640, 16640, 64, 1),
             (100, 256, 16, 3), (4096, 4096, 4100, 2)]
    cases += [(rng.randint(1, 3000), rng.randint(1, 3000), rng.randint(1, 5000), rng.randint(2, 5000))
              for _ in range(200)]
    cases += [(rng.randint(17000, 40000), rng.randint(1, 40000), rng.randint(1, 5000), 1) for _ in range(80)]
    checked = 0
    for M, N, K, batch in cases:
        for opA, opB in OP_PAIRS.values():
            if batch == 1 and _model_select(blocks, opA, opB, M, N, K) is not None:
                continue
            got = names[sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, batch)]
            assert got == _global_select(norms, opA, opB, M, N, K, batch), (opA, opB, M, N, K, batch)
            checked += 1
    assert checked > 800


def test_tuner_busy_time_is_the_selections():
    """The tuner normalises measured times with its own copy of the busy-time
    model; it must agree with the definition the selection is tested against."""
    import random
    from dense_fp32_matrix_02_amd import tune
    rng = random.Random(3)
    names = [n for n in sg.config_names() if n.startswith("mfma")]
    for _ in range(500):
        name = rng.choice(names)
        occ = rng.randint(1, 8)
        M, N, K, batch = rng.randint(1, 20000), rng.randint(1, 20000), rng.randint(1, 70000), rng.randint(1, 300)
        want = _busy(_id(name), occ, M, N, K, batch)
        assert tune.busy_time(*tune.config_geometry(name), occ, M, N, K, batch) == pytest.approx(want, rel=1e-12)


STREAMK_OVERHEAD_US = 40.0  # fixed cost of a stream-K call in the selection model
STREAMK_GAIN = 0.97         # stream-K is chosen below this fraction of the plain estimate


def _streamk_select(blocks, norms, sk, opA, opB, M, N, K):
    """Stream-K selection for aligned operands, written out: the plain path's
    estimate is the larger of the nearest-shape prediction and the median
    model's for the configuration the plain path runs (the median model's
    own choice when no measured shape is near); each stream-K configuration
    on its direct path whose tiles leave a partial last round of 256 x
    occupancy workgroups is predicted as its time per slab x tiles x
    (slabs + STORE_DEPTH / BK) / 256 + STREAMK_OVERHEAD_US; the least wins
    (first on a tie) if it is below STREAMK_GAIN of the plain estimate.
    K below tune.STREAMK_MIN_K keeps the plain path. Returns a name or None."""
    import math
    from dense_fp32_matrix_02_amd import tune
    if K < tune.STREAMK_MIN_K:
        return None
    plain = _model_predict(blocks, opA, opB, M, N, K)
    if plain is not None:
        est, name = plain
        for n, occ, us in norms[(opA, opB)]:
            if n == name:
                est = max(est, us * _busy(_id(n), occ, M, N, K))
    else:
        est, name = _global_predict(norms, opA, opB, M, N, K, 1)
    best = None
    for n, occ, us in sk.get((opA, opB), []):
        bm, bn, bk, _ = sg.sgemm_mi355_config_info(_id(n))
        if not _direct_path(n, M, N, K):
            continue
        tiles = math.ceil(M / bm) * math.ceil(N / bn)
        if tiles % (256 * occ) == 0:
            continue
        t = us * (tiles * (math.ceil(K / bk) + STORE_DEPTH / bk) / 256) + STREAMK_OVERHEAD_US
        if best is None or t < best[0]:
            best = (t, n)
    return best[1] if best is not None and best[0] < STREAMK_GAIN * est else None


def test_streamk_selection_matches_its_definition():
    """sgemm_mi355_select_streamk (host only) is the rule above, for every op
    pair, on the stream-K grid, on random shapes and on shapes with whole
    rounds of tiles, a K tail or ragged lines (no direct path)."""
    import random
    from tests._table import read_norms, read_streamk
    blocks, norms, sk = _table(), read_norms(), read_streamk()
    assert set(sk) == set(OP_PAIRS.values())
    names = sg.config_names()
    rng = random.Random(11)
    chosen = plain = 0
    for (opA, opB) in OP_PAIRS.values():
        cases = [(5120, 5120, 5120), (4608, 4608, 4608), (1280, 1280, 32768), (8192, 8192, 8192),
                 (4096, 4096, 4096), (5120, 5120, 5121), (5122, 5120, 5120), (5120, 5122, 5120), (3001, 2047, 1537)]
        cases += [(4 * rng.randint(16, 4096), 4 * rng.randint(16, 4096), 16 * rng.randint(8, 4096)) for _ in range(120)]
        cases += [(rng.randint(64, 16384), rng.randint(64, 16384), rng.randint(128, 65536)) for _ in range(40)]
        # short K, around the smallest K considered (1024)
        cases += [(10000, 10000, 30), (12000, 4000, 40), (10240, 10240, 1023), (10240, 10240, 1024)]
        cases += [(4 * rng.randint(512, 4096), 4 * rng.randint(512, 4096), 16 * rng.randint(1, 128)) for _ in range(40)]
        for M, N, K in cases:
            want = _streamk_select(blocks, norms, sk, opA, opB, M, N, K)
            got = sg.sgemm_mi355_select_streamk(opA, opB, M, N, K)
            assert (names[got] if got >= 0 else None) == want, (opA, opB, M, N, K)
            chosen += want is not None
            plain += want is None
        assert sg.sgemm_mi355_select_streamk(opA, opB, 8192, 8192, 8192) == -1  # whole rounds
        assert sg.sgemm_mi355_select_streamk(opA, opB, 10000, 10000, 30) == -1  # short K
    assert chosen > 100 and plain > 100


def test_streamk_table_and_errors():
    """The stream-K block names stream-K configurations of its op pair with
    positive times; the selection's argument errors."""
    from tests._table import read_streamk
    for pair, rows in read_streamk().items():
        assert len(rows) == 4
        for name, occ, us in rows:
            cid = _id(name)
            assert sg.sgemm_mi355_config_streamk(cid) == 1 and sg.sgemm_mi355_config_ops(cid) == pair
            assert occ >= 1 and 0.5 < us < 10.0
    assert sg.sgemm_mi355_config_streamk(10 ** 6) == sg.ERR_CONFIG
    with pytest.raises(sg.SgemmError):
        sg.sgemm_mi355_select_streamk(2, 0, 64, 64, 64)
    with pytest.raises(sg.SgemmError):
        sg.sgemm_mi355_select_streamk(0, 0, -1, 64, 64)
    assert sg.sgemm_mi355_select_streamk(0, 0, 0, 64, 64) == -1
    # arguments that describe no product need no workspace
    assert sg.sgemm_mi355_streamk_workspace_size(0, 0, 0, 64, 64, -1) == 0
    assert sg.sgemm_mi355_streamk_workspace_size(3, 0, 64, 64, 64, -1) == 0


def test_tuner_grids_reach_every_depth():
    """Every M, N in [64, 16384] and K in [16, 32768] is within a factor of
    two of a shape of the plain or the short-K grid (the nearest-shape radius)."""
    from dense_fp32_matrix_02_amd import tune
    ks = tune.GRID_KS + tune.SMALLK_KS
    near = lambda x, pts: any(x <= 2 * p and p <= 2 * x for p in pts)
    assert all(near(k, ks) for k in range(16, 32769))
    assert all(near(m, tune.GRID_SIDES) for m in range(64, 16385))
    assert not near(15, ks) and not near(32769, ks)


@pytest.mark.parametrize("argv", [["--passes", "0"], ["--smallk-grid", "--grid"],
                                  ["--smallk-grid", "--batch", "4"]])
def test_tuner_rejects_bad_options_before_timing(argv):
    from dense_fp32_matrix_02_amd import tune
    with pytest.raises(SystemExit):
        tune.main(argv)


def test_tuner_passes_keep_each_configurations_least_time():
    """time_passes times every configuration once per pass, passes in turn,
    and keeps each one's least timing."""
    from dense_fp32_matrix_02_amd import tune
    calls = []
    slow = {("a", 0): 14.0, ("a", 1): 7.0, ("b", 0): 8.0, ("b", 1): 9.0}

    def timer(name):
        n = sum(1 for c in calls if c == name)
        calls.append(name)
        return slow[(name, n)]
    assert tune.time_passes(["a", "b"], 2, timer) == {"a": 7.0, "b": 8.0}
    assert calls == ["a", "b", "a", "b"]
    assert tune.time_passes(["a"], 1, lambda n: 3.0) == {"a": 3.0}


def test_tuner_writes_the_table_it_documents(tmp_path):
    """tune.write_table on synthetic measurements: the candidates are the
    per-shape winners, times beyond TABLE_CUT x a shape's best are 0, every
    configuration's median time per busy unit is recorded, the stream-K block
    holds each configuration's median (time - overhead) per evenly dealt slab
    over the shapes where its direct kernel splits tiles (register-staged
    shapes and whole rounds left out), and the split-K block each shape's
    fastest split count."""
    import statistics
    from dense_fp32_matrix_02_amd import tune
    from tests._table import read_norms, read_split_table, read_streamk
    big, mid, sk = "mfma32_256x256x16_w4x4_lds2", "mfma32_128x128x32_w2x2_kg2", "mfma32_128x256x16_w2x4_lds2"
    occ = {big: 1, mid: 1, sk: 2}
    rows = [
        {"M": 8192, "N": 8192, "K": 8192, "ops": "nn", "batch": 1, "occupancy": occ,
         "times_ms": {big: 7.5, mid: 8.5, sk: 16.0}},
        {"M": 1024, "N": 1024, "K": 1024, "ops": "nn", "batch": 1, "occupancy": occ, "reps": 30, "passes": 2,
         "times_ms": {big: 0.07, mid: 0.03, sk: 0.04}},
        # stream-K grid rows: not plain shapes; one splits tiles, one is register-staged (K % 16),
        # one fills whole rounds of 256x256 tiles
        {"M": 5120, "N": 5120, "K": 5120, "ops": "nn", "batch": 1, "occupancy": occ, "streamk_grid": True,
         "times_ms": {big: 2.2}, "streamk_ms": {big: 1.9, sk: 1.95}},
        {"M": 2560, "N": 2560, "K": 8200, "ops": "nn", "batch": 1, "occupancy": occ, "streamk_grid": True,
         "times_ms": {big: 1.0}, "streamk_ms": {big: 0.8, sk: 0.81}},
        {"M": 2500, "N": 2500, "K": 8201, "ops": "nn", "batch": 1, "occupancy": occ, "streamk_grid": True,
         "times_ms": {big: 1.0}, "streamk_ms": {big: 5.0, sk: 5.0}},
        {"M": 4096, "N": 4096, "K": 4096, "ops": "nn", "batch": 1, "occupancy": occ, "streamk_grid": True,
         "times_ms": {big: 0.96}, "streamk_ms": {big: 0.96, sk: 1.0}},
        {"M": 64, "N": 64, "K": 4096, "ops": "nn", "batch": 1, "occupancy": occ,
         "times_ms": {}, "splitk_ms": {"1": 0.4, "2": 0.2, "4": 0.1, "8": 0.15}},
    ]
    path = tmp_path / "table.inc"
    tune.write_table(rows, str(path), reps=5)
    # rows without a recorded repetition count take the argument's
    assert ("time per launch of 5 to 30\n// launches run back to back, per configuration and shape, the least over "
            "up to 2 passes)") in path.read_text()
    blocks = _table(str(path))
    cands, shapes, times = blocks[(0, 0)]
    assert [n for n, _ in cands] == [big, mid]  # winners, in first-win order
    assert shapes == [(8192, 8192, 8192), (1024, 1024, 1024)]  # stream-K grid rows left out
    assert times[0] == [7500.0, 8500.0]
    assert times[1] == [0.0, 30.0]  # 70 us > 2 x 30 us: cut
    norms = {n: (o, us) for n, o, us in read_norms(str(path))[(0, 0)]}
    for n in (big, mid, sk):
        geo = tune.config_geometry(n)
        want = statistics.median(r["times_ms"][n] * 1e3 / tune.busy_time(*geo, occ[n], r["M"], r["N"], r["K"])
                                 for r in rows[:2] if n in r["times_ms"])
        assert norms[n][0] == occ[n] and norms[n][1] == pytest.approx(want, rel=1e-4)
    skn = {n: (o, us) for n, o, us in read_streamk(str(path))[(0, 0)]}
    assert set(skn) == {big, sk}

    def per_slab(ms, n, M, N, K):
        bm, bn, bk, _ = sg.sgemm_mi355_config_info(_id(n))
        return (ms * 1e3 - tune.STREAMK_OVERHEAD_US) / (-(-M // bm) * -(-N // bn) * (-(-K // bk) + STORE_DEPTH / bk) / 256)
    # 5120^3 and 2560^2 x 8200 count; 2500^2 x 8201 is register-staged, and 4096^3 fills whole
    # rounds in both tiles (256 tiles of 256x256 on 256 workgroups, 512 of 128x256 on 512)
    assert skn[big][1] == pytest.approx(statistics.median(
        [per_slab(1.9, big, 5120, 5120, 5120), per_slab(0.8, big, 2560, 2560, 8200)]), rel=1e-4)
    assert skn[sk] == (2, pytest.approx(statistics.median(
        [per_slab(1.95, sk, 5120, 5120, 5120), per_slab(0.81, sk, 2560, 2560, 8200)]), rel=1e-4))
    assert read_split_table(str(path)) == [(64, 64, 4096, 4)]
