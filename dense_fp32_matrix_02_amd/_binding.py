"""ctypes binding of libsgemm_mi355.so (argument marshalling only).

Every function of the C ABI in include/sgemm_mi355.h is exposed under the same
name and takes the same arguments: device addresses and a HIP stream handle
are passed as Python ints. ``matmul`` is a convenience wrapper that takes
torch device tensors, reads their addresses, strides and the current stream,
and calls ``sgemm_mi355`` (or a variant); all arithmetic runs in the
library's HIP kernels. There is no fallback: if the library is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm_mi355.so")

OK = 0
ERR_DIM, ERR_LD, ERR_NULL, ERR_ALIAS, ERR_EXTENT, ERR_LAUNCH, ERR_CONFIG, ERR_ALIGN = (
    -1, -2, -3, -4, -5, -6, -7, -8)
ERR_STRIDE, ERR_OP, ERR_WORKSPACE, ERR_SCRATCH = -9, -10, -11, -12
SCRATCH_BYTES = 32 << 20
OP_N, OP_T = 0, 1

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_LL = ctypes.c_longlong
_GEMM = [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P]
_GEMM_EX = [_I, _I, _I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, _P]
_GEMM_SB = [_I, _I, _I, _I, _I, _F, _P, _I, _LL, _P, _I, _LL, _F, _P, _I, _LL, _I, _P]


class SgemmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m dense_fp32_matrix_02_amd.build` "
            "(the GEMM has no non-HIP implementation)")
    # The library needs libamdhip64.so.7, and torch carries its own copy of the
    # HIP runtime under that soname. With torch loaded first the library binds
    # to torch's copy, so torch's streams and memory are valid for it; loaded
    # the other way round, torch would bring a second runtime into the process
    # and every launch on one of its streams would be rejected.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.sgemm_mi355.argtypes = _GEMM
    lib.sgemm_mi355_valu.argtypes = _GEMM
    lib.sgemm_mi355_with_config.argtypes = _GEMM + [_I]
    lib.sgemm_mi355_ex.argtypes = _GEMM_EX
    lib.sgemm_mi355_strided_batched.argtypes = _GEMM_SB
    lib.sgemm_mi355_strided_batched_with_config.argtypes = _GEMM_SB + [_I]
    lib.sgemm_mi355_splitk.argtypes = _GEMM_EX[:-1] + [_I, _P, ctypes.c_size_t, _P]
    lib.sgemm_mi355_splitk_with_config.argtypes = _GEMM_EX[:-1] + [_I, _P, ctypes.c_size_t, _P, _I]
    lib.sgemm_mi355_splitk_noalloc.argtypes = _GEMM_EX[:-1] + [_I, _P]
    lib.sgemm_mi355_splitk_workspace_size.argtypes = [_I, _I, _I, _I]
    lib.sgemm_mi355_splitk_workspace_size.restype = ctypes.c_size_t
    lib.sgemm_mi355_select_splitk.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
    lib.sgemm_mi355_streamk.argtypes = _GEMM_EX[:-1] + [_P, ctypes.c_size_t, _P]
    lib.sgemm_mi355_streamk_with_config.argtypes = _GEMM_EX[:-1] + [_P, ctypes.c_size_t, _P, _I]
    lib.sgemm_mi355_streamk_workspace_size.argtypes = [_I] * 6
    lib.sgemm_mi355_streamk_workspace_size.restype = ctypes.c_size_t
    lib.sgemm_mi355_select_streamk.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(_I)]
    lib.sgemm_mi355_config_streamk.argtypes = [_I]
    lib.sgemm_mi355_validate.argtypes = [_I, _I, _I, _P, _I, _P, _I, _P, _I]
    lib.sgemm_mi355_validate_ex.argtypes = [_I, _I, _I, _I, _I, _F, _P, _I, _LL, _P, _I, _LL, _F, _P,
                                            _I, _LL, _I]
    lib.sgemm_mi355_select_config_ex.argtypes = [_I] * 6
    lib.sgemm_mi355_select_config_valu.argtypes = [_I] * 3
    lib.sgemm_mi355_config_ops.argtypes = [_I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
    lib.sgemm_mi355_config_occupancy.argtypes = [_I, ctypes.POINTER(_I)]
    lib.sgemm_mi355_select_config.argtypes = [_I, _I, _I]
    lib.sgemm_mi355_selected_config.argtypes = [_I, _I, _I, _P, _I, _P, _I]
    lib.sgemm_mi355_config_staging.argtypes = [_I, _I, _I, _I, _P, _I, _P, _I]
    lib.sgemm_mi355_num_configs.argtypes = []
    lib.sgemm_mi355_config_name.argtypes = [_I]
    lib.sgemm_mi355_config_name.restype = ctypes.c_char_p
    lib.sgemm_mi355_config_info.argtypes = [_I] + [ctypes.POINTER(_I)] * 4
    lib.sgemm_mi355_tile_map.argtypes = [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
    lib.sgemm_mi355_strerror.argtypes = [_I]
    lib.sgemm_mi355_strerror.restype = ctypes.c_char_p
    lib.sgemm_mi355_version.argtypes = []
    lib.sgemm_mi355_version.restype = ctypes.c_char_p
    for name in ("sgemm_mi355", "sgemm_mi355_valu", "sgemm_mi355_with_config", "sgemm_mi355_validate",
                 "sgemm_mi355_select_config", "sgemm_mi355_num_configs", "sgemm_mi355_config_info",
                 "sgemm_mi355_tile_map", "sgemm_mi355_ex", "sgemm_mi355_strided_batched",
                 "sgemm_mi355_strided_batched_with_config", "sgemm_mi355_validate_ex",
                 "sgemm_mi355_select_config_ex", "sgemm_mi355_config_ops", "sgemm_mi355_splitk",
                 "sgemm_mi355_splitk_with_config", "sgemm_mi355_select_splitk",
                 "sgemm_mi355_select_config_valu", "sgemm_mi355_streamk", "sgemm_mi355_streamk_with_config",
                 "sgemm_mi355_select_streamk", "sgemm_mi355_config_streamk", "sgemm_mi355_selected_config",
                 "sgemm_mi355_config_staging", "sgemm_mi355_splitk_noalloc"):
        getattr(lib, name).restype = _I
    _lib = lib
    return lib


# ---- the C ABI, name for name ------------------------------------------------

def sgemm_mi355(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return load().sgemm_mi355(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_mi355_valu(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return load().sgemm_mi355_valu(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_mi355_with_config(M, N, K, A, lda, B, ldb, C, ldc, stream, config) -> int:
    return load().sgemm_mi355_with_config(M, N, K, A, lda, B, ldb, C, ldc, stream, config)


def sgemm_mi355_ex(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream) -> int:
    return load().sgemm_mi355_ex(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_mi355_strided_batched(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                                ldc, strideC, batch, stream) -> int:
    return load().sgemm_mi355_strided_batched(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                              strideB, beta, C, ldc, strideC, batch, stream)


def sgemm_mi355_strided_batched_with_config(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                            strideB, beta, C, ldc, strideC, batch, stream,
                                            config) -> int:
    return load().sgemm_mi355_strided_batched_with_config(
        opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
        stream, config)


def sgemm_mi355_splitk(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits, workspace,
                       workspace_bytes, stream) -> int:
    return load().sgemm_mi355_splitk(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                                     workspace, workspace_bytes, stream)


def sgemm_mi355_splitk_with_config(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                                   workspace, workspace_bytes, stream, config) -> int:
    return load().sgemm_mi355_splitk_with_config(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                                 splits, workspace, workspace_bytes, stream, config)


def sgemm_mi355_splitk_noalloc(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits, stream) -> int:
    return load().sgemm_mi355_splitk_noalloc(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits, stream)


def sgemm_mi355_splitk_workspace_size(M, N, K, splits) -> int:
    return load().sgemm_mi355_splitk_workspace_size(M, N, K, splits)


def sgemm_mi355_select_splitk(opA, opB, M, N, K):
    """Return (splits, config) the library suggests, or raise SgemmError."""
    sp, cf = _I(), _I()
    rc = load().sgemm_mi355_select_splitk(opA, opB, M, N, K, ctypes.byref(sp), ctypes.byref(cf))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_select_splitk")
    return sp.value, cf.value


def sgemm_mi355_streamk(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                        stream) -> int:
    return load().sgemm_mi355_streamk(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                      workspace_bytes, stream)


def sgemm_mi355_streamk_with_config(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                    workspace_bytes, stream, config) -> int:
    return load().sgemm_mi355_streamk_with_config(opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                                  workspace, workspace_bytes, stream, config)


def sgemm_mi355_streamk_workspace_size(opA, opB, M, N, K, config=-1) -> int:
    return load().sgemm_mi355_streamk_workspace_size(opA, opB, M, N, K, config)


def sgemm_mi355_select_streamk(opA, opB, M, N, K) -> int:
    """The configuration the stream-K call would run, or -1 (plain path); raises on bad arguments."""
    cf = _I()
    rc = load().sgemm_mi355_select_streamk(opA, opB, M, N, K, ctypes.byref(cf))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_select_streamk")
    return cf.value


def sgemm_mi355_config_streamk(config) -> int:
    return load().sgemm_mi355_config_streamk(config)


def sgemm_mi355_validate_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                            strideC, batch) -> int:
    return load().sgemm_mi355_validate_ex(opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
                                          beta, C, ldc, strideC, batch)


def sgemm_mi355_select_config_valu(M, N, K) -> int:
    return load().sgemm_mi355_select_config_valu(M, N, K)


def sgemm_mi355_select_config_ex(opA, opB, M, N, K, batch) -> int:
    return load().sgemm_mi355_select_config_ex(opA, opB, M, N, K, batch)


def sgemm_mi355_config_ops(config):
    """Return (opA, opB) the configuration was built for, or raise SgemmError."""
    a, b = _I(), _I()
    rc = load().sgemm_mi355_config_ops(config, ctypes.byref(a), ctypes.byref(b))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_config_ops")
    return a.value, b.value


def sgemm_mi355_config_occupancy(config) -> int:
    """Workgroups of the configuration one compute unit holds at once (needs
    a GPU), or raise SgemmError."""
    n = _I()
    rc = load().sgemm_mi355_config_occupancy(config, ctypes.byref(n))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_config_occupancy")
    return n.value


def sgemm_mi355_validate(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return load().sgemm_mi355_validate(M, N, K, A, lda, B, ldb, C, ldc)


def sgemm_mi355_select_config(M, N, K) -> int:
    return load().sgemm_mi355_select_config(M, N, K)


def sgemm_mi355_selected_config(M, N, K, A, lda, B, ldb) -> int:
    return load().sgemm_mi355_selected_config(M, N, K, A, lda, B, ldb)


def sgemm_mi355_config_staging(config, M, N, K, A, lda, B, ldb) -> int:
    return load().sgemm_mi355_config_staging(config, M, N, K, A, lda, B, ldb)


def sgemm_mi355_num_configs() -> int:
    return load().sgemm_mi355_num_configs()


def sgemm_mi355_config_name(config) -> str | None:
    r = load().sgemm_mi355_config_name(config)
    return r.decode() if r is not None else None


def sgemm_mi355_config_info(config):
    """Return (bm, bn, bk, threads) or raise SgemmError."""
    v = [_I() for _ in range(4)]
    rc = load().sgemm_mi355_config_info(config, *[ctypes.byref(x) for x in v])
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_config_info")
    return tuple(x.value for x in v)


def sgemm_mi355_tile_map(bid, tiles_m, tiles_n, group_m):
    """Return (tm, tn) of workgroup `bid`, or raise SgemmError."""
    tm, tn = _I(), _I()
    rc = load().sgemm_mi355_tile_map(bid, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_tile_map")
    return tm.value, tn.value


def sgemm_mi355_strerror(code) -> str:
    return load().sgemm_mi355_strerror(code).decode()


def sgemm_mi355_version() -> str:
    return load().sgemm_mi355_version().decode()


strerror = sgemm_mi355_strerror


def config_names():
    return [sgemm_mi355_config_name(i) for i in range(sgemm_mi355_num_configs())]


def config_id(name: str) -> int:
    names = config_names()
    if name not in names:
        raise KeyError(name)
    return names.index(name)


# ---- torch convenience wrapper (marshalling only) ---------------------------

def _empty_on(shape, device, stream):
    """A float32 tensor allocated with torch's caching allocator on `stream`,
    the stream the library launches on. The allocator ties a block to the
    stream it was allocated on and hands it out again only after the work
    queued on that stream up to its release has run, so a temporary
    (workspace) dropped on return cannot be reused while the kernels that
    read or write it are still pending."""
    import torch

    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=torch.float32, device=device)


def _ld(x, name):
    """Leading dimension (row stride in elements) of a 2-D tensor whose rows
    are contiguous. A dimension of size 1 may carry any stride in torch, so
    its stride is not looked at."""
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = x.shape
    if rows and cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    if rows > 1:
        if x.stride(0) < cols:
            raise ValueError(f"{name} row stride is smaller than its row length")
        return max(x.stride(0), 1)
    return max(cols, 1)


def matmul(A, B, out=None, *, kind: str = "mfma", config: int | None = None, stream=None):
    """C = A.B for FP32 torch tensors on the GPU through the C ABI.

    A (M x K) and B (K x N) may have padded rows (stride(0) >= row length);
    ``out`` (M x N, may be a padded view) receives C and is allocated with
    torch.empty when omitted. ``kind`` selects the matrix-core path ("mfma")
    or the vector comparison kernel ("valu"); ``config`` forces a kernel
    configuration id. Runs on ``stream`` (a torch stream, default: current).
    """
    import torch

    for x, n in ((A, "A"), (B, "B")):
        if x.dtype != torch.float32 or not x.is_cuda:
            raise TypeError(f"{n} must be a float32 GPU tensor")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    s_obj = stream or torch.cuda.current_stream(A.device)
    if out is None:
        out = _empty_on((M, N), A.device, s_obj)
    if out.shape != (M, N) or out.dtype != torch.float32 or not out.is_cuda:
        raise ValueError("out must be an M x N float32 GPU tensor")
    s = s_obj.cuda_stream
    args = (M, N, K, A.data_ptr(), _ld(A, "A"), B.data_ptr(), _ld(B, "B"),
            out.data_ptr(), _ld(out, "C"), s)
    if config is not None:
        rc = sgemm_mi355_with_config(*args, config)
    elif kind == "mfma":
        rc = sgemm_mi355(*args)
    elif kind == "valu":
        rc = sgemm_mi355_valu(*args)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355")
    return out


def _op_dims(X, op):
    return (X.shape[1], X.shape[0]) if op else (X.shape[0], X.shape[1])


def gemm(A, B, C=None, *, opA: int = OP_N, opB: int = OP_N, alpha: float = 1.0, beta: float = 0.0,
         config: int | None = None, stream=None):
    """C = alpha*op(A).op(B) + beta*C for FP32 GPU tensors through the C ABI.

    A, B and C are 2-D row-major tensors (rows may be padded); op = OP_T reads
    the stored matrix transposed. C is allocated (and beta must be 0) when
    omitted. ``config`` forces a configuration built for (opA, opB).
    """
    import torch

    M, K = _op_dims(A, opA)
    K2, N = _op_dims(B, opB)
    if K != K2:
        raise ValueError("inner dimensions differ")
    s_obj = stream or torch.cuda.current_stream(A.device)
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = _empty_on((M, N), A.device, s_obj)
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be M x N")
    for x, n in ((A, "A"), (B, "B"), (C, "C")):
        if x.dtype != torch.float32 or not x.is_cuda:
            raise TypeError(f"{n} must be a float32 GPU tensor")
    s = s_obj.cuda_stream
    args = (opA, opB, M, N, K, alpha, A.data_ptr(), _ld(A, "A"), 0, B.data_ptr(), _ld(B, "B"), 0,
            beta, C.data_ptr(), _ld(C, "C"), 0, 1, s)
    rc = (sgemm_mi355_strided_batched(*args) if config is None
          else sgemm_mi355_strided_batched_with_config(*args, config))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_strided_batched")
    return C


def gemm_strided_batched(A, B, C=None, *, opA: int = OP_N, opB: int = OP_N, alpha: float = 1.0,
                         beta: float = 0.0, config: int | None = None, stream=None):
    """Batched form on 3-D tensors (batch, rows, cols) with contiguous rows.

    The batch stride of each operand is its stride(0); a stride of 0 (an
    expanded tensor) shares one matrix across the batch.
    """
    import torch

    batch = C.shape[0] if C is not None else max(A.shape[0], B.shape[0])
    M, K = _op_dims(A[0], opA)
    K2, N = _op_dims(B[0], opB)
    if K != K2:
        raise ValueError("inner dimensions differ")
    s_obj = stream or torch.cuda.current_stream(A.device)
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = _empty_on((batch, M, N), A.device, s_obj)
    s = s_obj.cuda_stream
    sa = A.stride(0) if A.shape[0] > 1 else 0
    sb = B.stride(0) if B.shape[0] > 1 else 0
    args = (opA, opB, M, N, K, alpha, A.data_ptr(), _ld(A[0], "A"), sa, B.data_ptr(), _ld(B[0], "B"),
            sb, beta, C.data_ptr(), _ld(C[0], "C"), C.stride(0), batch, s)
    rc = (sgemm_mi355_strided_batched(*args) if config is None
          else sgemm_mi355_strided_batched_with_config(*args, config))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_strided_batched")
    return C


def gemm_splitk(A, B, C=None, *, splits: int | None = None, opA: int = OP_N, opB: int = OP_N,
                alpha: float = 1.0, beta: float = 0.0, workspace=None, config: int | None = None,
                stream=None):
    """Split-K product C = alpha*op(A).op(B) + beta*C through the C ABI.

    ``splits`` defaults to the library's suggestion; the workspace (a float32
    GPU tensor of at least sgemm_mi355_splitk_workspace_size bytes) is
    allocated with torch when omitted. Returns C.
    """
    import torch

    M, K = _op_dims(A, opA)
    K2, N = _op_dims(B, opB)
    if K != K2:
        raise ValueError("inner dimensions differ")
    s_obj = stream or torch.cuda.current_stream(A.device)
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = _empty_on((M, N), A.device, s_obj)
    if splits is None:
        splits, suggested = sgemm_mi355_select_splitk(opA, opB, M, N, K)
        config = suggested if config is None else config
    need = sgemm_mi355_splitk_workspace_size(M, N, K, splits)
    if workspace is None:
        workspace = _empty_on(((max(need, 4) + 3) // 4,), A.device, s_obj)
    s = s_obj.cuda_stream
    args = (opA, opB, M, N, K, alpha, A.data_ptr(), _ld(A, "A"), B.data_ptr(), _ld(B, "B"), beta,
            C.data_ptr(), _ld(C, "C"), splits, workspace.data_ptr(), workspace.numel() * 4, s)
    rc = (sgemm_mi355_splitk(*args) if config is None else sgemm_mi355_splitk_with_config(*args, config))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_splitk")
    return C


def gemm_streamk(A, B, C=None, *, opA: int = OP_N, opB: int = OP_N, alpha: float = 1.0, beta: float = 0.0,
                 workspace=None, config: int | None = None, stream=None):
    """Stream-K product C = alpha*op(A).op(B) + beta*C through the C ABI.

    Without ``config`` the library chooses (and may run the plain path); the
    workspace (a float32 GPU tensor of at least
    sgemm_mi355_streamk_workspace_size bytes, 16-byte aligned) is allocated
    with torch when omitted. Returns C.
    """
    import torch

    M, K = _op_dims(A, opA)
    K2, N = _op_dims(B, opB)
    if K != K2:
        raise ValueError("inner dimensions differ")
    s_obj = stream or torch.cuda.current_stream(A.device)
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = _empty_on((M, N), A.device, s_obj)
    need = sgemm_mi355_streamk_workspace_size(opA, opB, M, N, K, -1 if config is None else config)
    if workspace is None:
        workspace = _empty_on(((max(need, 16) + 3) // 4,), A.device, s_obj)
    s = s_obj.cuda_stream
    args = (opA, opB, M, N, K, alpha, A.data_ptr(), _ld(A, "A"), B.data_ptr(), _ld(B, "B"), beta,
            C.data_ptr(), _ld(C, "C"), workspace.data_ptr(), workspace.numel() * 4, s)
    rc = (sgemm_mi355_streamk(*args) if config is None else sgemm_mi355_streamk_with_config(*args, config))
    if rc != OK:
        raise SgemmError(rc, "sgemm_mi355_streamk")
    return C
