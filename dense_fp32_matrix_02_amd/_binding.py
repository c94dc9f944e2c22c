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

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_GEMM = [_I, _I, _I, _P, _I, _P, _I, _P, _I, _P]


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
    lib = ctypes.CDLL(path)
    lib.sgemm_mi355.argtypes = _GEMM
    lib.sgemm_mi355_valu.argtypes = _GEMM
    lib.sgemm_mi355_with_config.argtypes = _GEMM + [_I]
    lib.sgemm_mi355_validate.argtypes = [_I, _I, _I, _P, _I, _P, _I, _P, _I]
    lib.sgemm_mi355_select_config.argtypes = [_I, _I, _I]
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
                 "sgemm_mi355_tile_map"):
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


def sgemm_mi355_validate(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return load().sgemm_mi355_validate(M, N, K, A, lda, B, ldb, C, ldc)


def sgemm_mi355_select_config(M, N, K) -> int:
    return load().sgemm_mi355_select_config(M, N, K)


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

def _ld(x, name):
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if x.shape[0] and x.shape[1] and x.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    return max(x.stride(0) if x.shape[0] > 1 else x.shape[1], 1)


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
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if out.shape != (M, N) or out.dtype != torch.float32 or not out.is_cuda:
        raise ValueError("out must be an M x N float32 GPU tensor")
    s = (stream or torch.cuda.current_stream(A.device)).cuda_stream
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
