"""MI355X-native FP32 GEMM: C = A.B on row-major matrices (alpha = 1, beta = 0).

The computation lives in libsgemm_mi355.so (hand-written HIP for gfx950,
C ABI in include/sgemm_mi355.h); this package only loads it and marshals
arguments. Build it with ``python -m dense_fp32_matrix_02_amd.build``.
"""
from ._binding import (  # noqa: F401
    ERR_ALIAS, ERR_ALIGN, ERR_CONFIG, ERR_DIM, ERR_EXTENT, ERR_LAUNCH, ERR_LD, ERR_NULL, ERR_OP,
    ERR_SCRATCH, ERR_STRIDE, ERR_WORKSPACE, LIB_PATH, SCRATCH_BYTES, OK, OP_N, OP_T, SgemmError, config_id, config_names, gemm,
    gemm_splitk, gemm_streamk, gemm_strided_batched, load, matmul, sgemm_mi355, sgemm_mi355_config_info,
    sgemm_mi355_config_name, sgemm_mi355_config_occupancy, sgemm_mi355_config_ops, sgemm_mi355_ex,
    sgemm_mi355_num_configs,
    sgemm_mi355_select_config, sgemm_mi355_select_config_ex, sgemm_mi355_select_config_valu,
    sgemm_mi355_selected_config, sgemm_mi355_config_staging,
    sgemm_mi355_select_splitk, sgemm_mi355_select_streamk, sgemm_mi355_config_streamk,
    sgemm_mi355_streamk, sgemm_mi355_streamk_with_config, sgemm_mi355_streamk_workspace_size,
    sgemm_mi355_splitk, sgemm_mi355_splitk_noalloc, sgemm_mi355_splitk_with_config, sgemm_mi355_splitk_workspace_size, sgemm_mi355_strerror,
    sgemm_mi355_strided_batched, sgemm_mi355_strided_batched_with_config, sgemm_mi355_tile_map,
    sgemm_mi355_valu, sgemm_mi355_validate, sgemm_mi355_validate_ex, sgemm_mi355_version,
    sgemm_mi355_with_config, strerror)

__all__ = [n for n in dir() if not n.startswith("_")]
