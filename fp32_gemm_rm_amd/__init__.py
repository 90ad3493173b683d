"""Row-major FP32 GEMM for AMD Instinct MI355X (gfx950).

``C = alpha * A @ B + beta * C`` on row-major operands with leading
dimensions, with transposed operands, column-major storage and strided
batches as further forms, computed by hand-written HIP kernels in
``libsgemm_rm.so`` behind a C ABI (``include/sgemm_rm.h``).  The Python side
only marshals arguments.
"""
from .binding import (  # noqa: F401
    SGEMM_RM_OP_N,
    SGEMM_RM_OP_T,
    SGEMM_RM_VARIANT_AUTO,
    SGEMM_RM_VARIANT_LDS_TILED,
    SGEMM_RM_VARIANT_MFMA,
    SGEMM_RM_VARIANT_MFMA_T32,
    SGEMM_RM_VARIANT_MFMA_T16,
    SGEMM_RM_VARIANT_MFMA_T192,
    SGEMM_RM_VARIANT_MFMA_T64,
    SGEMM_RM_VARIANT_MFMA_T128,
    SGEMM_RM_VARIANT_MFMA_T256,
    SGEMM_RM_VARIANT_NAIVE,
    SGEMM_RM_VARIANT_REGBLOCK,
    TILE_VARIANTS,
    VARIANTS,
    SgemmArgumentError,
    SgemmError,
    SgemmLaunchError,
    library_path,
    load_library,
    sgemm,
    sgemm_batched,
    sgemm_cm,
    sgemm_cm_strided_batched_ex,
    sgemm_cm_strided_batched_ws,
    sgemm_rm,
    sgemm_rm_ex,
    sgemm_rm_op,
    sgemm_rm_op_strided_batched_ex,
    sgemm_rm_op_strided_batched_noalloc,
    sgemm_rm_op_strided_batched_ws,
    sgemm_rm_plan_tiles,
    sgemm_rm_strerror,
    sgemm_rm_strided_batched,
    sgemm_rm_strided_batched_ex,
    sgemm_rm_workspace_size,
)
