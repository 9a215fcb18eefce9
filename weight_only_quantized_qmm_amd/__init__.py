"""Split-K W4A16 group-128 quantized matmul for MI355X (gfx950).

The computation lives in libqmm.so (hand-written HIP kernels behind the C ABI
of include/qmm.h); this package is its ctypes binding. The library is loaded on
first use and every call raises if it is missing.
"""
from .binding import (  # noqa: F401
    EXPORTED_DATA, EXPORTED_FUNCTIONS, QMM_ERR_ALIGN, QMM_ERR_ARG, QMM_ERR_HIP, QMM_ERR_SCRATCH,
    QMM_ERR_SHAPE, QMM_ERR_SIZE, QMM_ERR_WORKSPACE, QMM_NOALLOC_SCRATCH_BYTES, QMM_OK, QMM_PARTIAL_BF16,
    QMM_PARTIAL_F32, QmmError,
    bf16_splitk, effective_split, lib, policy_preset, qmm_bf16_splitk, qmm_plan, qmm_policy,
    qmm_gemv_min_split, qmm_splitk_plan, qmm_splitk_reduce, qmm_status_string, qmm_w4a16_g128,
    qmm_attn_decode, qmm_attn_decode_split, qmm_attn_decode_workspace_bytes, qmm_streamk_workspace_bytes,
    qmm_splitk_reduce_cols, qmm_w4a16_g128_f32p, qmm_w4a16_g128_noalloc, qmm_w4a16_g128_pass1,
    qmm_w4a16_g128_streamk, qmm_w4a16_gemv,
    qmm_wna16, qmm_wna16_plan, w4a16, w4a16_workspace_bytes, wna16)
