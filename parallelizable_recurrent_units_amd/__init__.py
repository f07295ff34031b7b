"""One Simple Recurrent Unit layer's hot path on MI355X (gfx950).

The computation is that of Lei, "When Attention Meets Fast Recurrence"
(SRU background section, Eqs. 1-5): one projection GEMM followed by a fused
elementwise recurrence, plus its backward pass and a linear (v = 0) mode
evaluated as a time-chunked scan.  All of it runs in the HIP kernels of
``libsru.so`` behind the C ABI in ``include/sru.h``; this package only binds
that ABI (``_binding``), allocates outputs for convenience (``layer``) and
draws seeded synthetic inputs (``workloads``).
"""
from ._binding import (  # noqa: F401
    SRU_FACT_BWD_Q, SRU_FACT_BWD_X, SRU_FACT_Q, SRU_FACT_U, SRU_FACT_WGRAD_O, SRU_FACT_WGRAD_Q,
    SRU_WS_FACTORED_WEIGHT, sru_project_factored, sru_project_factored_bwd_weight,
    SruAttnCfg, sru_attention_forward, sru_attention_workspace_size, sru_step, sru_round_bf16,
    sru_attention_backward, sru_attention_backward_workspace_size,
    EXPORTED, LIB_PATH, SRU_BF16, SRU_BWD, SRU_ERR_INVALID_ARG, SRU_ERR_LAUNCH,
    SRU_ERR_NO_DEVICE, SRU_ERR_UNSUPPORTED, SRU_ERR_WORKSPACE, SRU_F32, SRU_FWD, SRU_OK,
    SRU_PROJ_BWD_DATA, SRU_PROJ_BWD_DATA_WT, SRU_PROJ_FWD, SRU_WS_BACKWARD, SRU_WS_BWD_WEIGHT, SRU_WS_LINEAR_BWD,
    SRU_WS_LINEAR_FWD,
    SruError, SruShape, load_library, sru_backward, sru_forward, sru_linear_scan, sru_project,
    sru_project_bwd_weight, sru_transpose_weight, sru_workspace_size,
    SRU_WS_ERROR_OFFSET, workspace_error_word, check_workspace,
    SRU_BACKWARD_STATIC_SCRATCH_BYTES, sru_backward_static)
