"""MI355X (gfx950) forward pass of MHLA -- Multi-Head Linear Attention with
token-level heads ("MHLA: Restoring Expressivity of Linear Attention via
Token-Level Multi-Head", §4.1).

The compute lives in ``libmhla.so`` (hand-written HIP kernels behind the C
ABI of ``include/mhla.h``).  This package is a thin ctypes binding whose
functions carry the C names; it only marshals arguments.  Building the
library: ``python -m token_level_head_mhla_amd.build``.
"""
from ._binding import (  # noqa: F401
    MHLA_DTYPE_BF16, MHLA_DTYPE_F32, MHLA_ERR_ALIAS, MHLA_ERR_HIP, MHLA_ERR_INVALID_ARG,
    MHLA_ERR_SHAPE, MHLA_ERR_UNSUPPORTED, MHLA_FLAG_CAUSAL, MHLA_FLAG_NO_NORM, MHLA_OK,
    MHLA_PATH_AUTO, MHLA_PATH_BLOCKED, MHLA_PATH_COLUMNS, MHLA_PATH_FUSED, MHLA_PATH_GENERIC,
    MHLA_PATH_PAIRS,
    MHLA_PHI_ELU1, MHLA_PHI_RELU, MHLA_MAX_LAUNCHES, MhlaError, BlockShape, EXPORTED_SYMBOLS,
    PreparedForward, library_path,
    load_library, mhla_backward, mhla_decode_prefill, mhla_decode_state_bytes, mhla_decode_step,
    mhla_decode_steps,
    mhla_error_string,
    mhla_forward, mhla_forward_ex, mhla_forward_noalloc, mhla_forward_path, mhla_forward_profiled,
    MHLA_NOALLOC_SCRATCH_BYTES,
    mhla_last_error, mhla_lb_init, mhla_num_blocks, mhla_plan, mhla_plan_ex, mhla_release,
    mhla_validate, mhla_workspace_bytes, mhla_workspace_bytes_ex,
)
