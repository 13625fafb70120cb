"""AcceptMoE verify-block MoE layer for MI355X (gfx950).

The compute lives in ``libacceptmoe.so`` (HIP kernels behind the C ABI in
``include/acceptmoe.h``); this package is its Python binding.  Importing it
without the built library raises ImportError: there is no CPU fallback.
"""

from ._lib import (  # noqa: F401
    AcceptMoEError,
    BF16,
    EHIP,
    EINVAL,
    ENOTSUP,
    ERR_BAD_TREE,
    ERR_COMMIT,
    ERR_DEPTH,
    ERR_NONFINITE,
    EXPORTED,
    F32,
    F_LOGITS_IN,
    F_NATURAL,
    F_NO_RENORM,
    FP8_E4M3FN,
    LIB_PATH,
    OK,
    STATS_BYTES,
    Inputs,
    Outputs,
    Shape,
    acceptmoe_select,
    acceptmoe_select_workspace_size,
    acceptmoe_set_stage_timer,
    STAGE_COMBINE,
    STAGE_DOWN,
    STAGE_EXPERTS,
    STAGE_GATEUP,
    STAGE_NONE,
    STAGE_PERMUTE,
    STAGE_SELECT,
    acceptmoe_workspace_size,
    decode_stats,
    dtype_code,
    make_shape,
    moe_combine,
    moe_grouped_swiglu,
    moe_grouped_swiglu_workspace_size,
    moe_route_permute,
    new_stats,
    raw,
    verify_block,
    version,
)
from .layer import VerifyLayer  # noqa: F401
