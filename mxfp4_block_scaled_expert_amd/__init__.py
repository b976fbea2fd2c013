"""mxq: scaled low-precision GEMM and routed fused-MoE experts for AMD MI355X (gfx950).

The compute lives in ``libmxq.so`` (hand-written HIP kernels behind the C ABI
of ``include/mxq.h``); ``ops`` is a thin torch binding that only marshals
arguments.  Build the library with ``python -m mxfp4_block_scaled_expert_amd.build``.
"""

from .ops import (  # noqa: F401
    init,
    per_token_group_quant_fp8,
    fp8_scaled_mm,
    fp8_scaled_bmm,
    block_fp8_linear,
    mxfp8_quant,
    mx_linear,
    moe_max_blocks,
    moe_align,
    fused_moe_fp8,
    fused_moe_mxfp4,
    fused_moe_workspace,
    moe_prepack,
    moe_prepack_scales,
    fused_moe_workspace_layout,
    silu_and_mul,
    Dispatch,
)
from ._lib import (  # noqa: F401
    LIB_PATH,
    MXQ_DISPATCH_PER_BLOCK,
    MXQ_DISPATCH_FORCED,
    MXQ_DISPATCH_LAYER_AVERAGE,
    MXQ_TINY_MFMA,
    MXQ_TINY_GEMV,
    MXQ_LAYOUT_PLAIN,
    MXQ_LAYOUT_TILED,
    MXQ_K_SPLIT_AUTO,
    MXQ_SORT_AUTO,
    MXQ_SORT_ALWAYS,
    MXQ_FUSE_AUTO,
    MXQ_FUSE_NONE,
)
