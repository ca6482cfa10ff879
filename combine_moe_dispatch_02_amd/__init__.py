"""MI355X-native single-GPU MoE dispatch -> expert FFN -> combine (libmoe355, C ABI + HIP).

The product path is the in-tree ``libmoe355.so``; importing this package does not
load it, the first call does, and fails loudly if it has not been built.
"""
from .layer import (  # noqa: F401
    MOE_BF16,
    MOE_FP8_E4M3_G128,
    MOE_MXFP4,
    MOE_WEIGHTS_MFMA_TILED,
    MOE_WEIGHTS_ROW_MAJOR,
    MoeError,
    Plan,
    StreamMoE,
    TileConfig,
    Workspace,
    device_cu_count,
    make_streams,
    moe_combine,
    moe_combine_backward,
    moe_dispatch_backward,
    moe_expert_ffn_backward,
    moe_expert_ffn_train,
    moe_pack_weights_transposed,
    moe_dispatch,
    moe_expert_ffn,
    moe_expert_ffn_combine,
    moe_get_error,
    moe_pack_mx_scales,
    moe_pack_weights,
    moe_plan,
    moe_plan_noalloc,
    moe_query_pool_rows,
    pool_rows_upper_bound,
    stream_moe,
    workspace_bytes,
)
