"""CPU oracle of the MoE dispatch -> expert FFN -> combine path.

Test infrastructure only: tests/, the smoke check and the benchmark's
CPU-baseline leg are its only users. Plain NumPy in float64; it shares no code
with the GPU library and imports nothing from it.
"""
from .e4m3 import E4M3_MAX, E4M3_VALUES, e4m3_decode, e4m3_encode  # noqa: F401
from .moe_backward import OracleGrads, expert_backward, expert_forward, moe_layer_backward, silu_grad  # noqa: F401
from .mx import (  # noqa: F401
    MX_BLOCK,
    dequantize_mx_e4m3,
    dequantize_mx_fp4,
    e2m1_decode,
    e8m0_decode,
    mx_shared_exponent,
    quantize_mx_e4m3,
    unpack_fp4,
)
from .moe_oracle import (  # noqa: F401
    GROUP,
    OraclePlan,
    OracleResult,
    bf16_bits,
    bf16_to_f64,
    combine,
    dequantize_blocks,
    dequantize_groups,
    dispatch,
    expert_ffn,
    expert_weights_f64,
    fp8_codes,
    max_norm_rel_err,
    moe_layer,
    plan,
    pool_rows_bound,
    quantize_groups,
    silu,
    token_rows,
)
