"""CPU oracle for the MoE decode/verify round — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy written from the pages' description of the round.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it.  The library itself never calls it and shares no code with it.

Parity status of each function is listed in moe_oracle's header.
"""
from .moe_oracle import (  # noqa: F401
    unpack_codes,
    unpack_scale_min,
    dequantize,
    unpack_superblocks,
    dequantize_q4s256,
    dequantize_any,
    router_logits,
    select_topk,
    selection_gap,
    routing_weights,
    silu,
    expert_matrices,
    swiglu_ffn,
    expert_forward,
    moe_layer,
    moe_round,
    build_worklist,
    tail_skip_keep,
)
