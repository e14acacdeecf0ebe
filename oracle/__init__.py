"""CPU oracle of the block-FP8 routed MoE layer — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. The HIP library and its Python binding never do.
"""
from .moe_oracle import (  # noqa: F401
    TIE_BAND,
    act_scale_exponent,
    dequantise,
    dequantise_activations,
    e4m3fn_decode,
    e4m3fn_round,
    expert_matrices,
    gate_weights,
    h_admissible_deviation,
    h_band_width,
    moe_layer,
    permutation,
    quantise_activations,
    router_logits,
    select_topk,
    silu,
    softmax,
    swiglu_expert,
    tie_flags,
)
