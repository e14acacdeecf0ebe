"""block_fp8_routed_amd — a Mixture-of-Experts FFN layer with block-FP8 (E4M3)
expert weights, as hand-written HIP kernels for AMD Instinct MI355X (gfx950)
behind the C ABI of libmoe_fp8.so (include/moe_fp8.h).

The Python names mirror the C entry points; they only marshal torch tensors
(device memory, the current stream) into the library.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    MOE_BF16,
    MOE_ERR_HIP,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_EV_COUNT,
    MOE_EV_DOWN,
    MOE_EV_END,
    MOE_EV_GATE_UP,
    MOE_EV_PERMUTED,
    MOE_EV_ROUTED,
    MOE_EV_START,
    MOE_F32,
    MOE_OK,
    Bank,
    MoeConfig,
    MoeError,
    MoeExpertBank,
    MoePhaseEvents,
    load,
    make_config,
    make_workspace,
    moe_dequant_e4m3,
    moe_quantize_act_e4m3,
    moe_forward,
    moe_permute,
    moe_route,
    status_string,
    version,
    workspace_bytes,
)
