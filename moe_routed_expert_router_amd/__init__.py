"""Routed-expert layer with a cold-expert gather, for AMD Instinct MI355X.

The computation lives in libmoe.so (hand-written HIP for gfx950 behind the C
ABI of include/moe.h); this package only loads it and marshals arguments.
Build it with ``python moe_routed_expert_router_amd/build.py``.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MoeError, MoeResidency, MoeShape, lib, residency, shape,
    MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED_SHAPE, MOE_ERR_MISALIGNED,
    MOE_ERR_NOT_DEVICE_ACCESSIBLE, MOE_ERR_BAD_RESIDENCY, MOE_ERR_WORKSPACE_TOO_SMALL,
    MOE_ERR_HIP, MOE_OUT_F32, MOE_OUT_BF16,
    moe_status_string, moe_last_error, moe_shape_check, moe_expert_bytes, moe_workspace_bytes,
    moe_residency_check, moe_host_alloc, moe_host_free, moe_route, moe_pick_set,
    moe_gather_cold, moe_expert_ffn, moe_layer_forward,
    MOE_MAX_SWAPS, moe_count_picks, moe_residency_plan, moe_residency_swap, moe_fingerprint,
    moe_profile_enable, moe_profile_reset, moe_profile_read, moe_probe_read, moe_probe_mfma,
    MOE_NOALLOC_WS_BYTES, moe_layer_forward_noalloc,
)
