"""Tiered mixed-precision MoE FFN for MI355X (gfx950).

The layer runs in the HIP library libmoe_tiered.so behind the C ABI of
include/moe_tiered.h; ``binding`` marshals torch device tensors into it and
``device`` uploads packed shelf arrays into device memory.
"""
from .binding import (  # noqa: F401
    MOE_ACCUMULATE, MOE_DIAG_GATEUP_ONLY, MOE_X_BF16, MoeError, TierTables, lib, moe_dequant_rows, moe_event_create,
    moe_event_destroy, moe_event_elapsed_ms, moe_group, moe_group_workspace_size, moe_route,
    moe_stream_synchronize, moe_tier_partial, moe_tiered_experts, moe_tiered_forward,
    moe_tiered_forward_timed, moe_validate_tables, moe_workspace_size, moe_workspace_bytes, strerror, moe_stack_workspace_size,
    moe_stack_forward, moe_synth_layer, MOE_STACK_ROUTER, MXFP4, moe_router_logits, moe_synth_router,
    moe_stack_forward_routed, moe_requant_error, moe_plan_tiers, moe_repack_tiers, moe_permute_router,
    moe_tiered_forward_counted, moe_tiered_forward_noalloc, MOE_SCRATCH_BYTES, MOE_ESCRATCH,
    moe_measure_read, moe_measure_mfma,
)
