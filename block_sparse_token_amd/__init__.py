"""MI355X-native UniPrefill-style prefill operator.

The compute path lives in ``libuniprefill.so`` (HIP kernels for gfx950 behind
the C ABI of ``include/uniprefill.h``); ``binding`` wraps its entry points
for torch tensors and ``step`` strings one operator call together.
Importing this package does not touch the GPU.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    UP_ACT_NONE,
    UP_ACT_SWIGLU,
    UP_SCOPE_PROMPT,
    UP_SCOPE_SEGMENT,
    Batch,
    UniprefillError,
    interleave_gate_up,
    lib,
    up_attn_workspace_bytes,
    up_block_offsets,
    up_block_scores,
    up_check_batch,
    up_compact,
    up_compact_workspace_bytes,
    up_kept_cache_slots,
    up_linear_attn_bf16,
    up_linear_attn_workspace_bytes,
    up_linear_bf16,
    up_prefill_attn,
    up_topp_select,
    up_version,
)
