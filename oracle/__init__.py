"""CPU oracle (test infrastructure only; see ``oracle.prefill``)."""
from .prefill import (  # noqa: F401
    KVCacheModel,
    apply_rope,
    attention,
    block_mass,
    compact,
    kept_cache_positions,
    normalise_scores,
    num_blocks,
    p_fixed_point,
    rope_frequencies,
    run_call,
    score_fixed_point,
    softmax_probs,
    topp_select,
    visible,
)
from .layers import feature_map, later_layer_flops, linear, linear_attention, silu, swiglu  # noqa: F401
