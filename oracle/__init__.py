"""Float64 CPU oracle (test infrastructure only; see attn_oracle's header)."""

from .attn_oracle import (  # noqa: F401
    apply_rope,
    apply_rope_interleaved,
    attention,
    attention_backward,
    attention_backward_shard,
    merge,
    attention_weights,
    causal_mask,
    kv_head_of,
    rope_angles,
    rope_frequencies,
    rotate_half,
    softmax_rows,
)
