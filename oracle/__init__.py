"""CPU oracle of the explicit-head_dim GQA attention layer (forward).

TEST INFRASTRUCTURE: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library.
"""
from .gqa_oracle import (  # noqa: F401
    ConfigError, Resolved, resolve_config, weight_shapes,
    attention_param_count, macs_per_token, project, split_heads,
    rms_norm_heads, rope_inv_freq, apply_rope, grouped_attention,
    merge_heads, qkv_normrope, layer_forward, layer_forward_rows,
)
