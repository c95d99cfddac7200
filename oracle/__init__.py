"""Float64 CPU oracle for scaled dot-product attention (test infrastructure only).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  It is independent of the HIP library: it imports nothing
from it and shares none of its code.
"""
from .sdpa_oracle import (  # noqa: F401
    LEARNABLE, OFF_BY_ONE, SOFTMAX_TYPES, VANILLA, attention, attention_group, attention_keys,
    attention_dropout, attention_packed, attention_rows, dropout_keep, dropout_threshold,
    packed_visible_mask, philox4x32_10, visible_rows,
    kv_head, sink_logit, visible_mask, visible_pairs,
)
