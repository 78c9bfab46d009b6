"""CPU fp64 oracle for Flash-LoRA-Attention and the LR precompute.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the package entry point's
smoke check and by the benchmark's CPU-baseline leg, never by the library itself.
"""

from .flash_lora_oracle import (  # noqa: F401
    attention_batch,
    attention_request,
    full_value_cache,
    kv_head_of,
    lr_precompute,
    query_positions,
    softmax_scale,
    visible,
)
