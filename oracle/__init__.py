"""CPU oracle for paged decode attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path (the HIP library and its binding) never
does, and shares no code with it.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    block_and_slot,
    bf16_ulp,
    gather_sequence,
    kv_append,
    kv_head_of,
    lse_combine,
    num_partitions,
    paged_attention,
    partition_attention,
    round_to_bf16,
    softmax_attention_row,
    visible_tokens,
)
from .rope import kv_append_rope, rope_angles, rope_rotate, token_positions  # noqa: F401,E402
