"""CPU oracle for the W4A16 MoE expert layer.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path
(``w4a16_int4_grouped_amd``) never imports it and shares no code with it.
"""
from .moe_oracle import (  # noqa: F401
    bf16_round, bf16_to_f64, unpack_nibbles, dequant, align, permute,
    contiguous_layout, silu, expert_ffn, combine, moe_indexed, moe_contiguous, moe_masked,
    compare,
)
