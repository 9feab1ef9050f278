"""Seeded synthetic inputs for the paged KV-cache hot path.

This is the one module that both the product path's tests/bench and the CPU
oracle consume.  It holds random draws and shapes only -- no attention, no
softmax, no scatter, no allocator logic.  Block tables are random distinct
physical ids (the pages' "scattered in one pool" placement); which slot a new
token goes to is decided by an allocator (the oracle's model in tests, the
product's allocator in the bench), not here.
"""

from .gen import (  # noqa: F401
    BLOCK_SIZE,
    WorkloadSpec,
    SPECS,
    f32_to_bf16_bits,
    normal_values,
    normal_values_parallel,
    draw_context_lens,
    pool_blocks_for,
    random_block_tables,
    make_decode_inputs,
)
