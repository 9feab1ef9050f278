"""MI355X-native paged KV-cache attention: a thin binding over ``libpagedkv.so``.

The hot path (slot write, copy-on-write block copy, split-context decode
attention, chunked-prefill attention, log-sum-exp merge, and the block copies
that swap preempted sequences to a pinned host pool and back) runs in hand-written HIP kernels for gfx950 behind
the C ABI declared in ``include/pagedkv.h``; the block allocator is C++ in the
same library.  This package only marshals arguments.  Importing it loads the
library and raises if it has not been built.
"""

from ._lib import (  # noqa: F401
    BLOCK_SIZE, PARTITION_TOKENS, PKV_BF16, PKV_F32, LIB_PATH, PagedKVError, check, lib,
)
from .ops import (  # noqa: F401
    pkv_write,
    pkv_attention_decode,
    pkv_attention_decode_plan,
    pkv_attention_decode_plan_upload,
    pkv_attention_decode_partitions,
    pkv_attention_decode_merge,
    pkv_attention_decode_append,
    pkv_attention_decode_partitions_append,
    pkv_decode_workspace_bytes,
    decode_workspace,
    pkv_attention_varlen,
    pkv_attention_varlen_plan_upload,
    pkv_attention_varlen_partitions,
    pkv_attention_varlen_plan,
    pkv_attention_varlen_decode_partitions,
    pkv_attention_varlen_prefill_tiles,
    pkv_attention_varlen_merge,
    pkv_varlen_workspace_bytes,
    varlen_workspace,
    pkv_lse_merge,
    pkv_copy_blocks,
    pkv_swap_blocks,
    DecodeGraph,
    pkv_check_tables,
    pkv_check_slots,
)
from .allocator import BlockAllocator  # noqa: F401

lib()  # fail loudly at import when the HIP library is missing
