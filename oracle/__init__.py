"""CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 NumPy statement of
what the paged-attention hot path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``paged_kv_cache_360_amd``) never imports, calls or
links anything here, and nothing here imports the product path: the two share no
code.  The only module both sides use is ``workloads`` (seeded random inputs,
none of the method's arithmetic).

Sources (web pages, cited by title and section):

* "vLLM — PagedAttention and Continuous Batching" (s-samarth.github.io), §2
  PagedAttention (2.2 the solution, 2.3 results, 2.4 why it needs a custom kernel).
* "vLLM and PagedAttention" (ai.zenoagi.com case study), §2 PagedAttention:
  the block-table figure, the bullet list on on-demand allocation / one pool /
  copy-on-write sharing, "Reworking the Attention Computation" and the
  simplified kernel sketch (cache layout and block-table argument).
* "How vLLM Works?: PagedAttention, Continuous Batching and the KV Cache"
  (peterindia.net), section 03 PagedAttention.

Modules:

* ``attention``  gather through the block table, fp64 softmax attention (decode
  and causal chunk), log-sum-exp merge of partial softmaxes.
* ``cache_ops``  the slot scatter write, the copy-on-write block copy and the
  block copy between the device pool and a host pool (swapping).
* ``allocator``  a Python model of the block allocator (refcounts, fork, CoW) and
  of its automatic prefix caching.

Every function here is pinned by tests under ``tests/`` against something other
than itself (closed forms, a library attention routine on contiguous K/V,
brute-force permutation invariance, worked numbers printed on the pages).
"""

from .attention import (  # noqa: F401
    widen,
    gather_kv,
    decode_attention,
    causal_chunk_attention,
    merge_partials,
    split_decode_partials,
)
from .cache_ops import write_kv, copy_blocks, swap_blocks  # noqa: F401
from .allocator import BlockAllocatorModel, PrefixCachingAllocatorModel, slot_for_position  # noqa: F401
