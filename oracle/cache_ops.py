"""Reference cache writes (test infrastructure only): slot scatter and block copy.

Both are bit copies; the result is unique, so the GPU must match these
byte for byte over the whole pool.
"""

import numpy as np


def write_kv(key_cache, value_cache, k, v, slot_mapping, block_size=16):
    """Store each new token's K and V into its slot; returns new (key_cache, value_cache).

    Token ``i`` with slot ``s = slot_mapping[i]`` goes to physical block
    ``s // block_size`` at offset ``s % block_size``, one ``[num_kv_heads, head_dim]``
    row.  The servers keep each token's keys and values in GPU memory and reuse them
    on later steps ("How vLLM Works?", section 01), in the block layout of
    "vLLM and PagedAttention", §2 (kernel sketch cache layout).  Slots outside
    ``[0, num_blocks * block_size)`` are skipped (negative = padding token).
    Inputs are not modified.  k, v: ``[T, Hkv, D]`` in the caches' storage dtype.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    nslots = kc.shape[0] * block_size
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= nslots:
            continue
        kc[s // block_size, s % block_size] = k[i]
        vc[s // block_size, s % block_size] = v[i]
    return kc, vc


def copy_blocks(key_cache, value_cache, pairs):
    """Copy-on-write block copies: for each ``(src, dst)``, block ``dst`` := block ``src``.

    Shared prefix blocks are copied before a sharer writes into them
    ("vLLM and PagedAttention", §2 bullet on shareable prefixes with copy-on-write;
    "vLLM — PagedAttention and Continuous Batching", §2.3).  A block is one
    contiguous ``[block_size, Hkv, D]`` slab in the pages' layout.  Pairs are
    applied in order; a destination that is also a later source is a caller error
    (the GPU copies all pairs concurrently).  Returns new arrays.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        kc[dst] = key_cache[src]
        vc[dst] = value_cache[src]
    return kc, vc


def swap_blocks(dst_key, dst_value, src_key, src_value, pairs):
    """Block copies between two pools of the same block shape: for each
    ``(src, dst)``, block ``dst`` of the destination := block ``src`` of the source.

    Swapping a preempted request's KV out to CPU memory and back ("vLLM and
    PagedAttention", §3 continuous batching, on preemption) moves whole
    blocks between the device pool and a host pool; each block is one contiguous
    ``[block_size, Hkv, D]`` slab in both.  Pairs whose ids fall outside either
    pool are skipped.  Returns new destination arrays.
    """
    kd = np.array(dst_key, copy=True)
    vd = np.array(dst_value, copy=True)
    ns, nd = src_key.shape[0], dst_key.shape[0]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        if 0 <= src < ns and 0 <= dst < nd:
            kd[dst] = src_key[src]
            vd[dst] = src_value[src]
    return kd, vd
