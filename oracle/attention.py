"""fp64 reference attention over a paged KV cache (test infrastructure only).

Plain definition, no blocking beyond what the method states:

* gather: a sequence's logical position j lives in physical block
  ``block_table[j // block_size]`` at offset ``j % block_size``
  ("vLLM and PagedAttention", §2, the block-table figure and the kernel sketch's
  ``key_cache``/``value_cache`` layout ``[num_blocks, block_size, heads, d_head]``;
  "vLLM — PagedAttention and Continuous Batching", §2.2, logical view over
  scattered physical blocks);
* attention for one decode token: ``softmax(scale * q . K^T) . V`` over the
  gathered K/V, computed in float64 with the max subtracted before ``exp``;
* grouped-query heads: q head ``h`` reads KV head ``h // (Hq // Hkv)``
  (consecutive q heads share a KV head; the pages do not fix this, and this is
  the reading the tests pin by equivalence with repeated-KV multi-head attention).

Storage conventions shared with the inputs (not with the GPU code):
``uint16`` arrays hold bfloat16 bit patterns, ``float32`` arrays hold fp32 values.
"""

import numpy as np


def widen(x):
    """Exact widening of stored values to float64.

    A bfloat16 value is the top 16 bits of a float32, so shifting the stored
    pattern left by 16 and reinterpreting gives the exact float32, which float64
    holds exactly.  float32/float64 inputs widen directly.
    """
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def gather_kv(key_cache, value_cache, table_row, ctx, block_size=16):
    """Logical K and V of one sequence, shape ``[ctx, num_kv_heads, head_dim]``, float64.

    Position j is read from physical block ``table_row[j // block_size]`` at slot
    ``j % block_size`` ("vLLM and PagedAttention", §2 block-table figure; the pages'
    cache layout ``[num_blocks, block_size, heads, d_head]``).  Entries of the
    table past ``ceil(ctx / block_size)`` and slots past ``ctx`` are never read.
    """
    j = np.arange(int(ctx))
    phys = np.asarray(table_row)[j // block_size].astype(np.int64)
    off = j % block_size
    return widen(key_cache[phys, off]), widen(value_cache[phys, off])


def _softmax_weighted_sum(x, V):
    """``sum_j softmax(x)_j * V[j]`` in float64 (x: [n], V: [n, D])."""
    m = np.max(x)
    w = np.exp(x - m)
    return (w @ V) / np.sum(w)


def decode_attention(q, key_cache, value_cache, block_tables, context_lens, scale,
                     block_size=16):
    """One decode token per sequence: ``out[s, h] = softmax(scale q[s,h] . K_s^T) . V_s``.

    Follows "vLLM and PagedAttention", §2 "Reworking the Attention Computation"
    (attention over K/V reached through the block table) with the exact softmax
    written out.  ``scale`` is taken as the float32 value the GPU receives,
    widened to float64.  A sequence with ``context_len == 0`` has an all-zero
    output (the pages are silent; zero is the empty-sum reading).

    Shapes: q ``[S, Hq, D]``; caches ``[NB, block_size, Hkv, D]``;
    block_tables ``[S, MB]``; context_lens ``[S]``.  Returns float64 ``[S, Hq, D]``.
    """
    qf = widen(q)
    S, Hq, D = qf.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        n = int(context_lens[s])
        if n == 0:
            continue
        K, V = gather_kv(key_cache, value_cache, block_tables[s], n, block_size)
        for h in range(Hq):
            g = h // G
            x = scale64 * (K[:, g, :] @ qf[s, h])
            out[s, h] = _softmax_weighted_sum(x, V[:, g, :])
    return out


def causal_chunk_attention(q, key_cache, value_cache, block_tables, context_lens,
                           query_start_loc, scale, block_size=16):
    """Variable-length causal attention over the paged cache (chunked prefill + decode).

    Sequence ``s`` owns query rows ``query_start_loc[s] .. query_start_loc[s+1]-1``;
    with ``qlen`` rows and ``ctx = context_lens[s]`` keys (the chunk's own tokens
    included, written before attention), row ``r`` sits at absolute position
    ``ctx - qlen + r`` and attends to keys ``0 .. ctx - qlen + r`` inclusive.  A decode
    sequence is the case ``qlen == 1``.  Chunked prefill splits a long prompt into
    pieces batched with decode ("How vLLM Works?", section 04; "vLLM and
    PagedAttention", key engineering optimizations); causality is the usual
    autoregressive mask.  Returns float64 ``[T, Hq, D]``.
    """
    qf = widen(q)
    T, Hq, D = qf.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    S = len(context_lens)
    for s in range(S):
        r0, r1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        qlen, n = r1 - r0, int(context_lens[s])
        if qlen == 0 or n == 0:
            continue
        if qlen > n:
            raise ValueError("a sequence has more query rows than context tokens")
        K, V = gather_kv(key_cache, value_cache, block_tables[s], n, block_size)
        for r in range(qlen):
            last = n - qlen + r          # inclusive
            for h in range(Hq):
                g = h // G
                x = scale64 * (K[: last + 1, g, :] @ qf[r0 + r, h])
                out[r0 + r, h] = _softmax_weighted_sum(x, V[: last + 1, g, :])
    return out


def split_decode_partials(x, V, partition_size):
    """Per-partition softmax statistics of one row of scores (split-context attention).

    The pages say each block's attention is computed separately and then
    accumulated ("vLLM and PagedAttention", §2 "Reworking the Attention
    Computation").  For positions split into consecutive partitions of
    ``partition_size``, partition ``p`` yields ``m_p = max x``, ``l_p = sum exp(x - m_p)``
    and ``o_p = sum exp(x - m_p) V / l_p``.  x: [n] float64, V: [n, D] float64.
    Returns (m [P], l [P], o [P, D]).
    """
    n = len(x)
    P = -(-n // partition_size)
    m = np.empty(P)
    l = np.empty(P)
    o = np.empty((P, V.shape[1]))
    for p in range(P):
        xs = x[p * partition_size:(p + 1) * partition_size]
        vs = V[p * partition_size:(p + 1) * partition_size]
        m[p] = np.max(xs)
        w = np.exp(xs - m[p])
        l[p] = np.sum(w)
        o[p] = (w @ vs) / l[p]
    return m, l, o


def merge_partials(m, l, o):
    """Log-sum-exp merge of partial softmax results (natural-log domain).

    ``M = max_p m_p``, ``w_p = l_p exp(m_p - M)``, ``out = sum_p w_p o_p / sum_p w_p``:
    the exact algebra of accumulating separately computed pieces of one softmax
    ("vLLM and PagedAttention", §2 "Reworking the Attention Computation").
    An empty partial (``m_p = -inf`` or ``l_p = 0``) has weight 0; if every partial
    is empty the result is zero.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    live = np.isfinite(m) & (l > 0)
    if not np.any(live):
        return np.zeros(o.shape[-1])
    M = np.max(m[live])
    w = np.where(live, l * np.exp(np.where(live, m, M) - M), 0.0)
    acc = np.zeros(o.shape[-1])
    for p in range(len(m)):
        if live[p]:
            acc += w[p] * o[p]
    return acc / np.sum(w)
