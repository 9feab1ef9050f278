"""Inputs whose correct attention output moves by a unit-scale amount when one
16-token block is dropped, counted twice or read from the wrong place, or when
partition partials are combined with wrong weights.

Why these exist: with N(0,1) queries the softmax weights are spread over the
whole context, so a wrong block moves the output by about 16/ctx of its size,
far inside the bf16 bars.  Here every output row (one sequence or chunk row,
one q head) has a *target* token t and a query pointing at t's key,

    q = alpha * K_t / |K_t|,

with alpha tuned (in float64, before the query is rounded to the storage
dtype) so that t carries about half of the softmax mass.  The output is then
about 0.5 * V_t + 0.5 * (the rest): losing t's block moves it by ~0.5 * |V_t|,
reading t twice moves it by ~0.17 * |V_t|, both far above the 2e-2 bars.
Targets are spread so that every logical block of a context is some row's
target for every KV head (where the row count allows), at varying offsets
inside the block, including the last token of a context and, for chunk rows,
the row's own position (the causal edge).

The tied-key inputs copy one key row i onto two more positions j and k that
share another 512-token partition, and saturate the query on it: the three
positions get exactly the same score and all but a negligible part of the
mass, so the output is (V_i + V_j + V_k) / 3 at unit scale.  The two
partitions' partial sums differ (1 against 2), so this checks both the maxima
and the sums the log-sum-exp merge weighs partitions by.

Each block, each partition and the computation it implies is stated on the
pages as accumulating separately computed per-block attention ("vLLM and
PagedAttention", §2 "Reworking the Attention Computation").  These builders
only shape inputs; expected values come from the oracle.  CPU code, shared by
the GPU tests and the CPU tests that show each check flags dropped and
duplicated blocks and wrong merge weights.
"""

import math

import numpy as np

import oracle
from workloads import BLOCK_SIZE, f32_to_bf16_bits, normal_values

PEAK_MASS = 0.5          # softmax mass the tuned query puts on its target token


def to_dtype(x, dtype):
    x = np.asarray(x, np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def tune_alpha(c, t_idx, mass=PEAK_MASS, iters=6):
    """Per column k, alpha with softmax(alpha * c[:, k])[t_idx[k]] == mass.

    c: [n, m] float64 projections (-inf where a position is not visible);
    t_idx: [m].  Newton's method on f(a) = a c_t - logsumexp(a c) - log(mass),
    which is concave and increasing in a while c_t is the column's largest
    entry, so iterates started at 0 (where f < 0) rise monotonically to the
    root (six steps reach it to ~1e-12 on 8192 N(0,1) keys; the mass only has
    to be near its target).  Columns with one visible position get alpha 1."""
    c = np.asarray(c, np.float64)
    m = c.shape[1]
    ct = c[t_idx, np.arange(m)]
    live = np.isfinite(c)
    nvis = live.sum(axis=0)
    a = np.zeros(m)
    cz = np.where(live, c, 0.0)
    for _ in range(iters):
        x = np.where(live, a[None, :] * cz, -np.inf)
        mx = x.max(axis=0)
        w = np.exp(x - mx[None, :])
        z = w.sum(axis=0)
        lse = mx + np.log(z)
        f = a * ct - lse - math.log(mass)
        fp = ct - (w * cz).sum(axis=0) / z
        a = a - f / np.maximum(fp, 1e-6)
    return np.where(nvis > 1, a, 1.0)


def _peaked_queries(K, heads, scale, targets, nvis, mass):
    """Queries [m, D] (float64, before rounding): column k reads KV head
    heads[k] of the logical keys K [n, Hkv, D] (float64), points at key
    targets[k] and sees positions < nvis[k].  Returns (q rows, masses reached
    in float64)."""
    m = len(targets)
    kt = K[targets, heads]                               # [m, D]
    unit = kt / np.linalg.norm(kt, axis=1, keepdims=True)
    c = np.empty((K.shape[0], m))
    for g in np.unique(heads):                           # one matrix product per KV head
        cols = np.nonzero(heads == g)[0]
        c[:, cols] = scale * (K[:, g, :] @ unit[cols].T)
    pos = np.arange(K.shape[0])[:, None]
    c = np.where(pos < nvis[None, :], c, -np.inf)
    a = tune_alpha(c, targets, mass)
    x = np.where(np.isfinite(c), a[None, :] * np.where(np.isfinite(c), c, 0.0), -np.inf)
    w = np.exp(x - x.max(axis=0)[None, :])
    reached = w[targets, np.arange(m)] / w.sum(axis=0)
    return a[:, None] * unit, reached


def _logical_keys(kc, table_row, n):
    """Keys of positions 0 .. n-1 of one sequence, float64 [n, Hkv, D]."""
    j = np.arange(n)
    return oracle.widen(kc[np.asarray(table_row)[j // BLOCK_SIZE].astype(np.int64), j % BLOCK_SIZE])


def decode_targets(ctxs, Hq, Hkv, last_token_head0=False):
    """Target position of each decode row (s, h): logical block
    (s*G + h%G + g*S*G) mod ceil(ctx_s/16) (g = h // G; with S*G >= the block
    count every block is a target of every KV head, and with fewer rows the KV
    heads take consecutive runs of blocks), at offset (5s + 3h + g) % 16 clamped
    to the context, except that a row whose block is the context's last targets
    the last token.  last_token_head0: head 0 of every sequence targets its last
    token (the new token of a decode step)."""
    ctxs = np.asarray(ctxs, np.int64)
    S, G = len(ctxs), Hq // Hkv
    targets = np.zeros((S, Hq), np.int64)
    for s in range(S):
        n = int(ctxs[s])
        nblk = -(-n // BLOCK_SIZE)
        for h in range(Hq):
            g, j = divmod(h, G)
            b = (s * G + j + g * S * G) % nblk
            off = (5 * s + 3 * h + g) % BLOCK_SIZE
            targets[s, h] = n - 1 if b == nblk - 1 else min(n - 1, b * BLOCK_SIZE + off)
        if last_token_head0:
            targets[s, 0] = n - 1
    return targets


def peaked_decode_queries(kc, tables, ctxs, Hq, targets, dtype, mass=PEAK_MASS):
    """Queries [S, Hq, D] in the storage dtype, row (s, h) pointing at key
    targets[s, h] of sequence s (keys gathered from kc through tables), with the
    scale tuned to give it `mass`.  Returns (q, masses reached before rounding)."""
    S = len(ctxs)
    Hkv, D = kc.shape[2], kc.shape[3]
    scale = 1.0 / math.sqrt(D)
    q64 = np.zeros((S, Hq, D))
    reached = np.zeros((S, Hq))
    heads = np.arange(Hq) // (Hq // Hkv)
    for s in range(S):
        n = int(ctxs[s])
        K = _logical_keys(kc, tables[s], n)
        q64[s], reached[s] = _peaked_queries(K, heads, float(np.float32(scale)), targets[s], np.full(Hq, n), mass)
    return to_dtype(q64, dtype), reached


def scattered_tables(rng, ctxs, num_blocks, shared):
    """Block tables [S, max blocks + 1] (-1 past each context).  shared: every
    sequence's table is its own permutation drawn from the whole pool (blocks
    are read by several sequences); otherwise the sequences split one
    permutation of the pool (private blocks)."""
    ctxs = np.asarray(ctxs, np.int64)
    nblks = -(-ctxs // BLOCK_SIZE)
    tables = np.full((len(ctxs), int(nblks.max()) + 1), -1, np.int32)
    if shared:
        for s, n in enumerate(nblks):
            tables[s, :n] = rng.permutation(num_blocks)[:n]
    else:
        perm = rng.permutation(num_blocks).astype(np.int32)
        off = 0
        for s, n in enumerate(nblks):
            tables[s, :n] = perm[off:off + n]
            off += int(n)
    return tables


def peaked_decode_case(seed, S, Hq, Hkv, D, ctx, dtype="bf16", mass=PEAK_MASS, spare_blocks=3):
    """A decode batch of S sequences, all with context `ctx`, over one shared pool
    of ceil(ctx/16) + spare blocks; each sequence's table is its own seeded
    permutation of the pool; targets from ``decode_targets``.

    Returns a dict with the oracle's input names plus "targets" [S, Hq] and
    "mass" [S, Hq] (the target's softmax mass with the unrounded query)."""
    rng = np.random.default_rng(seed)
    nblk = -(-ctx // BLOCK_SIZE)
    nb = nblk + spare_blocks
    kc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    vc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    ctxs = np.full(S, ctx, np.int32)
    tables = scattered_tables(rng, ctxs, nb, shared=True)
    targets = decode_targets(ctxs, Hq, Hkv)
    q, reached = peaked_decode_queries(kc, tables, ctxs, Hq, targets, dtype, mass)
    return {"dtype": dtype, "key_cache": kc, "value_cache": vc, "block_tables": tables,
            "context_lens": ctxs, "num_blocks": nb, "scale": np.float32(1.0 / math.sqrt(D)),
            "q": q, "targets": targets, "mass": reached}


def peaked_chunk_case(seed, Hq, Hkv, D, qlens, ctxs, dtype="bf16", mass=PEAK_MASS, spare_blocks=5,
                      q_of=None):
    """Variable-length rows (chunks and decode rows) over scattered blocks, every
    row peaked.  Sequence s has qlens[s] rows at the end of a ctxs[s]-token
    context; row r sees keys 0 .. ctx - qlen + r.  Head h of row r targets: the
    row's own position (the causal edge) for h % G == 0 (with G == 1: on even
    rows); otherwise visible block (r*G + h%G + 11g) mod the row's block count,
    so that over a chunk's rows the blocks of its context are covered for every
    KV head, at offset (3r + h) % 16 clamped to the row's keys.  Rows that see no
    key keep q = 0.

    q_of: optional set of sequence ids whose rows are peaked (others get N(0,1)
    queries).  Returns the oracle's varlen input names plus "targets" [T, Hq]
    (-1 for unpeaked rows) and "mass"."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    qlens = np.asarray(qlens, np.int32)
    ctxs = np.asarray(ctxs, np.int32)
    S = len(ctxs)
    nb = int((-(-ctxs // BLOCK_SIZE)).sum()) + spare_blocks
    tables = scattered_tables(rng, ctxs, nb, shared=False)
    kc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    vc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    T = int(qlens.sum())
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    scale = np.float32(1.0 / math.sqrt(D))
    q64 = rng.standard_normal((T, Hq, D))
    targets = np.full((T, Hq), -1, np.int64)
    mass_reached = np.full((T, Hq), np.nan)
    for s in range(S):
        if q_of is not None and s not in q_of:
            continue
        n, ql = int(ctxs[s]), int(qlens[s])
        K = _logical_keys(kc, tables[s], n)
        rows = np.arange(ql)
        keys = np.maximum(0, n - ql + rows + 1)           # keys each row sees
        tg = np.zeros((ql, Hq), np.int64)
        for r in range(ql):
            nbv = -(-int(keys[r]) // BLOCK_SIZE)
            for h in range(Hq):
                g, j = divmod(h, G)
                if keys[r] == 0:
                    tg[r, h] = 0
                elif j == 0 and (G > 1 or r % 2 == 0):
                    tg[r, h] = keys[r] - 1                    # the causal edge: the row's own key
                else:
                    b = (r * G + j + 11 * g) % nbv
                    tg[r, h] = min(int(keys[r]) - 1, b * BLOCK_SIZE + (3 * r + h) % BLOCK_SIZE)
        heads = np.arange(Hq) // G
        for r0 in range(0, ql, 64):                         # bounded temporaries: 64 rows at a time
            rr = np.arange(r0, min(ql, r0 + 64))
            qg, rch = _peaked_queries(K, np.tile(heads, len(rr)), float(scale), tg[rr].reshape(-1),
                                      np.repeat(keys[rr], Hq), mass)
            qg = qg.reshape(len(rr), Hq, D)
            qg[keys[rr] == 0] = 0.0
            q64[qsl[s] + rr] = qg
            mass_reached[qsl[s] + rr] = rch.reshape(len(rr), Hq)
        tg[keys == 0] = -1
        targets[qsl[s]:qsl[s + 1]] = tg
    return {"dtype": dtype, "key_cache": kc, "value_cache": vc, "block_tables": tables,
            "context_lens": ctxs, "num_blocks": nb, "scale": scale, "qsl": qsl,
            "max_query_len": int(qlens.max()), "q": to_dtype(q64, dtype), "targets": targets,
            "mass": mass_reached}


def _tied_positions(rng, kc, tables, visible):
    """For each sequence, a position i in one 512-token partition and two
    positions j < k in a later one, all < visible[s] (k the last visible
    position for every third sequence); key row i is copied onto j and k (all
    KV heads).  Returns [S, 3] (i, j, k)."""
    S = len(visible)
    pos = np.zeros((S, 3), np.int64)
    for s in range(S):
        n = int(visible[s])
        P = -(-n // 512)
        last = P - 1 if n - 512 * (P - 1) >= 2 else P - 2   # a partition with two positions
        pi = int(rng.integers(0, last))
        pj = int(rng.integers(pi + 1, last + 1))
        lo, hi = pj * 512, min(n, pj * 512 + 512)
        j, k = sorted(rng.choice(np.arange(lo, hi), 2, replace=False).tolist())
        if s % 3 == 0:
            k = hi - 1
            j = min(j, k - 1)
        i = pi * 512 + int(rng.integers(0, 512))
        pos[s] = (i, j, k)
        src = kc[tables[s, i // BLOCK_SIZE], i % BLOCK_SIZE].copy()
        for t in (j, k):
            kc[tables[s, t // BLOCK_SIZE], t % BLOCK_SIZE] = src
    return pos


def _saturated_query(kc, tables, s, i, Hq, alpha):
    """alpha * K_i / |K_i| for every q head of sequence s (float64 [Hq, D])."""
    ki = oracle.widen(kc[tables[s, i // BLOCK_SIZE], i % BLOCK_SIZE])   # [Hkv, D]
    G = Hq // ki.shape[0]
    unit = ki / np.linalg.norm(ki, axis=1, keepdims=True)
    return alpha * np.repeat(unit, G, axis=0)


def tied_keys_decode_case(seed, Hq, Hkv, D, ctxs, dtype="bf16", alpha=100.0, spare_blocks=3):
    """Decode rows over tied keys: in each sequence (its own blocks) key row i is
    copied onto j and k in a later 512-token partition, and every head's query
    is alpha * K_i / |K_i| with alpha large, so every output row is
    (V_i + V_j + V_k) / 3 at unit scale.  The positions vary by sequence.
    Returns the oracle's input names plus "tied" [S, 3] and "row_seq"."""
    rng = np.random.default_rng(seed)
    ctxs = np.asarray(ctxs, np.int32)
    assert np.all(ctxs > 513), "tied keys in two partitions need a context over 513"
    S = len(ctxs)
    nb = int((-(-ctxs // BLOCK_SIZE)).sum()) + spare_blocks
    tables = scattered_tables(rng, ctxs, nb, shared=False)
    kc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    vc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    tied = _tied_positions(rng, kc, tables, ctxs)
    q = np.stack([_saturated_query(kc, tables, s, int(tied[s, 0]), Hq, alpha) for s in range(S)])
    return {"dtype": dtype, "key_cache": kc, "value_cache": vc, "block_tables": tables,
            "context_lens": ctxs, "num_blocks": nb, "scale": np.float32(1.0 / math.sqrt(D)),
            "q": to_dtype(q, dtype), "tied": tied, "row_seq": np.arange(S)}


def tied_keys_chunk_case(seed, Hq, Hkv, D, qlens, ctxs, dtype="bf16", alpha=100.0, spare_blocks=5):
    """Tied keys for variable-length rows: per sequence, i, j and k are visible
    to all of its rows (<= ctx - qlen), and every row's query is saturated on
    K_i.  Returns the varlen input names plus "tied" [S, 3] and "row_seq" [T]
    (the sequence of each row)."""
    rng = np.random.default_rng(seed)
    qlens = np.asarray(qlens, np.int32)
    ctxs = np.asarray(ctxs, np.int32)
    vis = ctxs - qlens + 1
    assert np.all(vis > 513), "every row must see two partitions"
    S = len(ctxs)
    nb = int((-(-ctxs // BLOCK_SIZE)).sum()) + spare_blocks
    tables = scattered_tables(rng, ctxs, nb, shared=False)
    kc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    vc = normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype)
    tied = _tied_positions(rng, kc, tables, vis)
    row_seq = np.repeat(np.arange(S), qlens)
    q = np.stack([_saturated_query(kc, tables, s, int(tied[s, 0]), Hq, alpha) for s in row_seq])
    return {"dtype": dtype, "key_cache": kc, "value_cache": vc, "block_tables": tables,
            "context_lens": ctxs, "num_blocks": nb, "scale": np.float32(1.0 / math.sqrt(D)),
            "qsl": np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32), "max_query_len": int(qlens.max()),
            "q": to_dtype(q, dtype), "tied": tied, "row_seq": row_seq}


def tied_keys_expected(inp):
    """(V_i + V_j + V_k) / 3 for every row, the closed form the tied-key inputs
    reach (float64 [rows, Hq, D])."""
    T, Hq, D = inp["q"].shape
    G = Hq // inp["key_cache"].shape[2]
    out = np.zeros((T, Hq, D))
    for r, s in enumerate(inp["row_seq"]):
        t = inp["block_tables"][s]
        v = sum(oracle.widen(inp["value_cache"][t[p // BLOCK_SIZE], p % BLOCK_SIZE]) for p in inp["tied"][s])
        out[r] = np.repeat(v / 3.0, G, axis=0)
    return out
