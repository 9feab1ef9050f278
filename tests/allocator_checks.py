"""Allocator invariants and worked examples, usable against any allocator object.

The object must offer: add_seq, fork, append(seq, n) -> (slots, cow_pairs),
free_seq, block_table(seq), seq_len(seq), num_free(), refcount(block), and the
attributes num_blocks / block_size.  Used for the oracle's model and for the
product allocator behind the C ABI.
"""

import collections
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def check_invariants(alloc, live):
    """Structural invariants over the live sequences ``live`` (list of ids)."""
    bs = alloc.block_size
    counts = collections.Counter()
    for sid in live:
        tbl = alloc.block_table(sid)
        n = alloc.seq_len(sid)
        # each sequence holds exactly ceil(n / bs) blocks: only the last can be partial
        assert len(tbl) == -(-n // bs), (sid, n, len(tbl))
        assert len(set(tbl)) == len(tbl), "a block appears twice in one table"
        counts.update(tbl)
    # a block's count equals the number of table entries holding it
    for b in range(alloc.num_blocks):
        assert alloc.refcount(b) == counts.get(b, 0), (b, alloc.refcount(b), counts.get(b, 0))
    used = sum(1 for b in range(alloc.num_blocks) if alloc.refcount(b) > 0)
    assert used + alloc.num_free() == alloc.num_blocks


def check_hundred_tokens(alloc):
    g = golden()["hundredth_token_block"]
    alloc.add_seq(1)
    slots, pairs = alloc.append(1, g["tokens"])
    tbl = alloc.block_table(1)
    assert len(tbl) == g["blocks_held"]
    assert slots[g["tokens"] - 1] // g["block_size"] == tbl[g["block_of_last_token_1based"] - 1]
    assert pairs == []
    alloc.free_seq(1)


def check_paged_waste_under_one_block(alloc, rng):
    """Reserved-minus-used is below one block per sequence (vs the pages' static examples)."""
    g = golden()
    cases = [g["static_slot_4096_used_50"]["used"], *g["static_three_requests_2048"]["used"],
             g["static_slot_8192_used_500"]["used"]]
    for sid, n in enumerate(cases, start=10):
        alloc.add_seq(sid)
        # grow in random increments, as decode + prefill chunks would
        left = n
        while left:
            k = int(min(left, rng.integers(1, 40)))
            alloc.append(sid, k)
            left -= k
        reserved = len(alloc.block_table(sid)) * alloc.block_size
        assert 0 <= reserved - n < alloc.block_size
    # the static numbers themselves
    s = g["static_three_requests_2048"]
    assert [s["reserved_each"] - u for u in s["used"]] == s["wasted"]
    st = g["static_slot_4096_used_50"]
    assert st["reserved"] - st["used"] == st["wasted"]
    s8 = g["static_slot_8192_used_500"]
    assert round(100 * (1 - s8["used"] / s8["reserved"])) == s8["printed_unused_pct"]
    for sid in range(10, 10 + len(cases)):
        alloc.free_seq(sid)


def check_fork_and_cow(alloc):
    """Fork shares blocks; the first append into a shared partial block copies it once."""
    bs = alloc.block_size
    alloc.add_seq(100)
    alloc.append(100, 3 * bs + 5)                  # 4 blocks, last one partial (5 tokens)
    parent = alloc.block_table(100)
    alloc.fork(100, 101)
    alloc.fork(100, 102)
    for b in parent:
        assert alloc.refcount(b) == 3
    slots, pairs = alloc.append(101, 1)
    assert len(pairs) == 1 and pairs[0][0] == parent[-1]
    dst = pairs[0][1]
    assert alloc.block_table(101)[:-1] == parent[:-1] and alloc.block_table(101)[-1] == dst
    assert slots == [dst * bs + 5]
    assert alloc.refcount(parent[-1]) == 2 and alloc.refcount(dst) == 1
    # a second append to the now-private block copies nothing
    _, pairs = alloc.append(101, 2)
    assert pairs == []
    # the other child copies too; then the parent is the last sharer and writes in place
    _, pairs = alloc.append(102, 1)
    assert len(pairs) == 1
    slots, pairs = alloc.append(100, 1)
    assert pairs == [] and slots == [parent[-1] * bs + 5]
    # full shared blocks are never copied: a fork at a block boundary appends into a new block
    alloc.add_seq(103)
    alloc.append(103, 2 * bs)
    alloc.fork(103, 104)
    slots, pairs = alloc.append(104, 1)
    assert pairs == [] and alloc.block_table(104)[:2] == alloc.block_table(103)
    check_invariants(alloc, [100, 101, 102, 103, 104])
    for sid in (100, 101, 102, 103, 104):
        alloc.free_seq(sid)


def check_enomem_atomic(alloc, exc_type):
    """Running out of blocks changes nothing: tables, lengths, counts and the free count."""
    bs = alloc.block_size
    nb = alloc.num_blocks
    alloc.add_seq(200)
    alloc.append(200, (nb - 1) * bs - 3)          # leaves one free block, last block partial
    alloc.fork(200, 201)
    before = (alloc.block_table(200), alloc.block_table(201), alloc.num_free(),
              [alloc.refcount(b) for b in range(nb)], alloc.seq_len(201))
    try:
        alloc.append(201, 3 + bs + 1)             # needs the CoW block + 2 more: too many
        raise AssertionError("expected out-of-memory")
    except exc_type:
        pass
    after = (alloc.block_table(200), alloc.block_table(201), alloc.num_free(),
             [alloc.refcount(b) for b in range(nb)], alloc.seq_len(201))
    assert before == after
    # the same request that fits succeeds (CoW uses the last free block)
    _, pairs = alloc.append(201, 1)
    assert len(pairs) == 1 and alloc.num_free() == 0
    # recompute-style preemption: free and re-add, then appends work again
    alloc.free_seq(201)
    alloc.add_seq(201)
    alloc.append(201, 1)
    alloc.free_seq(201)
    alloc.free_seq(200)
    assert alloc.num_free() == nb


def random_ops(alloc, rng, steps, exc_type):
    """Seeded random add / fork / append / free sequence, checking invariants throughout."""
    live = []
    next_id = 1000
    for _ in range(steps):
        op = rng.integers(0, 10)
        if op == 0 or not live:
            alloc.add_seq(next_id)
            live.append(next_id)
            next_id += 1
        elif op == 1:
            p = live[rng.integers(len(live))]
            alloc.fork(p, next_id)
            live.append(next_id)
            next_id += 1
        elif op == 2 and len(live) > 1:
            sid = live.pop(rng.integers(len(live)))
            alloc.free_seq(sid)
        else:
            sid = live[rng.integers(len(live))]
            n = int(rng.integers(0, 40))
            before_tbl = alloc.block_table(sid)
            before_len = alloc.seq_len(sid)
            try:
                slots, pairs = alloc.append(sid, n)
            except exc_type:
                assert alloc.block_table(sid) == before_tbl and alloc.seq_len(sid) == before_len
                continue
            tbl = alloc.block_table(sid)
            bs = alloc.block_size
            assert slots == [tbl[p // bs] * bs + p % bs for p in range(before_len, before_len + n)]
            assert len(pairs) <= 1
            for src, dst in pairs:
                assert before_len % bs != 0 and before_tbl[-1] == src and tbl[len(before_tbl) - 1] == dst
        check_invariants(alloc, live)
    for sid in live:
        alloc.free_seq(sid)
    assert alloc.num_free() == alloc.num_blocks
