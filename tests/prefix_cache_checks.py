"""Automatic prefix caching: the behaviour the pages fix, usable against any
allocator object with add_seq_tokens / append_tokens / append / fork / free_seq /
block_table / seq_len / refcount / num_free / num_cached (the oracle's model and
the C++ allocator behind the C ABI).

Pages: "How vLLM Works?", section 05 (a block is keyed by its tokens and the
tokens before it; only full blocks are cached; extra values such as a cache
salt isolate tenants); "vLLM and PagedAttention", section 4 (later requests with
the same system prompt reuse its KV; a cache of released blocks).
"""

import collections

BS = 16


def prompt(n, start=0):
    return list(range(start, start + n))


def check_states(alloc, live):
    """Every block is exactly one of: referenced, cached with no user, free.
    Counts equal table entries; num_free counts free and cached-unused blocks."""
    counts = collections.Counter()
    for sid in live:
        tbl = alloc.block_table(sid)
        assert len(tbl) == -(-alloc.seq_len(sid) // BS)
        assert len(set(tbl)) == len(tbl)
        counts.update(tbl)
    for b in range(alloc.num_blocks):
        assert alloc.refcount(b) == counts.get(b, 0)
    used = sum(1 for b in range(alloc.num_blocks) if alloc.refcount(b) > 0)
    assert used + alloc.num_free() == alloc.num_blocks
    assert 0 <= alloc.num_cached() <= alloc.num_free()


def check_equal_prefix_same_blocks(alloc):
    """A second request with the same prompt reuses the full blocks, not the
    partial last one, and gets slot -1 (nothing to write) for those tokens."""
    p = prompt(40)                                   # 2 full blocks + 8 tokens
    s1, c1 = alloc.add_seq_tokens(1, p)
    assert c1 == 0 and min(s1) >= 0
    s2, c2 = alloc.add_seq_tokens(2, p)
    assert c2 == 32
    assert s2[:32] == [-1] * 32 and min(s2[32:]) >= 0
    t1, t2 = alloc.block_table(1), alloc.block_table(2)
    assert t2[:2] == t1[:2] and t2[2] != t1[2]       # partial blocks are never shared
    assert [alloc.refcount(b) for b in t1] == [2, 2, 1]
    # the uncached tokens' slots follow the table
    assert s2[32:] == [t2[2] * BS + i for i in range(8)]
    check_states(alloc, [1, 2])


def check_salt_isolates(alloc):
    p = prompt(48)
    alloc.add_seq_tokens(1, p, salt=11)
    _, c = alloc.add_seq_tokens(2, p, salt=12)
    assert c == 0
    assert not set(alloc.block_table(1)) & set(alloc.block_table(2))
    _, c = alloc.add_seq_tokens(3, p, salt=11)
    assert c == 48 and alloc.block_table(3) == alloc.block_table(1)
    check_states(alloc, [1, 2, 3])


def check_key_includes_everything_before(alloc):
    """Equal tokens in block 1 after a different block 0 are a different block;
    lookup stops at the first block not found."""
    a = prompt(48)
    b = [1000] + a[1:]                               # block 0 differs in one token
    c = a[:16] + [2000] + a[17:]                     # block 1 differs
    alloc.add_seq_tokens(1, a)
    _, cb = alloc.add_seq_tokens(2, b)
    assert cb == 0
    _, cc = alloc.add_seq_tokens(3, c)
    assert cc == 16
    t1, t3 = alloc.block_table(1), alloc.block_table(3)
    assert t3[0] == t1[0] and t3[1] != t1[1] and t3[2] != t1[2]   # block 2 equal but after a miss
    check_states(alloc, [1, 2, 3])


def check_appended_blocks_are_cached(alloc):
    """A block that fills through appends (a decode or a later chunk) becomes
    cacheable; one that stays partial does not."""
    alloc.add_seq_tokens(1, prompt(10))
    alloc.append_tokens(1, prompt(6, 10))             # block 0 now full
    alloc.append_tokens(1, prompt(5, 16))             # block 1 partial
    _, c = alloc.add_seq_tokens(2, prompt(40))
    assert c == 16
    assert alloc.block_table(2)[0] == alloc.block_table(1)[0]
    check_states(alloc, [1, 2])


def check_released_blocks_reused_then_taken_over(alloc):
    """Cached blocks outlive their sequences; a hit revives them; when no free
    block is left the least recently released are taken over, a sequence's
    later blocks before its earlier ones."""
    nb = alloc.num_blocks                            # expects 8 blocks
    assert nb == 8
    p = prompt(64)                                   # 4 full blocks
    alloc.add_seq_tokens(1, p)
    t1 = alloc.block_table(1)
    alloc.free_seq(1)
    assert alloc.num_cached() == 4 and alloc.num_free() == 8
    _, c = alloc.add_seq_tokens(2, p[:40])           # revives blocks 0 and 1
    assert c == 32 and alloc.block_table(2)[:2] == t1[:2]
    assert alloc.num_cached() == 2
    check_states(alloc, [2])
    # 3 free blocks and 2 cached unused ones are left; 4 new blocks take the
    # free ones and then the least recently released cached block: t1[3]
    # (released before t1[2])
    alloc.add_seq_tokens(3, prompt(64, 500))
    assert t1[3] in alloc.block_table(3) and t1[2] not in alloc.block_table(3)
    assert alloc.num_cached() == 1
    # the prefix's block 2 is still cached, block 3 is gone
    alloc.free_seq(2)
    _, c = alloc.add_seq_tokens(4, p)
    assert c == 48 and alloc.block_table(4)[:3] == t1[:3]
    check_states(alloc, [3, 4])


def check_enomem_all_or_nothing(alloc, exc):
    nb = alloc.num_blocks                            # expects 8 blocks
    alloc.add_seq_tokens(1, prompt(64))
    before = ([alloc.refcount(b) for b in range(nb)], alloc.num_free(), alloc.num_cached())
    try:
        alloc.add_seq_tokens(2, prompt(80, 900))     # 5 blocks, 4 left
        raise AssertionError("expected out-of-blocks")
    except exc:
        pass
    assert ([alloc.refcount(b) for b in range(nb)], alloc.num_free(), alloc.num_cached()) == before
    # a hit that revives cached blocks leaves fewer to take: counted before any change
    alloc.free_seq(1)                                # 4 cached, 4 free
    alloc.add_seq_tokens(3, prompt(16, 700))         # 1 free block used: 3 free + 4 cached
    try:
        alloc.add_seq_tokens(4, prompt(64) + prompt(64, 3000))   # 4 hits + 4 new: only 3 left
        raise AssertionError("expected out-of-blocks")
    except exc:
        pass
    assert alloc.num_cached() == 4 and alloc.num_free() == 7
    check_states(alloc, [3])


def check_fork_keeps_keys(alloc):
    """A forked child's full blocks are the parent's (already cached); its own
    appends after copy-on-write fill private blocks that are cached when full."""
    alloc.add_seq_tokens(1, prompt(24))              # block 0 full, block 1 has 8
    alloc.fork(1, 2)
    _, pairs = alloc.append_tokens(2, prompt(8, 24))  # fills the shared partial block: copy first
    assert len(pairs) == 1
    _, c = alloc.add_seq_tokens(3, prompt(40))
    assert c == 32 and alloc.block_table(3)[:2] == alloc.block_table(2)[:2]
    check_states(alloc, [1, 2, 3])


def check_plain_append_ends_caching(alloc):
    alloc.add_seq_tokens(1, prompt(8))
    alloc.append(1, 8)                               # ids unknown: block 0 fills uncached
    _, c = alloc.add_seq_tokens(2, prompt(16))
    assert c == 0
    check_states(alloc, [1, 2])
