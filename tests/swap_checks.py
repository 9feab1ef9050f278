"""Rules of preemption by swapping, usable against any allocator object.

The object must offer the allocator calls of allocator_checks plus
set_host_pool, swap_out, swap_in, is_swapped, host_table, num_free_host and
host_refcount.  Used for the oracle's model and for the product allocator
behind the C ABI.  ``err`` is the exception type(s) the object raises for a call
on a sequence in the wrong pool or an unknown / duplicate id.

What the pages fix ("vLLM and PagedAttention", §3 continuous batching, on the
scheduler's preemption; "How vLLM Works?", section 04): a preempted request's KV
leaves GPU memory for CPU memory and comes back once memory frees up, so after
a round trip each sequence must see exactly the K/V it had.  The content check
below runs the allocator's copy pairs through the oracle's pool-to-pool copy on
NumPy pools and compares every swapped sequence's gathered K/V bit for bit,
after the device blocks it gave up have been poisoned and reused.
"""

import collections

import numpy as np

import oracle


def check_swap_invariants(alloc, on_device, swapped):
    """Counts equal table entries in both pools; every block is used or free."""
    bs = alloc.block_size
    dev, host = collections.Counter(), collections.Counter()
    for sid in on_device:
        assert not alloc.is_swapped(sid)
        tbl = alloc.block_table(sid)
        assert len(tbl) == -(-alloc.seq_len(sid) // bs)
        dev.update(tbl)
    for sid in swapped:
        assert alloc.is_swapped(sid)
        tbl = alloc.host_table(sid)
        assert len(tbl) == -(-alloc.seq_len(sid) // bs)
        host.update(tbl)
    for b in range(alloc.num_blocks):
        assert alloc.refcount(b) == dev.get(b, 0), b
    nh = alloc.num_host_blocks
    for h in range(nh):
        assert alloc.host_refcount(h) == host.get(h, 0), h
    assert sum(1 for h in range(nh) if host.get(h, 0)) + alloc.num_free_host() == nh


def check_sharing_survives_group_round_trip(alloc):
    """A fork swapped out with its parent keeps sharing: one host block per
    distinct device block, shared again after the swap-in, and the first append
    into the shared partial block still copies it."""
    bs = alloc.block_size
    alloc.set_host_pool(32)
    alloc.add_seq(1)
    alloc.append(1, 3 * bs + 4)                      # 4 blocks, last partial
    alloc.fork(1, 2)
    alloc.append(2, 1)                               # child copies the partial block
    free_dev, free_host = alloc.num_free(), alloc.num_free_host()
    pairs = alloc.swap_out([1, 2])
    assert len(pairs) == 5                           # 3 shared full + 2 partial copies
    assert len({d for d, _ in pairs}) == 5 and len({h for _, h in pairs}) == 5
    assert alloc.num_free() == free_dev + 5 and alloc.num_free_host() == free_host - 5
    h1, h2 = alloc.host_table(1), alloc.host_table(2)
    assert h1[:3] == h2[:3] and h1[3] != h2[3]
    assert [alloc.host_refcount(h) for h in h1] == [2, 2, 2, 1]
    check_swap_invariants(alloc, [], [1, 2])
    back = alloc.swap_in([1, 2])
    assert [h for h, _ in back] == list(dict.fromkeys(h1 + h2))
    t1, t2 = alloc.block_table(1), alloc.block_table(2)
    assert t1[:3] == t2[:3] and [alloc.refcount(b) for b in t1] == [2, 2, 2, 1]
    assert alloc.num_free_host() == free_host and alloc.num_free() == free_dev
    alloc.fork(2, 3)
    _, cow = alloc.append(3, 1)
    assert len(cow) == 1 and cow[0][0] == t2[3]
    check_swap_invariants(alloc, [1, 2, 3], [])
    for sid in (1, 2, 3):
        alloc.free_seq(sid)


def check_partial_group_copies_and_keeps_shared(alloc):
    """Swapping out a fork without its parent copies every block the fork holds;
    the blocks the parent still holds stay on the device."""
    bs = alloc.block_size
    alloc.set_host_pool(16)
    alloc.add_seq(10)
    alloc.append(10, 2 * bs + 1)
    alloc.fork(10, 11)
    parent = alloc.block_table(10)
    free_dev = alloc.num_free()
    pairs = alloc.swap_out([11])
    assert [d for d, _ in pairs] == parent
    assert alloc.num_free() == free_dev               # the parent still holds all three
    assert [alloc.refcount(b) for b in parent] == [1, 1, 1]
    alloc.append(10, 1)                               # parent writes in place now: no copy
    assert alloc.block_table(10) == parent
    back = alloc.swap_in([11])
    assert len(back) == 3 and set(alloc.block_table(11)).isdisjoint(parent)
    check_swap_invariants(alloc, [10, 11], [])
    alloc.free_seq(10)
    alloc.free_seq(11)


def check_wrong_pool_and_bad_groups(alloc, err):
    alloc.set_host_pool(8)
    alloc.add_seq(20)
    alloc.append(20, 20)
    alloc.add_seq(21)
    alloc.append(21, 5)
    alloc.swap_out([20])
    for call in (lambda: alloc.append(20, 1), lambda: alloc.fork(20, 22), lambda: alloc.block_table(20),
                 lambda: alloc.swap_out([20]), lambda: alloc.swap_in([21]), lambda: alloc.swap_in([20, 20]),
                 lambda: alloc.swap_out([999]), lambda: alloc.add_seq(20), lambda: alloc.set_host_pool(4)):
        try:
            call()
        except err:
            continue
        raise AssertionError("expected an error")
    assert alloc.is_swapped(20) and not alloc.is_swapped(21)
    assert alloc.seq_len(20) == 20
    free_host = alloc.num_free_host()
    alloc.free_seq(20)                                # host blocks return
    assert alloc.num_free_host() == free_host + 2
    alloc.free_seq(21)
    assert alloc.num_free() == alloc.num_blocks and alloc.num_free_host() == 8


def check_out_of_blocks_changes_nothing(alloc):
    """Both directions are all-or-nothing."""
    bs = alloc.block_size
    nb = alloc.num_blocks
    alloc.set_host_pool(3)
    alloc.add_seq(30)
    alloc.append(30, 2 * bs)
    alloc.add_seq(31)
    alloc.append(31, 2 * bs)

    def state():
        return ([alloc.block_table(s) for s in (30, 31)], alloc.num_free(), alloc.num_free_host(),
                [alloc.refcount(b) for b in range(nb)], [alloc.host_refcount(h) for h in range(3)])

    before = state()
    try:
        alloc.swap_out([30, 31])                      # 4 blocks, 3 host blocks
        raise AssertionError("expected out-of-memory")
    except MemoryError:
        pass
    assert state() == before
    alloc.swap_out([30])
    alloc.append(31, (alloc.num_free() - 1) * bs)     # leave one free device block
    sw = (alloc.host_table(30), alloc.num_free(), alloc.num_free_host())
    try:
        alloc.swap_in([30])                           # needs two
        raise AssertionError("expected out-of-memory")
    except MemoryError:
        pass
    assert (alloc.host_table(30), alloc.num_free(), alloc.num_free_host()) == sw
    alloc.free_seq(31)
    alloc.swap_in([30])
    alloc.free_seq(30)
    assert alloc.num_free() == nb and alloc.num_free_host() == 3


def check_content_round_trip(alloc, rng, rounds=6, hkv=2, d=8):
    """Random sequences with forks and copy-on-write on NumPy pools: every
    swapped sequence's K/V, gathered through its table after the swap-in, equals
    what it was before the swap-out, bit for bit, although the device blocks it
    gave up were poisoned and handed to other sequences in between."""
    bs = alloc.block_size
    nb = alloc.num_blocks
    nh = 3 * nb
    alloc.set_host_pool(nh)
    kc = np.full((nb, bs, hkv, d), np.nan, np.float32)
    vc = kc.copy()
    hk = np.full((nh, bs, hkv, d), np.nan, np.float32)
    hv = hk.copy()
    live, swapped, nxt = [], [], 0

    def write(sid, n):
        nonlocal kc, vc
        slots, cow = alloc.append(sid, n)
        if cow:
            kc, vc = oracle.copy_blocks(kc, vc, cow)
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        kc, vc = oracle.write_kv(kc, vc, k, v, np.array(slots, np.int32), bs)

    def logical(sid):
        return oracle.gather_kv(kc, vc, np.array(alloc.block_table(sid), np.int32), alloc.seq_len(sid), bs)

    for _ in range(rounds):
        # grow: new sequences, forks, appends, while blocks last
        for _ in range(6):
            try:
                if not live or rng.integers(3) == 0:
                    alloc.add_seq(nxt)
                    live.append(nxt)
                    nxt += 1
                    write(live[-1], int(rng.integers(1, 3 * bs)))
                elif rng.integers(2) == 0:
                    alloc.fork(live[int(rng.integers(len(live)))], nxt)
                    live.append(nxt)
                    nxt += 1
                else:
                    write(live[int(rng.integers(len(live)))], int(rng.integers(1, bs + 3)))
            except MemoryError:
                break
        # swap a random group out; poison what it released; reuse it
        if live:
            group = [int(s) for s in rng.choice(live, size=int(rng.integers(1, len(live) + 1)), replace=False)]
            before = {s: logical(s) for s in group}
            pairs = alloc.swap_out(group)
            if pairs:
                hk, hv = oracle.swap_blocks(hk, hv, kc, vc, pairs)
            for s in group:
                live.remove(s)
                swapped.append((s, before[s]))
            for b in range(nb):
                if alloc.refcount(b) == 0:
                    kc[b] = np.nan
                    vc[b] = -np.inf
            try:
                alloc.add_seq(nxt)
                live.append(nxt)
                nxt += 1
                write(live[-1], int(rng.integers(1, 4 * bs)))
            except MemoryError:
                pass
            check_swap_invariants(alloc, live, [s for s, _ in swapped])
        # bring back as many as fit, oldest first, freeing device sequences if needed
        while swapped:
            sid, want = swapped[0]
            try:
                pairs = alloc.swap_in([sid])
            except MemoryError:
                if not live:
                    raise
                alloc.free_seq(live.pop(0))
                continue
            if pairs:
                kc, vc = oracle.swap_blocks(kc, vc, hk, hv, pairs)
            swapped.pop(0)
            live.append(sid)
            got = logical(sid)
            assert got[0].tobytes() == want[0].tobytes() and got[1].tobytes() == want[1].tobytes(), sid
        check_swap_invariants(alloc, live, [])
    for s in live:
        alloc.free_seq(s)
    assert alloc.num_free() == nb and alloc.num_free_host() == nh
