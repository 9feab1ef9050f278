"""Pins of the oracle's swapping model and its pool-to-pool copy (CPU).

The allocator model's swap-out / swap-in and ``oracle.swap_blocks`` are pinned
together by the content round trip (each swapped sequence gathers the same K/V
bit for bit after its old device blocks were poisoned and reused), and the
model alone by the counting rules in swap_checks.  ``swap_blocks`` is pinned on
its own by a brute-force byte comparison: every destination block named by a
pair equals its source block, every other byte is unchanged.
"""

import numpy as np
import pytest

import oracle
import swap_checks as sc


def model(nb=24, caching=True):
    cls = oracle.PrefixCachingAllocatorModel if caching else oracle.BlockAllocatorModel
    m = cls(nb, 16)
    m.num_host_blocks = 0
    orig = m.set_host_pool

    def set_host_pool(n):
        orig(n)
        m.num_host_blocks = n
    m.set_host_pool = set_host_pool
    return m


@pytest.mark.parametrize("caching", [False, True])
def test_sharing_survives_group_round_trip(caching):
    sc.check_sharing_survives_group_round_trip(model(caching=caching))


@pytest.mark.parametrize("caching", [False, True])
def test_partial_group(caching):
    sc.check_partial_group_copies_and_keeps_shared(model(caching=caching))


def test_wrong_pool_and_bad_groups():
    sc.check_wrong_pool_and_bad_groups(model(), (KeyError, ValueError))


def test_out_of_blocks_changes_nothing():
    sc.check_out_of_blocks_changes_nothing(model(nb=8))


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
@pytest.mark.parametrize("caching", [False, True])
def test_content_round_trip(seed, caching):
    sc.check_content_round_trip(model(nb=20, caching=caching), np.random.default_rng(seed))


def test_swap_blocks_brute_force():
    rng = np.random.default_rng(0)
    src_k = rng.integers(0, 2**16, (5, 16, 2, 4), dtype=np.uint16)
    src_v = rng.integers(0, 2**16, (5, 16, 2, 4), dtype=np.uint16)
    dst_k = rng.integers(0, 2**16, (7, 16, 2, 4), dtype=np.uint16)
    dst_v = rng.integers(0, 2**16, (7, 16, 2, 4), dtype=np.uint16)
    pairs = [(4, 0), (0, 6), (2, 3), (9, 1), (1, -1)]        # the last two name no block
    k, v = oracle.swap_blocks(dst_k, dst_v, src_k, src_v, pairs)
    for b in range(7):
        src = {0: 4, 6: 0, 3: 2}.get(b)
        want_k = src_k[src] if src is not None else dst_k[b]
        want_v = src_v[src] if src is not None else dst_v[b]
        assert k[b].tobytes() == want_k.tobytes() and v[b].tobytes() == want_v.tobytes()
    assert k is not dst_k and dst_k[0].tobytes() != src_k[4].tobytes()   # inputs untouched


def test_content_pin_catches_a_wrong_pair_order():
    """A planted mistake (the copy run the wrong way round) fails the round trip."""
    m = model(nb=20, caching=False)
    orig = oracle.swap_blocks
    try:
        oracle.swap_blocks = lambda dk, dv, sk, sv, pairs: orig(dk, dv, sk, sv, [(b, a) for a, b in pairs])
        with pytest.raises(AssertionError):
            sc.check_content_round_trip(m, np.random.default_rng(1))
    finally:
        oracle.swap_blocks = orig
