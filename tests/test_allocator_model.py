"""The oracle's allocator model against the pages' worked numbers and invariants (CPU)."""

import numpy as np
import pytest

import oracle
from allocator_checks import (check_enomem_atomic, check_fork_and_cow, check_hundred_tokens,
                              check_paged_waste_under_one_block, random_ops)


def make(nb=64, seed=0):
    order = np.random.default_rng(seed).permutation(nb)
    return oracle.BlockAllocatorModel(nb, 16, free_order=order)


def test_hundred_tokens_seven_blocks():
    check_hundred_tokens(make())


def test_paged_waste_under_one_block():
    check_paged_waste_under_one_block(make(nb=1024), np.random.default_rng(1))


def test_fork_and_cow():
    check_fork_and_cow(make())


def test_enomem_atomic():
    check_enomem_atomic(make(nb=20), MemoryError)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_ops(seed):
    random_ops(make(nb=48, seed=seed), np.random.default_rng(seed), 400, MemoryError)


def test_slot_for_position():
    table = [42, 17, 5, 99, 31]            # the pages' logical -> physical example ids
    assert oracle.slot_for_position(table, 0) == 42 * 16
    assert oracle.slot_for_position(table, 17) == 17 * 16 + 1
    assert oracle.slot_for_position(table, 79) == 31 * 16 + 15
