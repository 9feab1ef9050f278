"""The oracle's prefix-caching allocator model against the pages' rules (CPU)."""

import numpy as np
import pytest

import oracle
import prefix_cache_checks as pc


def make(nb=64, seed=0):
    order = np.random.default_rng(seed).permutation(nb)
    return oracle.PrefixCachingAllocatorModel(nb, 16, free_order=order)


@pytest.mark.parametrize("check", [pc.check_equal_prefix_same_blocks, pc.check_salt_isolates,
                                   pc.check_key_includes_everything_before,
                                   pc.check_appended_blocks_are_cached, pc.check_fork_keeps_keys,
                                   pc.check_plain_append_ends_caching])
def test_rule(check):
    check(make())


def test_released_blocks_reused_then_taken_over():
    pc.check_released_blocks_reused_then_taken_over(make(nb=8))


def test_enomem_all_or_nothing():
    pc.check_enomem_all_or_nothing(make(nb=8), MemoryError)


def test_system_prompt_scenario():
    """The pages' scenario: a 1500-token system prompt and short user queries.
    After the first request, each request computes only its partial system-prompt
    block and its own query: 1500 = 93*16 + 12, so 1488 of its tokens are reused."""
    m = make(nb=4096)
    system = pc.prompt(1500)
    rng = np.random.default_rng(5)
    reused = []
    for i in range(20):
        query = pc.prompt(int(rng.integers(8, 64)), 10_000 + 100 * i)
        _, c = m.add_seq_tokens(i, system + query)
        reused.append(c)
    assert reused[0] == 0 and all(c == 1488 for c in reused[1:])
    pc.check_states(m, list(range(20)))
