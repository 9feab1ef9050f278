"""The partition launch's load cache policy hint, on the GPU.

The plan flags a launch whose decode sequences share a first block (a shared
prefix or a fork, "vLLM and PagedAttention", §2 shareable prefixes with
copy-on-write): the partition kernel then keeps the default cache policy for
its block loads, so shared blocks stay cached for their other readers;
otherwise the loads stream.  The flag is the fifth word of the plan's ticket
header at the start of the workspace.  The hint changes no result: the same
batch decoded with and without a shared first block (the shared block holding
the same bytes as the private one it replaces) gives identical outputs, and
the shared batch matches the oracle on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import normal_values_parallel

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None

SCHED_SHARED_WORD = 4   # ticket header word written by the plan


def _decode(tables, ctx, kc, vc, q, scale, bound):
    S, Hq, D = q.shape
    ws = pkv.decode_workspace(S, Hq, D, bound)
    out = torch.empty_like(q)
    pkv.pkv_attention_decode(out, q, kc, vc, dev(tables), dev(ctx), scale, bound, workspace=ws)
    torch.cuda.synchronize()
    flag = int(ws[:64].cpu().numpy().view(np.int32)[SCHED_SHARED_WORD])
    return out, flag


def test_shared_first_block_flag_and_identical_results():
    S, Hq, Hkv, D, C = 64, 32, 8, 128, 1500
    say(f"cache hint: {S} sequences of {C} tokens, GQA {Hq}/{Hkv}")
    mb = -(-C // 16)
    nb = S * mb + 16
    rng = np.random.default_rng(11)
    tables = rng.permutation(nb)[:S * mb].astype(np.int32).reshape(S, mb)
    ctx = np.full(S, C, np.int32)
    kh = normal_values_parallel(41, (nb, 16, Hkv, D), "bf16")
    vh = normal_values_parallel(42, (nb, 16, Hkv, D), "bf16")
    # every sequence's first block holds the same bytes as sequence 0's, so
    # pointing their tables at sequence 0's block changes nothing but sharing
    for s in range(1, S):
        kh[tables[s, 0]] = kh[tables[0, 0]]
        vh[tables[s, 0]] = vh[tables[0, 0]]
    kc, vc = dev(kh), dev(vh)
    qh = normal_values_parallel(43, (S, Hq, D), "bf16")
    q = dev(qh)
    scale = float(np.float32(1.0 / math.sqrt(D)))

    out_private, flag_private = _decode(tables, ctx, kc, vc, q, scale, C)
    shared = tables.copy()
    shared[1:, 0] = tables[0, 0]
    out_shared, flag_shared = _decode(shared, ctx, kc, vc, q, scale, C)
    assert flag_private == 0, "no first block is shared: the launch should stream"
    assert flag_shared == 1, "first blocks are shared: the launch should keep the default policy"
    assert host(out_private).tobytes() == host(out_shared).tobytes()
    rows = np.array([0, 1, S - 1])
    ref = oracle.decode_attention(qh[rows], kh, vh, shared[rows], ctx[rows], np.float32(scale))
    assert_close(host_f64(out_shared)[rows], ref, "bf16", "cache hint, shared first block")


def test_more_first_blocks_than_hash_slots_keeps_the_cached_policy():
    """5000 decode sequences with distinct first blocks overflow the plan's
    4096-slot table: a first block whose probe run finds no slot counts as
    shared, so the launch keeps the default policy (the safe side); results are
    unchanged."""
    S, Hq, Hkv, D, C = 5000, 8, 2, 64, 40
    say(f"cache hint: {S} sequences of {C} tokens")
    mb = -(-C // 16)
    nb = S * mb + 8
    rng = np.random.default_rng(12)
    tables = rng.permutation(nb)[:S * mb].astype(np.int32).reshape(S, mb)
    ctx = np.full(S, C, np.int32)
    kh = normal_values_parallel(51, (nb, 16, Hkv, D), "bf16")
    vh = normal_values_parallel(52, (nb, 16, Hkv, D), "bf16")
    qh = normal_values_parallel(53, (S, Hq, D), "bf16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out, flag = _decode(tables, ctx, dev(kh), dev(vh), dev(qh), scale, C)
    assert flag == 1
    rows = np.array([0, 1, 2047, 4095, 4096, S - 1])
    ref = oracle.decode_attention(qh[rows], kh, vh, tables[rows], ctx[rows], np.float32(scale))
    assert_close(host_f64(out)[rows], ref, "bf16", "cache hint, 5000 first blocks")
