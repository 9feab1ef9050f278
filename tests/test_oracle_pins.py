"""The oracle pinned to facts other than itself (CPU only).

Pins: a library attention routine on contiguous K/V, brute-force permutation
invariance of the block table, closed forms (one-token context, zero query,
collapsed softmax), masking of poisoned unused memory, GQA == repeated-KV MHA,
split == unsplit for the log-sum-exp merge, round-trip and untouched-bytes checks
for the scatter write and the block copy, and the IEEE definition of bf16.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle_pins import DECODE_CHECKS, random_case, sdpa_reference
from workloads import f32_to_bf16_bits

BS = 16


@pytest.mark.parametrize("name", sorted(DECODE_CHECKS))
def test_decode_pin(name):
    check, bound = DECODE_CHECKS[name]
    assert check(oracle.decode_attention) <= bound


def test_widen_bf16_is_ieee():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, math.inf, -math.inf, 2.0 ** -133, -0.0, 3.140625]
    got = oracle.widen(bits)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    assert np.isnan(oracle.widen(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_generator_bf16_rounding_is_rne():
    # halfway cases round to even; above/below halfway round to nearest
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0 - 2 ** -7 - 2 ** -9,
                  65504.0, np.inf, -np.inf, 0.0], dtype=np.float32)
    got = oracle.widen(f32_to_bf16_bits(x))
    want = [1.0, 1.0 + 4 * 2 ** -8, 1.0 + 2 ** -7, -2.0 - 2 ** -6, 65536.0, np.inf, -np.inf, 0.0]
    assert list(got) == want
    assert np.isnan(oracle.widen(f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))))[0]


def test_bf16_inputs_match_sdpa_on_rounded_values():
    """bf16 storage: the oracle reads the rounded values exactly."""
    c = random_case(21, [7, 30], 4, 2, 16)
    kb, vb, qb = (f32_to_bf16_bits(np.nan_to_num(c[k])) for k in ("kc", "vc", "q"))
    got = oracle.decode_attention(qb, kb, vb, c["tables"], c["ctx"], c["scale"])
    ks = [oracle.widen(f32_to_bf16_bits(k)) for k in c["ks"]]
    vs = [oracle.widen(f32_to_bf16_bits(v)) for v in c["vs"]]
    ref = sdpa_reference(oracle.widen(qb), ks, vs, c["scale"], 4)
    assert np.max(np.abs(got - ref)) < 1e-12


# --------------------------------------------------------------------- causal chunk
def test_causal_chunk_matches_masked_sdpa():
    rng = np.random.default_rng(31)
    Hq, Hkv, D = 4, 2, 16
    ctx = [40, 23, 1]
    qlen = [9, 1, 1]
    c = random_case(31, ctx, Hq, Hkv, D)
    T = sum(qlen)
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    got = oracle.causal_chunk_attention(q, c["kc"], c["vc"], c["tables"], c["ctx"], qsl, c["scale"])
    for s in range(len(ctx)):
        n, L = ctx[s], qlen[s]
        K = torch.from_numpy(c["ks"][s].astype(np.float64)).repeat_interleave(2, 1).permute(1, 0, 2)[None]
        V = torch.from_numpy(c["vs"][s].astype(np.float64)).repeat_interleave(2, 1).permute(1, 0, 2)[None]
        Q = torch.from_numpy(q[qsl[s]:qsl[s + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        pos = torch.arange(n - L, n)[:, None]
        mask = torch.arange(n)[None, :] <= pos                       # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=float(c["scale"]))
        assert np.max(np.abs(got[qsl[s]:qsl[s + 1]] - ref[0].permute(1, 0, 2).numpy())) < 1e-12


def test_causal_chunk_decode_rows_equal_decode():
    c = random_case(32, [5, 50, 17], 8, 2, 8)
    qsl = np.arange(4, dtype=np.int32)
    a = oracle.causal_chunk_attention(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], qsl, c["scale"])
    b = oracle.decode_attention(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- merge
def test_merge_hand_example():
    # scores (0, ln 3) -> softmax (1/4, 3/4); V = (1, 0) -> 0.25, split one token per partition
    m = np.array([0.0, math.log(3.0)])
    l = np.array([1.0, 1.0])
    o = np.array([[1.0], [0.0]])
    assert abs(oracle.merge_partials(m, l, o)[0] - 0.25) < 1e-15


@pytest.mark.parametrize("psize", [1, 7, 16, 512, 1000, 4096])
def test_merge_split_equals_unsplit(psize):
    rng = np.random.default_rng(psize)
    n, D = 1000, 12
    x = rng.standard_normal(n) * 3.0
    V = rng.standard_normal((n, D))
    m, l, o = oracle.split_decode_partials(x, V, psize)
    got = oracle.merge_partials(m, l, o)
    w = np.exp(x - x.max())
    want = (w @ V) / w.sum()
    assert np.max(np.abs(got - want)) < 1e-13


def test_merge_empty_partials():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(40)
    V = rng.standard_normal((40, 4))
    m, l, o = oracle.split_decode_partials(x, V, 16)
    m2 = np.concatenate([[-np.inf], m, [-np.inf]])
    l2 = np.concatenate([[0.0], l, [0.0]])
    o2 = np.concatenate([np.full((1, 4), np.nan), o, np.full((1, 4), np.nan)])
    assert np.max(np.abs(oracle.merge_partials(m2, l2, o2) - oracle.merge_partials(m, l, o))) == 0.0
    z = oracle.merge_partials(np.full(3, -np.inf), np.zeros(3), np.full((3, 4), np.nan))
    assert np.array_equal(z, np.zeros(4))


def test_merge_single_partial_is_identity():
    o = np.array([[0.5, -2.0, 3.25]])
    assert np.array_equal(oracle.merge_partials([1.7], [3.0], o), o[0])


# --------------------------------------------------------------------------- write
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_round_trip_and_untouched(dtype):
    rng = np.random.default_rng(41)
    NB, Hkv, D = 12, 2, 8
    if dtype == "f32":
        kc = rng.standard_normal((NB, BS, Hkv, D)).astype(np.float32)
        vc = rng.standard_normal((NB, BS, Hkv, D)).astype(np.float32)
    else:
        kc = rng.integers(0, 2 ** 16, (NB, BS, Hkv, D), dtype=np.uint16)
        vc = rng.integers(0, 2 ** 16, (NB, BS, Hkv, D), dtype=np.uint16)
    slots = rng.choice(NB * BS, size=30, replace=False).astype(np.int32)
    slots[3] = -1
    slots[7] = -5
    k = (rng.standard_normal((30, Hkv, D)).astype(np.float32) if dtype == "f32"
         else rng.integers(0, 2 ** 16, (30, Hkv, D), dtype=np.uint16))
    v = k[::-1].copy()
    k2, v2 = oracle.write_kv(kc, vc, k, v, slots)
    flat_k, flat_v = k2.reshape(NB * BS, Hkv, D), v2.reshape(NB * BS, Hkv, D)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written.add(int(s))
        assert flat_k[s].tobytes() == k[i].tobytes()
        assert flat_v[s].tobytes() == v[i].tobytes()
    keep = np.array([i not in written for i in range(NB * BS)])
    assert flat_k[keep].tobytes() == kc.reshape(NB * BS, Hkv, D)[keep].tobytes()
    assert flat_v[keep].tobytes() == vc.reshape(NB * BS, Hkv, D)[keep].tobytes()
    # inputs untouched
    assert not np.shares_memory(k2, kc)


def test_write_then_gather_through_table():
    """Write a sequence token by token via its table, then gather it back in order."""
    rng = np.random.default_rng(42)
    NB, Hkv, D, n = 9, 1, 4, 100
    table = rng.permutation(NB)[:7].astype(np.int32)          # 100 tokens -> 7 blocks
    kc = np.zeros((NB, BS, Hkv, D), np.float32)
    vc = np.zeros((NB, BS, Hkv, D), np.float32)
    toks = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    slots = [oracle.slot_for_position(table, p) for p in range(n)]
    assert slots[99] // BS == table[6]                        # the 100th token sits in the 7th block
    kc, vc = oracle.write_kv(kc, vc, toks, -toks, np.array(slots, np.int32))
    K, V = oracle.gather_kv(kc, vc, table, n)
    assert np.array_equal(K, toks.astype(np.float64))
    assert np.array_equal(V, -toks.astype(np.float64))


def test_copy_blocks_bitwise():
    rng = np.random.default_rng(43)
    kc = rng.integers(0, 2 ** 16, (10, BS, 2, 8), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, (10, BS, 2, 8), dtype=np.uint16)
    pairs = np.array([[1, 7], [3, 2], [1, 9]], np.int32)
    k2, v2 = oracle.copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        assert k2[d].tobytes() == kc[s].tobytes() and v2[d].tobytes() == vc[s].tobytes()
    for b in set(range(10)) - {7, 2, 9}:
        assert k2[b].tobytes() == kc[b].tobytes() and v2[b].tobytes() == vc[b].tobytes()
