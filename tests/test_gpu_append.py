"""GPU parity of the append form of decode (bf16): the new token's K/V are read
from the inputs and written to the cache inside the partition launch.

The bar is exactness against the two-call path it replaces: pkv_write of each
sequence's new token at slot table[(ctx-1)/16]*16 + (ctx-1)%16, then
pkv_attention_decode.  Both the output and the whole cache must match that path
byte for byte; the output is also checked against the oracle (write, then
attention) at the bf16 bar.  Contexts place the new token at every kind of
position: alone in the context, at a block's last and first row, at the first
token of a partition and of a two-partition work item, and at a ragged tail.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import (BLOCK_SIZE, SPECS, draw_context_lens, normal_values, pool_blocks_for,
                       random_block_tables)

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None

APPEND_CASES = {
    # name: (Hq, Hkv, D, context lengths including the new token)
    "gqa4_d128": (32, 8, 128, [1, 16, 17, 513, 1025, 1500, 2048, 5000]),
    "mha_d128": (32, 32, 128, [1, 15, 16, 17, 511, 512, 513, 1024, 1025]),
    "gqa2_d64": (8, 4, 64, [2, 31, 530, 1600]),
    "gqa8_d128": (16, 2, 128, [5, 260, 777, 2100]),
    "gqa4_d64": (16, 4, 64, [1, 16, 48, 4097]),
}


def case(seed, Hq, Hkv, D, ctx, spare_blocks=5):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    nb = int(sum(-(-c // BLOCK_SIZE) for c in ctx)) + spare_blocks
    mb = max(1, int(-(-ctx.max() // BLOCK_SIZE)) + 2)
    S = len(ctx)
    return {
        "context_lens": ctx, "block_tables": random_block_tables(rng, ctx, nb, mb), "num_blocks": nb,
        "key_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "value_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "q": normal_values(rng, (S, Hq, D), "bf16"),
        "k_new": normal_values(rng, (S, Hkv, D), "bf16"),
        "v_new": normal_values(rng, (S, Hkv, D), "bf16"),
        "scale": np.float32(1.0 / math.sqrt(D)),
    }


def new_slots(inp):
    tables, ctx = inp["block_tables"], inp["context_lens"]
    return np.array([oracle.slot_for_position(tables[s], int(ctx[s]) - 1) if ctx[s] > 0 else -1
                     for s in range(len(ctx))], np.int32)


def two_call(inp):
    """pkv_write of the new tokens, then pkv_attention_decode: (out, kc, vc) on the host."""
    kc, vc, q = dev(inp["key_cache"]), dev(inp["value_cache"]), dev(inp["q"])
    pkv.pkv_write(kc, vc, dev(inp["k_new"]), dev(inp["v_new"]), dev(new_slots(inp)))
    out = torch.empty_like(q)
    mx = int(inp["context_lens"].max(initial=0))
    pkv.pkv_attention_decode(out, q, kc, vc, dev(inp["block_tables"]), dev(inp["context_lens"]),
                             float(inp["scale"]), mx)
    torch.cuda.synchronize()
    return host(out), host(kc), host(vc)


def append_call(inp):
    kc, vc, q = dev(inp["key_cache"]), dev(inp["value_cache"]), dev(inp["q"])
    out = torch.empty_like(q)
    mx = int(inp["context_lens"].max(initial=0))
    pkv.pkv_attention_decode_append(out, q, dev(inp["k_new"]), dev(inp["v_new"]), kc, vc,
                                    dev(inp["block_tables"]), dev(inp["context_lens"]),
                                    float(inp["scale"]), mx)
    torch.cuda.synchronize()
    return out, host(kc), host(vc)


@pytest.mark.parametrize("name", sorted(APPEND_CASES))
def test_append_equals_write_then_decode(name):
    hq, hkv, d, ctx = APPEND_CASES[name]
    say(f"append {name}: hq={hq} hkv={hkv} d={d} ctx={ctx}")
    inp = case(sum(map(ord, name)), hq, hkv, d, ctx)
    ref_out, ref_kc, ref_vc = two_call(inp)
    out, kc, vc = append_call(inp)
    assert host(out).tobytes() == ref_out.tobytes()
    assert kc.tobytes() == ref_kc.tobytes() and vc.tobytes() == ref_vc.tobytes()
    kr, vr = oracle.write_kv(inp["key_cache"], inp["value_cache"], inp["k_new"], inp["v_new"],
                             new_slots(inp))
    assert kc.tobytes() == kr.tobytes() and vc.tobytes() == vr.tobytes()
    want = oracle.decode_attention(inp["q"], kr, vr, inp["block_tables"], inp["context_lens"],
                                   inp["scale"])
    assert_close(host_f64(out), want, "bf16", name)


def test_append_sees_only_its_new_token_when_alone():
    """Context of one token: the output is the new V row itself (repeated over the
    group's q heads), whatever the cache held at that slot before."""
    say("append ctx=1")
    inp = case(7, 32, 8, 128, [1] * 5)
    out, kc, _ = append_call(inp)
    got = host(out)
    for s in range(5):
        want = np.repeat(inp["v_new"][s], 4, axis=0)
        assert got[s].tobytes() == want.tobytes()
        b = inp["block_tables"][s, 0]
        assert kc[b, 0].tobytes() == inp["k_new"][s].tobytes()


def test_append_empty_context_and_out_of_pool_block():
    """ctx == 0 appends nothing and gives zeros; a new-token block id outside the
    pool is neither read nor written (the two-call path skips that slot too)."""
    say("append edges")
    inp = case(11, 32, 8, 128, [0, 40, 700, 33])
    inp["block_tables"][3, (33 - 1) // 16] = inp["num_blocks"] + 7      # new token's block: outside
    ref_out, ref_kc, ref_vc = two_call(inp)
    out, kc, vc = append_call(inp)
    assert host(out).tobytes() == ref_out.tobytes()
    assert kc.tobytes() == ref_kc.tobytes() and vc.tobytes() == ref_vc.tobytes()
    assert not np.any(host_f64(out)[0])


def test_three_call_append_form_equals_one_call():
    """plan (own stream), partitions_append, merge == the one-call append."""
    say("plan / partitions_append / merge")
    inp = case(13, 32, 8, 128, [40, 513, 1100, 3000, 7])
    ref, ref_kc, ref_vc = append_call(inp)
    q, kc, vc = dev(inp["q"]), dev(inp["key_cache"]), dev(inp["value_cache"])
    kn, vn = dev(inp["k_new"]), dev(inp["v_new"])
    tables, ctx = dev(inp["block_tables"]), dev(inp["context_lens"])
    mx = int(inp["context_lens"].max())
    sc = float(inp["scale"])
    out = torch.empty_like(q)
    ws = pkv.decode_workspace(5, 32, 128, mx)
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    with torch.cuda.stream(side):
        pkv.pkv_attention_decode_plan(out, q, kc, vc, tables, ctx, sc, mx, workspace=ws, stream=side)
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    pkv.pkv_attention_decode_partitions_append(out, q, kn, vn, kc, vc, tables, ctx, sc, mx, workspace=ws)
    pkv.pkv_attention_decode_merge(out, q, kc, vc, tables, ctx, sc, mx, workspace=ws)
    torch.cuda.synchronize()
    assert host(out).tobytes() == host(ref).tobytes()
    assert host(kc).tobytes() == ref_kc.tobytes() and host(vc).tobytes() == ref_vc.tobytes()


def test_append_full_size_bench_batch():
    """The benchmark's batch (128 sequences, GQA 32/8, d 128, contexts log-uniform
    in [512, 8192]): append form == write + decode, output and cache, byte for byte."""
    spec = SPECS["gqa32x8_bf16_s128_ctx512_8192"]
    say(f"append full size {spec.name}")
    rng = np.random.default_rng(4242)
    ctx = draw_context_lens(rng, spec)
    nb = pool_blocks_for(spec, ctx)
    mb = int(-(-ctx.max() // BLOCK_SIZE))
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    inp = {
        "context_lens": ctx, "block_tables": random_block_tables(rng, ctx, nb, mb), "num_blocks": nb,
        "key_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "value_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "q": normal_values(rng, (S, Hq, D), "bf16"),
        "k_new": normal_values(rng, (S, Hkv, D), "bf16"),
        "v_new": normal_values(rng, (S, Hkv, D), "bf16"),
        "scale": np.float32(1.0 / math.sqrt(D)),
    }
    ref_out, ref_kc, ref_vc = two_call(inp)
    out, kc, vc = append_call(inp)
    assert host(out).tobytes() == ref_out.tobytes()
    assert kc.tobytes() == ref_kc.tobytes() and vc.tobytes() == ref_vc.tobytes()
