"""GPU parity for variable-length attention: decode rows and chunked-prefill rows.

``pkv_attention_varlen`` through the C ABI against ``oracle.causal_chunk_attention``
(row r of a chunk of q rows over ctx keys sees keys 0 .. ctx - q + r), at sizes
that span several 16-column tiles, 16-token blocks and 512-token partitions with
ragged tails; and at the full mixed-step size (one 512-row chunk at the end of a
4096-token context plus 192 decode sequences) on sampled rows, where each
sampled row is the decode of its own truncated context in the oracle.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import (BLOCK_SIZE, SPECS, draw_context_lens, f32_to_bf16_bits, normal_values,
                       normal_values_parallel, pool_blocks_for, random_block_tables)

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None


def mixed_case(seed, Hq, Hkv, D, qlens, ctxs, spare=5):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctxs, np.int32)
    qlens = np.asarray(qlens, np.int32)
    nb = int(sum(-(-c // BLOCK_SIZE) for c in ctx)) + spare
    mb = max(1, int(-(-ctx.max() // BLOCK_SIZE)) + 1)
    tables = random_block_tables(rng, ctx, nb, mb)
    T = int(qlens.sum())
    return {
        "context_lens": ctx, "block_tables": tables, "num_blocks": nb,
        "qsl": np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32),
        "key_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "value_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "q": normal_values(rng, (T, Hq, D), "bf16"),
        "scale": np.float32(1.0 / math.sqrt(D)),
        "max_query_len": int(qlens.max()),
    }


def gpu_varlen(inp, kc=None, vc=None):
    q = dev(inp["q"])
    out = torch.full_like(q, float("nan"))
    kc = dev(inp["key_cache"]) if kc is None else kc
    vc = dev(inp["value_cache"]) if vc is None else vc
    ctx = inp["context_lens"]
    pkv.pkv_attention_varlen(out, q, kc, vc, dev(inp["block_tables"]), dev(ctx), dev(inp["qsl"]),
                             float(inp["scale"]), inp["max_query_len"], int(ctx.max()))
    torch.cuda.synchronize()
    return out


def oracle_varlen(inp):
    return oracle.causal_chunk_attention(inp["q"], inp["key_cache"], inp["value_cache"],
                                         inp["block_tables"], inp["context_lens"], inp["qsl"],
                                         inp["scale"])


VARLEN_CASES = {
    # name: (Hq, Hkv, D, query lengths, context lengths)
    "gqa4_d128": (32, 8, 128, [1, 40, 1, 17, 3, 130], [600, 40, 1, 530, 1100, 1500]),
    "gqa4_d128_long_chunk": (32, 8, 128, [300, 1, 1], [1300, 2048, 77]),
    "mha_d64": (8, 8, 64, [1, 70, 2, 65], [90, 800, 513, 65]),
    "gqa8_d128": (16, 2, 128, [9, 1, 33, 8], [1024, 517, 600, 8]),
    "gqa2_d64": (8, 4, 64, [31, 1, 12], [700, 1000, 12]),
    # one tile row group per 256 / G rows: chunks at, one past and one short of
    # that size, with last rows that cross a 512-key partition boundary
    "mha_d128": (16, 16, 128, [64, 1, 257, 5], [64, 900, 1030, 520]),
    "gqa2_d128": (16, 8, 128, [128, 129, 2], [128, 1000, 2]),
    "gqa8_d64": (32, 4, 64, [33, 32, 1], [33, 600, 3000]),
    # prefill rows only (no decode work), row groups of 64 at partition edges
    "gqa4_d128_item_edges": (32, 8, 128, [64, 65, 128, 63], [64, 577, 640, 1087]),
    # a chunk deep in a long context (40 partitions: many items per row group,
    # merged from many slots) beside a long decode row
    "gqa4_d64_long_context": (16, 4, 64, [160, 1], [20000, 9000]),
}


@pytest.mark.parametrize("name", sorted(VARLEN_CASES))
def test_varlen_matches_oracle(name):
    hq, hkv, d, qlens, ctxs = VARLEN_CASES[name]
    say(f"varlen {name}: hq={hq} hkv={hkv} d={d} q={qlens} ctx={ctxs}")
    inp = mixed_case(zlib.crc32(name.encode()) % 1000, hq, hkv, d, qlens, ctxs)
    got = host_f64(gpu_varlen(inp))
    assert_close(got, oracle_varlen(inp), "bf16", name)


def test_varlen_many_short_chunks():
    """Many chunks of 2 .. 12 rows over short contexts, so that a persistent
    workgroup runs several one- and two-block items in a row (the key stream
    prefetched across item boundaries), interleaved with decode rows."""
    rng = np.random.default_rng(53)
    n = 150
    qlens = rng.integers(2, 13, n)
    qlens[rng.random(n) < 0.2] = 1
    ctxs = np.maximum(qlens, rng.integers(1, 260, n))
    ctxs[::7] = qlens[::7]                      # chunks that are the whole context
    say(f"varlen many short chunks: {n} seqs, {int(qlens.sum())} rows")
    inp = mixed_case(53, 32, 8, 128, qlens, ctxs)
    got = host_f64(gpu_varlen(inp))
    assert_close(got, oracle_varlen(inp), "bf16", "short chunks")


def test_varlen_runs_of_padded_items():
    """Chunks over contexts of 150 .. 600 keys: prefill items of about 5 to 19
    two-block steps (padded to an even count of at least six), several
    per persistent workgroup, so that the key stream runs from one short item into
    the next again and again; some rows cross the 512-key partition edge."""
    rng = np.random.default_rng(71)
    n = 200
    qlens = rng.integers(2, 41, n)
    qlens[rng.random(n) < 0.15] = 1
    ctxs = np.maximum(qlens, rng.integers(150, 601, n))
    say(f"varlen runs of padded items: {n} seqs, {int(qlens.sum())} rows")
    inp = mixed_case(71, 32, 8, 128, qlens, ctxs)
    got = host_f64(gpu_varlen(inp))
    assert_close(got, oracle_varlen(inp), "bf16", "padded items")


def prefill_span(qlens, ctxs, G, Hkv, cus):
    """The plan's span rule restated: prefill items cover two partitions when the
    rounds of items per compute unit at span 2 are at most half those at span 1."""
    rpi = 256 // G
    n1 = n2 = 0
    for q, c in zip(qlens, ctxs):
        if q <= 1:
            continue
        for r0 in range(0, q, rpi):
            keys = max(0, c - q + min(q, r0 + rpi))
            n = max(1, -(-keys // 512))
            n1, n2 = n1 + n, n2 + (n + 1) // 2
    r1, r2 = -(-n1 * Hkv // cus), -(-n2 * Hkv // cus)
    return 2 if r1 > 1 and 2 * r2 <= r1 else 1


SPAN2_CASES = {
    # rows with 1, 2, 4 and 5 partitions; two-partition items whose second
    # partition is empty, partly used, or absent (odd partition counts)
    "mha_d64": (32, 32, 64, [256, 256, 100, 1], [2300, 1000, 560, 3000]),
    "gqa4_d128": (32, 8, 128, [256, 256, 1], [2500, 2600, 777]),
}


@pytest.mark.parametrize("name", sorted(SPAN2_CASES))
def test_varlen_two_partition_prefill_items(name):
    hq, hkv, d, qlens, ctxs = SPAN2_CASES[name]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"varlen span-2 {name}: cus={cus} span={prefill_span(qlens, ctxs, hq // hkv, hkv, cus)}")
    inp = mixed_case(zlib.crc32(name.encode()) % 1000 + 7, hq, hkv, d, qlens, ctxs)
    got = host_f64(gpu_varlen(inp))
    assert_close(got, oracle_varlen(inp), "bf16", name)


def test_varlen_unit_scale_zero_query():
    """q = 0: row r's output is the mean of V over its visible keys (the closed
    form of equal scores; V = a sign pattern plus a token-dependent part of half
    its size, so the means are near unit scale and differ from row to row).
    Dropped or doubled blocks are caught by the peaked sweeps
    (test_gpu_structural)."""
    say("varlen zero-query unit scale")
    inp = mixed_case(41, 32, 8, 128, [100, 1, 37], [700, 1200, 37])
    rng = np.random.default_rng(41)
    sign = np.where(rng.random((8, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    per_token = 0.5 * rng.standard_normal(inp["value_cache"].shape).astype(np.float32)
    inp["value_cache"] = f32_to_bf16_bits(sign[None, None] + per_token)
    inp["q"] = np.zeros_like(inp["q"])
    ref = oracle_varlen(inp)
    assert np.min(np.max(np.abs(ref), axis=-1)) > 0.5
    assert_close(host_f64(gpu_varlen(inp)), ref, "bf16", "zero-query")


def test_varlen_poisoned_unused_memory_changes_nothing():
    say("varlen poison")
    inp = mixed_case(43, 32, 8, 128, [20, 1, 5], [530, 300, 17], spare=9)
    clean = host(gpu_varlen(inp))
    used = np.zeros((inp["num_blocks"], 16), bool)
    for s, c in enumerate(inp["context_lens"]):
        for jj in range(c):
            used[inp["block_tables"][s, jj // 16], jj % 16] = True
    kc, vc = inp["key_cache"].copy(), inp["value_cache"].copy()
    kc[~used] = np.uint16(0x7F80)
    vc[~used] = np.uint16(0x7FC0)
    got = host(gpu_varlen(inp, kc=dev(kc), vc=dev(vc)))
    assert got.tobytes() == clean.tobytes()


def test_varlen_one_row_sequences_equal_decode():
    """All sequences with one query row: the decode path, bit for bit."""
    say("varlen decode rows == decode")
    ctx = [1, 15, 600, 2000, 513, 4000]
    inp = mixed_case(45, 32, 8, 128, [1] * len(ctx), ctx)
    a = host(gpu_varlen(inp))
    q = dev(inp["q"])
    out = torch.empty_like(q)
    pkv.pkv_attention_decode(out, q, dev(inp["key_cache"]), dev(inp["value_cache"]),
                             dev(inp["block_tables"]), dev(inp["context_lens"]), float(inp["scale"]),
                             max(ctx))
    torch.cuda.synchronize()
    assert a.tobytes() == host(out).tobytes()


def test_varlen_rows_past_context_are_zero():
    """More query rows than keys: rows that see no key get zeros; row r >= 4 of a
    10-row chunk over 6 keys sees keys 0 .. r - 4 (the decode of that prefix)."""
    say("varlen q > ctx")
    inp = mixed_case(47, 8, 8, 64, [10, 1], [6, 30])
    got = host_f64(gpu_varlen(inp))
    assert np.all(got[:4] == 0)
    keys = np.arange(4, 10) - 3
    ref = oracle.decode_attention(inp["q"][4:10], inp["key_cache"], inp["value_cache"],
                                  np.repeat(inp["block_tables"][:1], 6, 0), keys, inp["scale"])
    assert_close(got[4:10], ref, "bf16", "rows with keys")


def test_varlen_full_size_mixed_step_sampled():
    spec = SPECS["mixed_chunk512_ctx4096_gqa32x8_bf16_s192"]
    seed = 1004
    say(f"full-size mixed step {spec.name}")
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    dec_ctx = draw_context_lens(rng, spec)
    ctx = np.concatenate([[spec.chunk_ctx], dec_ctx]).astype(np.int32)
    qlens = np.concatenate([[spec.chunk_rows], np.ones(len(dec_ctx), np.int32)]).astype(np.int32)
    nb = pool_blocks_for(spec, ctx)
    tables = random_block_tables(rng, ctx, nb, spec.max_blocks_per_seq)
    T = int(qlens.sum())
    inp = {
        "context_lens": ctx, "block_tables": tables, "num_blocks": nb,
        "qsl": np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32),
        "key_cache": normal_values_parallel(seed * 10 + 1, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "value_cache": normal_values_parallel(seed * 10 + 2, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "q": normal_values_parallel(seed * 10 + 3, (T, Hq, D), "bf16"),
        "scale": np.float32(1.0 / math.sqrt(D)),
        "max_query_len": int(qlens.max()),
    }
    got = host_f64(gpu_varlen(inp))
    again = host_f64(gpu_varlen(inp))
    assert np.array_equal(got, again), "two runs differ"
    # prefill rows: row r sees keys 0 .. 3584 + r, the decode of a truncated context
    rows = np.array([0, 1, 15, 16, 100, 255, 256, 300, 447, 510, 511])
    keys = spec.chunk_ctx - spec.chunk_rows + rows + 1
    ref = oracle.decode_attention(inp["q"][rows], inp["key_cache"], inp["value_cache"],
                                  np.repeat(tables[:1], len(rows), 0), keys, inp["scale"])
    assert_close(got[rows], ref, "bf16", "prefill rows")
    seqs = np.unique(np.concatenate([np.argsort(dec_ctx)[[0, -1]], rng.choice(len(dec_ctx), 6, replace=False)])) + 1
    dref = oracle.decode_attention(inp["q"][inp["qsl"][seqs]], inp["key_cache"], inp["value_cache"],
                                   tables[seqs], ctx[seqs], inp["scale"])
    assert_close(got[inp["qsl"][seqs]], dref, "bf16", "decode rows")


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64), (32, 32, 128)])
def test_varlen_long_chunk_many_items_per_cu_sampled(Hq, Hkv, D):
    """A 2048-row chunk over 8192 keys: prefill items of 256/G rows x the G q
    heads of a KV head over two partitions, four to eight per compute unit
    (GQA 32/8 D 128: 2048 items; GQA 16/2 D 64, whose waves split the K and V
    loads between them: 1024; MHA 32 D 128: 2048), so each workgroup's load
    stream runs across item boundaries many times.  Rows at item edges and the
    causal end are compared with the oracle on their truncated contexts; two
    runs agree bit for bit."""
    C, CC = 2048, 8192
    rng = np.random.default_rng(2048 + D + Hkv)
    ctx = np.array([CC], np.int32)
    nb = CC // BLOCK_SIZE + 16
    tables = rng.permutation(nb)[:CC // BLOCK_SIZE].astype(np.int32)[None, :]
    inp = {
        "context_lens": ctx, "block_tables": tables, "num_blocks": nb,
        "qsl": np.array([0, C], np.int32),
        "key_cache": normal_values_parallel(2049, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "value_cache": normal_values_parallel(2050, (nb, BLOCK_SIZE, Hkv, D), "bf16"),
        "q": normal_values_parallel(2051, (C, Hq, D), "bf16"),
        "scale": np.float32(1.0 / math.sqrt(D)),
        "max_query_len": C,
    }
    say(f"varlen long chunk: {C} rows over {CC} keys, Hq {Hq} Hkv {Hkv} D {D}")
    got = host_f64(gpu_varlen(inp))
    again = host_f64(gpu_varlen(inp))
    assert np.array_equal(got, again), "two runs differ"
    rows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, 1023, 1024, 1535, 1536, 2046, 2047])
    keys = CC - C + rows + 1
    ref = oracle.decode_attention(inp["q"][rows], inp["key_cache"], inp["value_cache"],
                                  np.repeat(tables, len(rows), 0), keys, inp["scale"])
    assert_close(got[rows], ref, "bf16", "long chunk rows")


@pytest.mark.parametrize("order", ["decode_first", "prefill_first"])
def test_varlen_launches_one_by_one_equal_one_call(order):
    """pkv_attention_varlen's four launches made one by one (plan, the decode
    partitions and the prefill tiles in either order, merge) give the one-call
    output byte for byte on a mixed batch (a 300-row chunk over 2600 keys and
    decode rows of 1..3000 keys), which matches the oracle on sampled rows."""
    Hq, Hkv, D = 32, 8, 128
    rng = np.random.default_rng(7 if order == "decode_first" else 8)
    S, C, MB = 12, 300, 200
    ctx = rng.integers(1, 3001, size=S).astype(np.int32)
    ctx[0] = 2600
    qlens = np.array([C] + [1] * (S - 1), np.int32)
    qsl_h = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl_h[-1])
    nb = S * MB + 4
    tables = np.full((S, MB), -1, np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    off = 0
    for s in range(S):
        n = -(-int(ctx[s]) // 16)
        tables[s, :n] = perm[off:off + n]
        off += n
    kc_h = normal_values_parallel(11, (nb, BLOCK_SIZE, Hkv, D), "bf16")
    vc_h = normal_values_parallel(12, (nb, BLOCK_SIZE, Hkv, D), "bf16")
    q_h = normal_values(rng, (T, Hq, D), "bf16")
    kc, vc, q = dev(kc_h), dev(vc_h), dev(q_h)
    tab, lens, qsl = dev(tables), dev(ctx), dev(qsl_h)
    bound = 16 * MB
    scale = float(np.float32(1.0 / math.sqrt(D)))
    say(f"varlen one by one ({order}): chunk {C} rows over {ctx[0]} keys, {S - 1} decode rows")
    ws1 = pkv.varlen_workspace(S, T, Hq, Hkv, D, C, bound)
    ref = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pkv.pkv_attention_varlen(ref, q, kc, vc, tab, lens, qsl, scale, C, bound, workspace=ws1)
    ws2 = pkv.varlen_workspace(S, T, Hq, Hkv, D, C, bound)
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    args = (out, q, kc, vc, tab, lens, qsl, scale, C, bound)
    pkv.pkv_attention_varlen_plan(*args, workspace=ws2)
    middle = [pkv.pkv_attention_varlen_decode_partitions, pkv.pkv_attention_varlen_prefill_tiles]
    for fn in (middle if order == "decode_first" else middle[::-1]):
        fn(*args, workspace=ws2)
    pkv.pkv_attention_varlen_merge(*args, workspace=ws2)
    torch.cuda.synchronize()
    assert host(out).tobytes() == host(ref).tobytes()
    got = host_f64(out)
    rows = np.array([0, 1, C // 2, C - 1])               # chunk rows: row r sees ctx[0] - C + r + 1 keys
    ref = oracle.decode_attention(q_h[rows], kc_h, vc_h, np.repeat(tables[:1], len(rows), 0),
                                  ctx[0] - C + rows + 1, np.float32(scale))
    assert_close(got[rows], ref, "bf16", "one by one: chunk rows")
    seqs = np.arange(1, S)
    dref = oracle.decode_attention(q_h[qsl_h[seqs]], kc_h, vc_h, tables[seqs], ctx[seqs], np.float32(scale))
    assert_close(got[qsl_h[seqs]], dref, "bf16", "one by one: decode rows")


def test_varlen_plan_upload_equals_one_call():
    """Two steps of a mixed batch (a 100-row chunk and decode rows) through
    pkv_attention_varlen_plan_upload (plan from pinned lengths; slots and lengths
    uploaded as bytes, tables by rows), pkv_write of the uploaded slots and
    pkv_attention_varlen_partitions: the device metadata equals the staging,
    outputs equal the one-call varlen on a second copy of the pools byte for
    byte, both pools equal the pool the oracle's writes build, and sampled rows
    match the oracle on that pool."""
    Hq, Hkv, D = 32, 8, 128
    rng = np.random.default_rng(91)
    S, C = 21, 100
    MB = 200
    nb = S * MB + 8
    T = C + S - 1
    kc0 = normal_values_parallel(92, (nb, BLOCK_SIZE, Hkv, D), "bf16")
    vc0 = normal_values_parallel(93, (nb, BLOCK_SIZE, Hkv, D), "bf16")
    kc, vc = dev(kc0), dev(vc0)
    kc2, vc2 = kc.clone(), vc.clone()
    exp_k, exp_v = kc0, vc0
    qlens = np.array([C] + [1] * (S - 1), np.int32)
    qsl_h = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    qsl = dev(qsl_h)
    head = T + S + (-(T + S)) % 4                      # slots | lens, padded to 16 bytes
    stage = torch.zeros(head + S * MB, dtype=torch.int32, pin_memory=True)
    dmeta = torch.full((head + S * MB,), -3, dtype=torch.int32, device="cuda")
    bound = 16 * MB
    ws = pkv.varlen_workspace(S, T, Hq, Hkv, D, C, bound)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    for step, (lo, hi) in enumerate([(1, 1500), (300, 3100)]):
        ctx = rng.integers(lo, hi + 1, size=S).astype(np.int32)
        ctx[0] = 700 + 400 * step                       # the chunk's context (its rows are the last C tokens)
        tables = np.full((S, MB), -1, np.int32)
        perm = rng.permutation(nb).astype(np.int32)     # distinct blocks within the step
        off = 0
        for s in range(S):
            n = -(-int(ctx[s]) // 16)
            tables[s, :n] = perm[off:off + n]
            off += n
        pos = np.concatenate([ctx[0] - C + np.arange(C), ctx[1:] - 1])          # rows' own positions
        seq = np.concatenate([np.zeros(C, np.int64), np.arange(1, S)])
        slots = (tables[seq, pos // 16] * 16 + pos % 16).astype(np.int32)
        h = stage.numpy()
        h[:T], h[T:T + S], h[head:] = slots, ctx, tables.reshape(-1)
        q = dev(normal_values(rng, (T, Hq, D), "bf16"))
        kn_h, vn_h = normal_values(rng, (T, Hkv, D), "bf16"), normal_values(rng, (T, Hkv, D), "bf16")
        kn, vn = dev(kn_h), dev(vn_h)
        say(f"varlen plan_upload step {step}: chunk ctx {ctx[0]}, decode ctx {ctx[1:].min()}..{ctx[1:].max()}")
        d_slots, d_lens = dmeta[:T], dmeta[T:T + S]
        d_tab = dmeta[head:].view(S, MB)
        out = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        pkv.pkv_attention_varlen_plan_upload(out, q, kc, vc, d_tab, d_lens, qsl, scale, C, bound, stage[T:T + S],
                                             stage[:head], dmeta[:head], workspace=ws,
                                             host_block_tables=stage[head:].view(S, MB))
        pkv.pkv_write(kc, vc, kn, vn, d_slots)
        pkv.pkv_attention_varlen_partitions(out, q, kc, vc, d_tab, d_lens, qsl, scale, C, bound, workspace=ws)
        ref = torch.full_like(out, float("nan"))
        pkv.pkv_write(kc2, vc2, kn, vn, dev(slots))
        pkv.pkv_attention_varlen(ref, q, kc2, vc2, dev(tables), dev(ctx), qsl, scale, C, bound)
        torch.cuda.synchronize()
        got_meta = host(dmeta)
        assert got_meta[:T + S].tobytes() == h[:T + S].tobytes(), "slots / lengths differ from the staging"
        gt = got_meta[head:].reshape(S, MB)
        for s in range(S):
            n = -(-int(ctx[s]) // 16)
            assert np.array_equal(gt[s, :n], tables[s, :n]), s
        assert host(out).tobytes() == host(ref).tobytes(), f"step {step}: differs from the one-call varlen"
        exp_k, exp_v = oracle.write_kv(exp_k, exp_v, kn_h, vn_h, slots)
        assert host(kc).tobytes() == exp_k.tobytes() and host(vc).tobytes() == exp_v.tobytes()
        assert host(kc2).tobytes() == exp_k.tobytes() and host(vc2).tobytes() == exp_v.tobytes()
        rows = np.unique(np.concatenate([[0, 1, 50, C - 1], C + rng.choice(S - 1, 5, replace=False)]))
        want = oracle.causal_chunk_attention(host(q), exp_k, exp_v, tables, ctx, qsl_h, np.float32(scale))
        assert_close(host_f64(out)[rows], want[rows], "bf16", f"varlen plan_upload step {step}")
        torch.cuda.synchronize()                        # the staging is rewritten for the next step
