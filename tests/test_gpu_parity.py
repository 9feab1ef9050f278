"""GPU parity: the HIP path through the C ABI against the CPU oracle (gfx950 only).

Integer/byte work (slot write, block copy) must match bit for bit over the whole
pool.  Attention must meet the fp32 / bf16 bars of ``gpu_util``.  Cases span
several 16-token blocks and 512-token partitions with ragged tails, every GQA
group size built (1, 2, 4, 8), both head dims (64, 128) and both dtypes.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import (BLOCK_SIZE, SPECS, make_decode_inputs, normal_values,
                       random_block_tables)

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None


def explicit_case(seed, dtype, Hq, Hkv, D, ctx, spare_blocks=5, table_fill=-1):
    """Seeded inputs with the given context lengths (generator functions only)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    nb = int(sum(-(-c // BLOCK_SIZE) for c in ctx)) + spare_blocks
    mb = max(1, int(-(-ctx.max() // BLOCK_SIZE)) + 2)
    tables = random_block_tables(rng, ctx, nb, mb, fill=table_fill)
    S = len(ctx)
    return {
        "dtype": dtype, "context_lens": ctx, "block_tables": tables, "num_blocks": nb,
        "key_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype),
        "value_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dtype),
        "q": normal_values(rng, (S, Hq, D), dtype),
        "scale": np.float32(1.0 / math.sqrt(D)),
    }


def gpu_decode(inp, kc=None, vc=None, q=None, tables=None, ctx=None):
    q = dev(inp["q"]) if q is None else q
    kc = dev(inp["key_cache"]) if kc is None else kc
    vc = dev(inp["value_cache"]) if vc is None else vc
    tables = dev(inp["block_tables"]) if tables is None else tables
    ctx_h = inp["context_lens"]
    ctx = dev(ctx_h) if ctx is None else ctx
    out = torch.empty_like(q)
    pkv.pkv_attention_decode(out, q, kc, vc, tables, ctx, float(inp["scale"]), int(ctx_h.max(initial=0)))
    torch.cuda.synchronize()
    return out


def oracle_decode(inp, seqs=None):
    idx = np.arange(len(inp["context_lens"])) if seqs is None else np.asarray(seqs)
    return oracle.decode_attention(inp["q"][idx], inp["key_cache"], inp["value_cache"],
                                   inp["block_tables"][idx], inp["context_lens"][idx], inp["scale"])


# ------------------------------------------------------------------ write / copy
@pytest.mark.parametrize("dtype,nb,hkv,d,t", [
    ("f32", 64, 8, 64, 4),
    ("bf16", 400, 8, 128, 128),
    ("bf16", 300, 32, 128, 64),
    ("f32", 50, 2, 128, 37),
])
def test_write_whole_pool_bitexact(dtype, nb, hkv, d, t):
    say(f"write {dtype} nb={nb} hkv={hkv} d={d} t={t}")
    rng = np.random.default_rng(nb + t)
    kc = normal_values(rng, (nb, 16, hkv, d), dtype)
    vc = normal_values(rng, (nb, 16, hkv, d), dtype)
    k = normal_values(rng, (t, hkv, d), dtype)
    v = normal_values(rng, (t, hkv, d), dtype)
    slots = rng.choice(nb * 16, size=t, replace=False).astype(np.int32)
    slots[::7] = -1                                  # padding tokens are skipped
    slots[1] = nb * 16 + 5                           # beyond the pool: skipped
    kc_d, vc_d = dev(kc), dev(vc)
    pkv.pkv_write(kc_d, vc_d, dev(k), dev(v), dev(slots))
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[ok >= nb * 16] = -1
    kr, vr = oracle.write_kv(kc, vc, k, v, ok)
    assert host(kc_d).tobytes() == kr.tobytes()
    assert host(vc_d).tobytes() == vr.tobytes()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_blocks_bitexact(dtype):
    say(f"copy_blocks {dtype}")
    rng = np.random.default_rng(3)
    nb = 40
    kc = normal_values(rng, (nb, 16, 8, 128), dtype)
    vc = normal_values(rng, (nb, 16, 8, 128), dtype)
    pairs = np.array([[1, 30], [2, 31], [17, 5], [39, 0]], np.int32)
    bad = np.array([[1, nb], [-3, 4]], np.int32)     # out-of-range ids are skipped
    kc_d, vc_d = dev(kc), dev(vc)
    pkv.pkv_copy_blocks(kc_d, vc_d, dev(np.concatenate([pairs, bad])))
    torch.cuda.synchronize()
    kr, vr = oracle.copy_blocks(kc, vc, pairs)
    assert host(kc_d).tobytes() == kr.tobytes()
    assert host(vc_d).tobytes() == vr.tobytes()


# ------------------------------------------------------------- decode parity
DECODE_CASES = {
    # name: (dtype, Hq, Hkv, D, context lengths)
    "mha_d128_bf16": ("bf16", 32, 32, 128, [1, 15, 16, 17, 511, 512, 513, 1500, 2048]),
    "mha_d128_f32": ("f32", 32, 32, 128, [1, 15, 16, 17, 511, 512, 513, 1500, 2048]),
    "gqa4_d128_bf16": ("bf16", 32, 8, 128, [1, 33, 512, 513, 1024, 2047, 3000, 5000]),
    "gqa4_d128_f32": ("f32", 32, 8, 128, [1, 33, 512, 513, 1024, 2047, 3000, 5000]),
    "mha_d64_f32": ("f32", 8, 8, 64, [3, 64, 100, 700, 1025]),
    "mha_d64_bf16": ("bf16", 8, 8, 64, [3, 64, 100, 700, 1025]),
    "gqa2_d64_bf16": ("bf16", 8, 4, 64, [2, 31, 530, 1600]),
    "gqa2_d128_f32": ("f32", 8, 4, 128, [2, 31, 530, 1600]),
    "gqa8_d128_bf16": ("bf16", 16, 2, 128, [5, 260, 777, 2100]),
    "gqa8_d64_f32": ("f32", 16, 2, 64, [5, 260, 777, 2100]),
    "gqa4_d64_bf16": ("bf16", 16, 4, 64, [1, 16, 48, 4097]),
    # around the context at which a sequence's items grow from two partitions
    # to four (nine partitions: more than 4096 tokens), with ragged last items
    "item_size_edges_bf16": ("bf16", 32, 8, 128, [4096, 4097, 4607, 4608, 4609, 6144, 6145, 8193]),
    # long contexts: more than 64 partial results in a row (the merge's
    # lane-parallel maxima then take a second round), thousands of table entries
    "long_gqa4_d64_bf16": ("bf16", 8, 2, 64, [70000, 40961, 3]),
    # 256 partitions in one row (four-partition items throughout), beside a
    # sequence one token past a partition edge and a one-token sequence
    "very_long_gqa4_d64_bf16": ("bf16", 4, 1, 64, [131072, 65537, 1]),
    "very_long_gqa4_d64_f32": ("f32", 4, 1, 64, [131072, 1]),
    "long_gqa4_d64_f32": ("f32", 8, 2, 64, [35000, 33]),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_matches_oracle(name):
    dtype, hq, hkv, d, ctx = DECODE_CASES[name]
    say(f"decode {name}: hq={hq} hkv={hkv} d={d} ctx={ctx}")
    inp = explicit_case(zlib.crc32(name.encode()) % 1000, dtype, hq, hkv, d, ctx)
    got = host_f64(gpu_decode(inp))
    assert_close(got, oracle_decode(inp), dtype, name)


@pytest.mark.parametrize("seed", range(1000, 1010))
def test_tiny_write_then_decode(seed):
    """Tiny fp32 MHA batch: write each sequence's new token, then attend (it sees itself)."""
    spec = SPECS["tiny_f32_mha_s4_h8_d64"]
    say(f"tiny flow seed={seed}")
    inp = make_decode_inputs(spec, seed)
    ctx, tables = inp["context_lens"], inp["block_tables"]
    slots = np.array([oracle.slot_for_position(tables[s], int(ctx[s]) - 1)
                      for s in range(spec.num_seqs)], np.int32)
    kr, vr = oracle.write_kv(inp["key_cache"], inp["value_cache"], inp["k_new"], inp["v_new"], slots)
    ref = oracle.decode_attention(inp["q"], kr, vr, tables, ctx, inp["scale"])
    kc, vc = dev(inp["key_cache"]), dev(inp["value_cache"])
    pkv.pkv_write(kc, vc, dev(inp["k_new"]), dev(inp["v_new"]), dev(slots))
    out = gpu_decode(inp, kc=kc, vc=vc)
    assert host(kc).tobytes() == kr.tobytes() and host(vc).tobytes() == vr.tobytes()
    assert_close(host_f64(out), ref, "f32", f"tiny seed {seed}")


# -------------------------------------------------------- closed forms, edges
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_token_context_is_exact(dtype):
    say(f"one-token {dtype}")
    inp = explicit_case(5, dtype, 32, 8, 128, [1] * 6)
    got = host(gpu_decode(inp))
    for s in range(6):
        b = inp["block_tables"][s, 0]
        want = np.repeat(inp["value_cache"][b, 0], 4, axis=0)   # q head h reads KV head h // 4
        assert got[s].tobytes() == want.tobytes()


def test_zero_query_unit_scale_bf16():
    """q = 0: uniform weights, out = the mean of V over the context (the closed
    form of equal scores).  V = a sign pattern per (KV head, dim) plus a
    token-dependent part of half its size, so the mean stays near unit scale
    and still depends on which tokens are summed.  At long contexts one
    block's share of a uniform mean is too small for the bf16 bars; dropped or
    doubled blocks are caught by the peaked sweeps (test_gpu_structural)."""
    say("zero-query unit scale")
    inp = explicit_case(6, "bf16", 32, 8, 128, [1, 17, 600, 2000, 4500])
    rng = np.random.default_rng(6)
    sign = np.where(rng.random((8, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    per_token = 0.5 * rng.standard_normal(inp["value_cache"].shape).astype(np.float32)
    from workloads import f32_to_bf16_bits
    inp["value_cache"] = f32_to_bf16_bits(sign[None, None] + per_token)
    inp["q"] = np.zeros_like(inp["q"])
    got = host_f64(gpu_decode(inp))
    ref = oracle_decode(inp)
    assert np.min(np.max(np.abs(ref), axis=-1)) > 0.5
    assert_close(got, ref, "bf16", "zero-query")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaky_query_selects_token(dtype):
    """q aligned with one key: the softmax collapses onto that token's V (unit scale)."""
    n = 1300
    js = [0, 15, 16, 511, 512, 1023, 1024, 1299]
    say(f"peaky {dtype}")
    inp = explicit_case(7, dtype, 8, 8, 128, [n] * len(js))
    kf = oracle.widen(inp["key_cache"])
    q = np.zeros((len(js), 8, 128))
    for s, j in enumerate(js):
        k = kf[inp["block_tables"][s, j // 16], j % 16]          # [Hkv, D]
        q[s] = 60.0 * k / np.linalg.norm(k, axis=1, keepdims=True)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        inp["q"] = f32_to_bf16_bits(q.astype(np.float32))
    else:
        inp["q"] = q.astype(np.float32)
    got = host_f64(gpu_decode(inp))
    ref = oracle_decode(inp)
    assert_close(got, ref, dtype, "peaky")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_poisoned_unused_memory_changes_nothing(dtype):
    """NaN/Inf in unused slots and free blocks, garbage table tails: output bitwise unchanged."""
    say(f"poison {dtype}")
    inp = explicit_case(8, dtype, 32, 8, 128, [3, 17, 512, 700, 1999], spare_blocks=9)
    clean = host(gpu_decode(inp))
    kc, vc = inp["key_cache"].copy(), inp["value_cache"].copy()
    used = np.zeros((inp["num_blocks"], 16), bool)
    for s, c in enumerate(inp["context_lens"]):
        for j in range(c):
            used[inp["block_tables"][s, j // 16], j % 16] = True
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    inf = np.uint16(0x7F80) if dtype == "bf16" else np.float32(np.inf)
    kc[~used] = inf
    vc[~used] = nan
    tables = inp["block_tables"].copy()
    tables[tables == -1] = 2 ** 30                       # never dereferenced
    got = host(gpu_decode(inp, kc=dev(kc), vc=dev(vc), tables=dev(tables)))
    assert got.tobytes() == clean.tobytes()


def test_deterministic_and_renaming_invariant():
    """Two runs are bitwise equal, and renaming physical blocks changes no bit."""
    say("determinism / renaming")
    inp = explicit_case(9, "bf16", 32, 8, 128, [40, 513, 1100, 3000], spare_blocks=0)
    a = host(gpu_decode(inp))
    b = host(gpu_decode(inp))
    assert a.tobytes() == b.tobytes()
    perm = np.random.default_rng(9).permutation(inp["num_blocks"])
    kc = np.empty_like(inp["key_cache"]); kc[perm] = inp["key_cache"]
    vc = np.empty_like(inp["value_cache"]); vc[perm] = inp["value_cache"]
    t = inp["block_tables"]
    tables = np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
    c = host(gpu_decode(inp, kc=dev(kc), vc=dev(vc), tables=dev(tables)))
    assert c.tobytes() == a.tobytes()


def test_empty_context_gives_zero():
    say("empty context")
    inp = explicit_case(10, "bf16", 32, 8, 128, [0, 100, 0, 900])
    got = host_f64(gpu_decode(inp))
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_close(got[[1, 3]], oracle_decode(inp, [1, 3]), "bf16", "nonempty rows")


def test_gqa_equals_repeated_mha_on_gpu():
    say("gqa == repeated mha")
    inp = explicit_case(11, "f32", 32, 8, 128, [77, 600, 1800])
    a = host_f64(gpu_decode(inp))
    rep = dict(inp)
    rep["key_cache"] = np.repeat(inp["key_cache"], 4, axis=2)
    rep["value_cache"] = np.repeat(inp["value_cache"], 4, axis=2)
    b = host_f64(gpu_decode(rep))
    assert_close(a, b, "f32", "gqa vs mha")


# ------------------------------------------------------------------ LSE merge
@pytest.mark.parametrize("dtype,d,maxp", [("f32", 128, 9), ("bf16", 128, 9), ("f32", 64, 9),
                                          ("f32", 128, 70), ("bf16", 64, 70)])
def test_lse_merge_isolated(dtype, d, maxp):
    say(f"lse merge {dtype} d={d} maxp={maxp}")
    rng = np.random.default_rng(12 + maxp)
    rows = 40
    counts = rng.integers(0, maxp + 1, rows).astype(np.int32)
    counts[0], counts[1] = 1, maxp
    pm = np.full((rows, maxp), -np.inf)
    pl = np.zeros((rows, maxp))
    po = np.zeros((rows, maxp, d))
    ref = np.zeros((rows, d))
    for r in range(rows):
        n = int(counts[r]) * 37 + 5
        x = rng.standard_normal(n) * 4
        V = rng.standard_normal((n, d))
        m, l, o = oracle.split_decode_partials(x, V, 37)
        m, l, o = m[:counts[r]], l[:counts[r]], o[:counts[r]]
        if counts[r] > 2:                                   # an empty partial in the middle
            m[1], l[1], o[1] = -np.inf, 0.0, np.nan
        pm[r, :counts[r]], pl[r, :counts[r]], po[r, :counts[r]] = m, l, o
        ref[r] = oracle.merge_partials(m, l, o)
    out = torch.empty((rows, d), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    pkv.pkv_lse_merge(out, dev((pm / math.log(2)).astype(np.float32)), dev(pl.astype(np.float32)),
                      dev(po.astype(np.float32)), dev(counts))
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.all(got[counts == 0] == 0)
    live = counts > 0
    # inputs were rounded to fp32 before the merge; the bar is the fp32/bf16 one
    assert_close(got[live], ref[live], dtype, "merge")


def test_three_call_form_equals_one_call():
    """plan, partitions and merge called one at a time (plan on its own stream,
    ordered by an event) give the one-call result bit for bit."""
    say("plan / partitions / merge")
    inp = explicit_case(13, "bf16", 32, 8, 128, [40, 513, 1100, 3000, 7])
    ref = host(gpu_decode(inp))
    q, kc, vc = dev(inp["q"]), dev(inp["key_cache"]), dev(inp["value_cache"])
    tables, ctx = dev(inp["block_tables"]), dev(inp["context_lens"])
    mx = int(inp["context_lens"].max())
    out = torch.empty_like(q)
    ws = pkv.decode_workspace(5, 32, 128, mx)
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    with torch.cuda.stream(side):
        pkv.pkv_attention_decode_plan(out, q, kc, vc, tables, ctx, float(inp["scale"]), mx, workspace=ws,
                                      stream=side)
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    pkv.pkv_attention_decode_partitions(out, q, kc, vc, tables, ctx, float(inp["scale"]), mx, workspace=ws)
    pkv.pkv_attention_decode_merge(out, q, kc, vc, tables, ctx, float(inp["scale"]), mx, workspace=ws)
    torch.cuda.synchronize()
    assert host(out).tobytes() == ref.tobytes()


def test_decode_more_sequences_than_plan_threads():
    """2500 sequences (more than the plan workgroup's 1024 threads, so each
    thread plans several), contexts 1..1200: sampled rows against the oracle,
    and the fused upload + plan launch (row-wise tables from pinned memory)
    gives the same bytes as the one-call decode."""
    rng = np.random.default_rng(77)
    S, Hq, Hkv, D = 2500, 8, 2, 64
    ctx = rng.integers(1, 1201, size=S).astype(np.int32)
    say(f"decode S={S} ctx 1..1200 (plan threads handle several sequences)")
    inp = explicit_case(78, "bf16", Hq, Hkv, D, ctx)
    got_t = gpu_decode(inp)
    got = host_f64(got_t)
    idx = np.unique(np.concatenate([np.argsort(ctx)[:3], np.argsort(ctx)[-3:], rng.choice(S, 34, replace=False)]))
    assert_close(got[idx], oracle_decode(inp, idx), "bf16", "decode S=2500")
    # the same step through the fused upload + plan launch
    tables = inp["block_tables"]
    MB = tables.shape[1]
    bound = int(ctx.max())
    stage_t = torch.from_numpy(np.ascontiguousarray(tables)).pin_memory()
    lens_h = torch.from_numpy(ctx.copy()).pin_memory()
    dummy = torch.zeros(4, dtype=torch.int32).pin_memory()
    d_tab = torch.full((S, MB), -5, dtype=torch.int32, device="cuda")
    d_lens = torch.zeros(S, dtype=torch.int32, device="cuda")
    d_dummy = torch.zeros(4, dtype=torch.int32, device="cuda")
    q, kc, vc = dev(inp["q"]), dev(inp["key_cache"]), dev(inp["value_cache"])
    out = torch.empty_like(q)
    ws = pkv.decode_workspace(S, Hq, D, bound)
    scale = float(inp["scale"])
    d_lens.copy_(dev(ctx))
    pkv.pkv_attention_decode_plan_upload(out, q, kc, vc, d_tab, d_lens, scale, bound, lens_h, dummy, d_dummy,
                                         workspace=ws, host_block_tables=stage_t)
    pkv.pkv_attention_decode_partitions(out, q, kc, vc, d_tab, d_lens, scale, bound, workspace=ws)
    pkv.pkv_attention_decode_merge(out, q, kc, vc, d_tab, d_lens, scale, bound, workspace=ws)
    torch.cuda.synchronize()
    assert host(out).tobytes() == host(got_t).tobytes()
