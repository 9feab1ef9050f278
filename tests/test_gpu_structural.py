"""Structural parity on the GPU: checks that fail on a dropped, doubled or
misplaced block, a short causal mask or wrong merge weights.

Inputs come from ``structural_checks``: every output row is peaked on one
target token that carries half its softmax mass (over the rows every block of
a context is a target, at varying offsets, with the last token and each chunk
row's causal edge among them), or saturated on three tied keys in two
partitions.  Outputs are unit scale, so the bf16 bars (2e-2 absolute and
row-relative) are tight against such mistakes: the CPU tests in
``test_structural_pins`` show each kind, planted in the oracle, misses them by
more than five times.  Every call goes through the C ABI; expected values come
from the oracle ("vLLM and PagedAttention", §2 "Reworking the Attention
Computation": per-block attention through the block table, accumulated).

Cases: the one-call decode at context 8192 (GQA 32/8 with every block a target
of every KV head, and MHA with the heads tiling the blocks), D = 64 with G = 8,
and fp32 on the vector-ALU kernel; the decode loop exactly as bench.py runs it
(fused upload + plan with the previous step's merge riding along, the append
form writing each step's new token, which is a target, over slots poisoned with
NaN before they are written); chunked prefill at the mixed-step shape alone and
with its 192 decode rows, and at shapes whose rows cross 512-key edges and
whose items span two partitions; tied keys for decode (bf16 and fp32) and for
chunk rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import structural_checks as sc
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import SPECS, draw_context_lens, normal_values_parallel, pool_blocks_for

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None


def gpu_decode(inp):
    q = dev(inp["q"])
    out = torch.full_like(q, float("nan"))
    ctx = inp["context_lens"]
    pkv.pkv_attention_decode(out, q, dev(inp["key_cache"]), dev(inp["value_cache"]), dev(inp["block_tables"]),
                             dev(ctx), float(inp["scale"]), int(ctx.max()))
    torch.cuda.synchronize()
    return host_f64(out)


def gpu_varlen(inp):
    q = dev(inp["q"])
    out = torch.full_like(q, float("nan"))
    ctx = inp["context_lens"]
    pkv.pkv_attention_varlen(out, q, dev(inp["key_cache"]), dev(inp["value_cache"]), dev(inp["block_tables"]),
                             dev(ctx), dev(inp["qsl"]), float(inp["scale"]), inp["max_query_len"], int(ctx.max()))
    torch.cuda.synchronize()
    return host_f64(out)


def oracle_decode(inp):
    return oracle.decode_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                   inp["context_lens"], inp["scale"])


def oracle_varlen(inp):
    return oracle.causal_chunk_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                         inp["context_lens"], inp["qsl"], inp["scale"])


def unit_scale(ref):
    return float(np.min(np.max(np.abs(ref), axis=-1)))


SWEEPS = {
    # name: (seed, S, Hq, Hkv, D, ctx, dtype)
    "gqa32x8_d128_ctx8192_bf16": (31, 128, 32, 8, 128, 8192, "bf16"),   # every block x every KV head
    "mha8_d128_ctx8192_bf16": (32, 64, 8, 8, 128, 8192, "bf16"),        # the 8 heads tile the 512 blocks
    "gqa16x2_d64_ctx4096_bf16": (33, 32, 16, 2, 64, 4096, "bf16"),      # G = 8, every block x every KV head
    "gqa32x8_d128_ctx2048_f32": (34, 32, 32, 8, 128, 2048, "f32"),      # the vector-ALU kernel, fp32 bar
}


@pytest.mark.parametrize("name", sorted(SWEEPS))
def test_peaked_sweep_decode(name):
    seed, S, Hq, Hkv, D, ctx, dtype = SWEEPS[name]
    say(f"peaked decode sweep {name}")
    inp = sc.peaked_decode_case(seed, S, Hq, Hkv, D, ctx, dtype)
    ref = oracle_decode(inp)
    assert unit_scale(ref) > 0.3
    assert_close(gpu_decode(inp), ref, dtype, f"peaked decode {name}")


def test_peaked_sweep_bench_decode_loop():
    """The bench's decode loop at its workload's shape (128 sequences, GQA 32/8,
    contexts log-uniform in [512, 8192]) for three steps of growth: per step the
    fused upload + plan from pinned staging (tables by rows; the previous
    step's merge riding along; workspaces alternating) and the append-form
    partitions, which read each sequence's new token from k_new / v_new and
    store it.  The new tokens' slots hold NaN before their step.  Head 0 of
    every sequence targets that step's new token; the other heads sweep the
    blocks.  Every step's output matches the oracle over the pool as the
    oracle's write leaves it, and the final pool equals that pool byte for
    byte."""
    spec = SPECS["gqa32x8_bf16_s128_ctx512_8192"]
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    steps = 3
    rng = np.random.default_rng(1002)
    ctx0 = draw_context_lens(rng, spec).astype(np.int64)
    final = ctx0 + steps - 1
    nb = pool_blocks_for(spec, final)
    tables = sc.scattered_tables(rng, final, nb, shared=False)
    MB = tables.shape[1]
    bound = 16 * MB
    say(f"peaked bench decode loop S={S} nb={nb} MB={MB} steps={steps}")
    kc0 = normal_values_parallel(41, (nb, 16, Hkv, D), "bf16")
    vc0 = normal_values_parallel(42, (nb, 16, Hkv, D), "bf16")
    slots = [np.array([tables[s, (c - 1) // 16] * 16 + (c - 1) % 16 for s, c in enumerate(ctx0 + i)], np.int32)
             for i in range(steps)]
    for sl in slots:                                   # the tokens to come: NaN until written
        kc0.reshape(-1, Hkv, D)[sl] = np.uint16(0x7FC0)
        vc0.reshape(-1, Hkv, D)[sl] = np.uint16(0x7FC0)
    kn = normal_values_parallel(43, (steps, S, Hkv, D), "bf16")
    vn = normal_values_parallel(44, (steps, S, Hkv, D), "bf16")
    exp_k, exp_v, qs = [], [], []
    k, v = kc0, vc0
    for i in range(steps):
        k, v = oracle.write_kv(k, v, kn[i], vn[i], slots[i])
        exp_k.append(k)
        exp_v.append(v)
        ctx_i = (ctx0 + i).astype(np.int32)
        tg = sc.decode_targets(ctx_i, Hq, Hkv, last_token_head0=True)
        q, _ = sc.peaked_decode_queries(k, tables, ctx_i, Hq, tg, "bf16")
        qs.append(q)

    kc, vc = dev(kc0), dev(vc0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    meta_len = 2 * S + S * MB
    meta_len += -meta_len % 4
    stage = [torch.zeros(meta_len, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    dmeta = [torch.zeros(meta_len, dtype=torch.int32, device="cuda") for _ in range(2)]
    wss = [pkv.decode_workspace(S, Hq, D, bound) for _ in range(2)]
    out = [torch.full((S, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    keep = []
    for i in range(steps):
        b = i % 2
        h = stage[b].numpy()
        h[:S] = slots[i]
        h[S:2 * S] = ctx0 + i
        h[2 * S:2 * S + S * MB] = tables.reshape(-1)
        q_d, kn_d, vn_d = dev(qs[i]), dev(kn[i]), dev(vn[i])
        keep.append((q_d, kn_d, vn_d))
        d_lens, d_tab = dmeta[b][S:2 * S], dmeta[b][2 * S:2 * S + S * MB].view(S, MB)
        merge_kw = dict(merge_out=out[i - 1], merge_workspace=wss[1 - b]) if i > 0 else {}
        pkv.pkv_attention_decode_plan_upload(out[i], q_d, kc, vc, d_tab, d_lens, scale, bound, stage[b][S:2 * S],
                                             stage[b][:2 * S], dmeta[b][:2 * S], workspace=wss[b],
                                             host_block_tables=stage[b][2 * S:2 * S + S * MB].view(S, MB),
                                             **merge_kw)
        pkv.pkv_attention_decode_partitions_append(out[i], q_d, kn_d, vn_d, kc, vc, d_tab, d_lens, scale, bound,
                                                   workspace=wss[b])
        torch.cuda.synchronize()                       # the staging set is rewritten two steps later
    last = (steps - 1) % 2
    pkv.pkv_attention_decode_merge(out[-1], keep[-1][0], kc, vc, dmeta[last][2 * S:2 * S + S * MB].view(S, MB),
                                   dmeta[last][S:2 * S], scale, bound, workspace=wss[last])
    torch.cuda.synchronize()
    assert host(kc).tobytes() == exp_k[-1].tobytes(), "K pool differs from the oracle's writes"
    assert host(vc).tobytes() == exp_v[-1].tobytes(), "V pool differs from the oracle's writes"
    for i in range(steps):
        ctx_i = (ctx0 + i).astype(np.int32)
        ref = oracle.decode_attention(qs[i], exp_k[i], exp_v[i], tables, ctx_i, np.float32(scale))
        assert unit_scale(ref) > 0.3
        assert_close(host_f64(out[i]), ref, "bf16", f"peaked bench loop step {i}")


CHUNK_SWEEPS = {
    # name: (seed, Hq, Hkv, D, query lengths, context lengths)
    # the mixed step's chunk alone: 512 rows at positions 3584 .. 4095
    "chunk512_ctx4096_gqa32x8": (51, 32, 8, 128, [512], [4096]),
    # rows that cross 1024- and 2048-key edges; a decode row; items of two partitions
    "edges_gqa32x8": (52, 32, 8, 128, [300, 1, 64, 256], [1300, 2000, 600, 2300]),
    "edges_mha_d64": (53, 32, 32, 64, [256, 256, 100, 1], [2300, 1000, 560, 3000]),
    "edges_gqa8_d64": (54, 32, 4, 64, [200, 33, 1], [2100, 600, 900]),
    # two prefill items per compute unit (512 rows over 8192 keys: 512 items of
    # two partitions), so every workgroup's load stream crosses an item boundary
    "two_items_per_cu_gqa32x8": (55, 32, 8, 128, [512], [8192]),
}


@pytest.mark.parametrize("name", sorted(CHUNK_SWEEPS))
def test_peaked_sweep_chunk(name):
    seed, Hq, Hkv, D, qlens, ctxs = CHUNK_SWEEPS[name]
    say(f"peaked chunk sweep {name}: q={qlens} ctx={ctxs}")
    inp = sc.peaked_chunk_case(seed, Hq, Hkv, D, qlens, ctxs)
    ref = oracle_varlen(inp)
    assert unit_scale(ref) > 0.3
    assert_close(gpu_varlen(inp), ref, "bf16", f"peaked chunk {name}")


def test_peaked_sweep_mixed_step_full_size():
    """The mixed step the bench times: one 512-row chunk at the end of a
    4096-token context batched with 192 decode rows (contexts uniform in
    [256, 4096]), every row peaked; all 704 rows against the oracle."""
    spec = SPECS["mixed_chunk512_ctx4096_gqa32x8_bf16_s192"]
    rng = np.random.default_rng(1004)
    dec = draw_context_lens(rng, spec)
    qlens = [spec.chunk_rows] + [1] * len(dec)
    ctxs = [spec.chunk_ctx] + dec.tolist()
    say(f"peaked mixed step: chunk {spec.chunk_rows} rows + {len(dec)} decode rows")
    inp = sc.peaked_chunk_case(55, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, qlens, ctxs)
    ref = oracle_varlen(inp)
    assert unit_scale(ref) > 0.3
    assert_close(gpu_varlen(inp), ref, "bf16", "peaked mixed step")


TIED_DECODE = {
    # name: (seed, Hq, Hkv, D, context lengths, dtype)
    "gqa32x8_d128_bf16": (61, 32, 8, 128, [514, 1025, 1500, 2048, 3000, 4097, 8192, 6000, 700, 5555], "bf16"),
    "gqa32x8_d128_f32": (62, 32, 8, 128, [514, 1025, 1500, 2048, 3000, 4097, 8192, 6000, 700, 5555], "f32"),
    "mha8_d64_bf16": (63, 8, 8, 64, [600, 1030, 2600, 5000, 8000], "bf16"),
}


@pytest.mark.parametrize("name", sorted(TIED_DECODE))
def test_tied_keys_decode(name):
    seed, Hq, Hkv, D, ctxs, dtype = TIED_DECODE[name]
    say(f"tied keys decode {name}")
    inp = sc.tied_keys_decode_case(seed, Hq, Hkv, D, ctxs, dtype)
    got = gpu_decode(inp)
    assert_close(got, oracle_decode(inp), dtype, f"tied decode {name}")
    assert_close(got, sc.tied_keys_expected(inp), dtype, f"tied decode {name} (closed form)")


def test_tied_keys_chunk():
    say("tied keys chunk rows")
    inp = sc.tied_keys_chunk_case(64, 32, 8, 128, [512, 1, 100, 300, 1], [4096, 3000, 2000, 1300, 8000])
    got = gpu_varlen(inp)
    assert_close(got, oracle_varlen(inp), "bf16", "tied chunk")
    assert_close(got, sc.tied_keys_expected(inp), "bf16", "tied chunk (closed form)")
