"""Pin checks for the attention oracle, written against facts other than the oracle.

Each ``check_*`` takes the decode function under test (signature of
``oracle.decode_attention``) and returns the largest violation it found (0.0 when
the property holds exactly).  ``test_oracle_pins.py`` asserts each is within its
bound for the real oracle; ``test_oracle_mutations.py`` plants plausible mistakes in
a copy of the oracle and asserts that at least one check catches each one.
"""

import itertools
import math

import numpy as np
import torch

BS = 16


def _bf16_exact(x):
    """float64 values that are exactly representable in bf16 (and so in fp32)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def scatter_logical(rng, logical_k, logical_v, num_blocks, mb, fill=-1):
    """Place per-sequence logical K/V into a pool through random block tables.

    Test-local placement (independent of the oracle's write): sequence s's token j
    goes to block tables[s, j // 16], offset j % 16.  Unused slots hold NaN.
    """
    Hkv, D = logical_k[0].shape[1:]
    kc = np.full((num_blocks, BS, Hkv, D), np.nan, dtype=np.float32)
    vc = np.full((num_blocks, BS, Hkv, D), np.nan, dtype=np.float32)
    perm = rng.permutation(num_blocks)
    tables = np.full((len(logical_k), mb), fill, dtype=np.int32)
    off = 0
    for s, (K, V) in enumerate(zip(logical_k, logical_v)):
        n = K.shape[0]
        nb = -(-n // BS)
        tables[s, :nb] = perm[off:off + nb]
        off += nb
        for j in range(n):
            kc[tables[s, j // BS], j % BS] = K[j]
            vc[tables[s, j // BS], j % BS] = V[j]
    return kc, vc, tables


def random_case(seed, ctx, Hq, Hkv, D, extra_blocks=3):
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in ctx]
    vs = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in ctx]
    nblocks = sum(-(-n // BS) for n in ctx) + extra_blocks
    mb = max(-(-n // BS) for n in ctx) + 1
    kc, vc, tables = scatter_logical(rng, ks, vs, nblocks, mb)
    q = rng.standard_normal((len(ctx), Hq, D)).astype(np.float32)
    scale = np.float32(1.0 / math.sqrt(D))
    return dict(ks=ks, vs=vs, kc=kc, vc=vc, tables=tables, q=q, scale=scale,
                ctx=np.asarray(ctx, dtype=np.int32))


def sdpa_reference(q, ks, vs, scale, Hq):
    """Contiguous-cache attention from torch's fused routine, CPU float64, KV repeated for GQA."""
    outs = []
    for s in range(len(ks)):
        K = torch.from_numpy(ks[s].astype(np.float64))      # [n, Hkv, D]
        V = torch.from_numpy(vs[s].astype(np.float64))
        G = Hq // K.shape[1]
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)  # [1, Hq, n, D]
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)
        Q = torch.from_numpy(q[s].astype(np.float64)).unsqueeze(1).unsqueeze(0)  # [1, Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=float(scale))
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


# ---------------------------------------------------------------------------
def check_vs_contiguous_sdpa(decode):
    """Paged attention over scattered blocks == contiguous attention (MHA and GQA)."""
    worst = 0.0
    for seed, (Hq, Hkv, D), ctx in [
        (1, (4, 4, 16), [1, 16, 17, 40]),
        (2, (8, 2, 32), [5, 33, 64, 90]),
        (3, (6, 3, 8), [31, 32, 48]),
    ]:
        c = random_case(seed, ctx, Hq, Hkv, D)
        got = decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
        ref = sdpa_reference(c["q"], c["ks"], c["vs"], c["scale"], Hq)
        worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


def check_permutation_invariance(decode):
    """All 720 renamings of a 6-block pool give bitwise-identical outputs."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 4, 2, 8
    ctx = np.array([40, 33], dtype=np.int32)        # 3 + 3 blocks = the whole pool
    kc = rng.standard_normal((6, BS, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((6, BS, Hkv, D)).astype(np.float32)
    tables = np.array([[0, 1, 2], [3, 4, 5]], dtype=np.int32)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    scale = np.float32(0.3)
    base = decode(q, kc, vc, tables, ctx, scale)
    worst = 0.0
    for perm in itertools.permutations(range(6)):
        perm = np.asarray(perm)
        kp = np.empty_like(kc)
        vp = np.empty_like(vc)
        kp[perm] = kc                     # old block b now lives at perm[b]
        vp[perm] = vc
        out = decode(q, kp, vp, perm[tables].astype(np.int32), ctx, scale)
        if not np.array_equal(out, base):
            worst = max(worst, float(np.max(np.abs(out - base))) or 1.0)
    return worst


def check_one_token(decode):
    """Context of one token: softmax of one score is 1, so out == that token's V exactly."""
    c = random_case(11, [1, 1, 1], 8, 2, 16)
    got = decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
    worst = 0.0
    for s in range(3):
        v = c["vs"][s][0].astype(np.float64)                # [Hkv, D]
        want = np.repeat(v, 4, axis=0)                      # q head h reads KV head h // 4
        worst = max(worst, float(np.max(np.abs(got[s] - want))))
    return worst


def check_zero_query_mean(decode):
    """q = 0: every score is 0, the weights are uniform, out = mean of the context's V."""
    c = random_case(12, [1, 15, 16, 17, 50], 4, 2, 8)
    q = np.zeros_like(c["q"])
    got = decode(q, c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
    worst = 0.0
    for s, V in enumerate(c["vs"]):
        want = np.repeat(V.astype(np.float64).mean(axis=0), 2, axis=0)
        worst = max(worst, float(np.max(np.abs(got[s] - want))))
    return worst


def check_peaky_query(decode):
    """q aligned with one key, scaled up: the softmax collapses onto that token's V."""
    worst = 0.0
    n = 70
    for j in (0, 15, 16, 31, 32, 47, 69):
        c = random_case(100 + j, [n], 2, 1, 32)
        k = c["ks"][0][j, 0].astype(np.float64)
        q = np.zeros((1, 2, 32), dtype=np.float32)
        q[0, :] = (400.0 / float(c["scale"])) * k / np.linalg.norm(k) / np.linalg.norm(k)
        got = decode(q, c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
        want = c["vs"][0][j, 0].astype(np.float64)
        worst = max(worst, float(np.max(np.abs(got[0] - want[None, :]))))
    return worst


def check_poisoned_unused(decode):
    """NaN/Inf in slots past the context, in free blocks and garbage table tails change nothing."""
    c = random_case(13, [3, 17, 32, 45], 4, 4, 16, extra_blocks=4)
    clean = decode(c["q"], np.nan_to_num(c["kc"]), np.nan_to_num(c["vc"]),
                   c["tables"], c["ctx"], c["scale"])
    kc = np.where(np.isnan(c["kc"]), np.inf, c["kc"]).astype(np.float32)
    vc = c["vc"].copy()                                 # NaN stays in unused V slots
    tables = c["tables"].copy()
    tables[tables < 0] = 2 ** 30                       # out-of-range ids past the used blocks
    got = decode(c["q"], kc, vc, tables, c["ctx"], c["scale"])
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - clean)))


def check_gqa_equals_repeated_mha(decode):
    """Grouped-query attention == multi-head attention with each KV head repeated G times."""
    c = random_case(14, [9, 40, 64], 8, 2, 16)
    got = decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["scale"])
    kr = np.repeat(c["kc"], 4, axis=2)
    vr = np.repeat(c["vc"], 4, axis=2)
    mha = decode(c["q"], kr, vr, c["tables"], c["ctx"], c["scale"])
    return float(np.max(np.abs(got - mha)))


def check_empty_context_zero(decode):
    c = random_case(15, [5, 20], 2, 2, 8)
    ctx = c["ctx"].copy()
    ctx[0] = 0
    got = decode(c["q"], c["kc"], c["vc"], c["tables"], ctx, c["scale"])
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got[0])))


DECODE_CHECKS = {
    "contiguous_sdpa": (check_vs_contiguous_sdpa, 1e-12),
    "permutation_invariance": (check_permutation_invariance, 0.0),
    "one_token": (check_one_token, 0.0),
    "zero_query_mean": (check_zero_query_mean, 1e-13),
    "peaky_query": (check_peaky_query, 1e-12),
    "poisoned_unused": (check_poisoned_unused, 0.0),
    "gqa_equals_repeated_mha": (check_gqa_equals_repeated_mha, 0.0),
    "empty_context_zero": (check_empty_context_zero, 0.0),
}
