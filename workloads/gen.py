"""Seeded generators: context lengths, scattered block tables and N(0,1) tensors.

Storage conventions: fp32 data is ``numpy.float32``; bf16 data is ``numpy.uint16``
holding bfloat16 bit patterns, produced from fp32 draws by round-to-nearest-even.
Every consumer (oracle and GPU path alike) reads the rounded values, so input
rounding is never counted as kernel error.
"""

import math
from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16          # tokens per KV block (the pages' usual block size)
_CHUNK = 1 << 24         # elements per generation chunk (bounds host temporaries)


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and length distribution of one synthetic decode batch (one layer)."""

    name: str
    dtype: str               # "f32" or "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ctx_kind: str            # "uniform" | "loguniform" | "fixed" | "prefix"
    ctx_lo: int              # inclusive bounds (for "fixed": lo == hi)
    ctx_hi: int
    pool_blocks: int = 0     # 0 -> ceil(1.25 * blocks needed)
    prefix_len: int = 0      # "prefix": shared prefix length; ctx = prefix + tail
    chunk_rows: int = 0      # chunked prefill: rows of the one prefill chunk
    chunk_ctx: int = 0       # chunked prefill: total context of that sequence

    @property
    def max_ctx(self):
        """Largest context any sequence can have (sets the table width)."""
        return max(self.prefix_len + self.ctx_hi, self.chunk_ctx)

    @property
    def max_blocks_per_seq(self):
        return -(-self.max_ctx // BLOCK_SIZE)


SPECS = {s.name: s for s in [
    # tiny multi-head fp32 batch with a 64-block pool
    WorkloadSpec("tiny_f32_mha_s4_h8_d64", "f32", 4, 8, 8, 64, "uniform", 1, 100, pool_blocks=64),
    # Llama-2-7B-shaped layer: 32 q = 32 KV heads, d 128
    WorkloadSpec("llama2_7b_mha_bf16_s64_ctx1_2048", "bf16", 64, 32, 32, 128, "uniform", 1, 2048),
    # grouped-query 32/8, long log-uniform contexts
    WorkloadSpec("gqa32x8_bf16_s128_ctx512_8192", "bf16", 128, 32, 8, 128, "loguniform", 512, 8192),
    # 256 sequences sharing a 1500-token prefix, private tails of 8..512 tokens
    WorkloadSpec("prefix1500_gqa32x8_bf16_s256_tail8_512", "bf16", 256, 32, 8, 128, "prefix", 8, 512,
                 prefix_len=1500),
    # one 512-row prefill chunk (context 4096) + 192 decode sequences of 256..4096
    WorkloadSpec("mixed_chunk512_ctx4096_gqa32x8_bf16_s192", "bf16", 192, 32, 8, 128, "uniform", 256, 4096,
                 chunk_rows=512, chunk_ctx=4096),
    # fixed-context sweeps
    WorkloadSpec("gqa32x8_bf16_s128_ctx2048", "bf16", 128, 32, 8, 128, "fixed", 2048, 2048),
    WorkloadSpec("gqa32x8_bf16_s128_ctx4096", "bf16", 128, 32, 8, 128, "fixed", 4096, 4096),
    WorkloadSpec("gqa32x8_bf16_s128_ctx8192", "bf16", 128, 32, 8, 128, "fixed", 8192, 8192),
    WorkloadSpec("mha32_bf16_s64_ctx2048", "bf16", 64, 32, 32, 128, "fixed", 2048, 2048),
    WorkloadSpec("mha32_bf16_s64_ctx4096", "bf16", 64, 32, 32, 128, "fixed", 4096, 4096),
]}


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    NaN inputs become a quiet NaN with the input's sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # add 0x7FFF plus the lowest kept bit, then keep the top half; the uint32 sum
    # wraps only for negative NaN patterns, which are replaced below
    with np.errstate(over="ignore"):
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out = (r >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = (u[nan] >> np.uint32(16)).astype(np.uint16) | np.uint16(0x0040)
    return out


def normal_values(rng, shape, dtype):
    """i.i.d. N(0,1) draws of ``shape``, stored as ``dtype`` ("f32" or "bf16")."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        v = rng.standard_normal(b - a, dtype=np.float32)
        out[a:b] = v if dtype == "f32" else f32_to_bf16_bits(v)
    return out.reshape(shape)


def draw_context_lens(rng, spec, n=None):
    """Context lengths (inclusive integer ranges) for ``n`` sequences of ``spec``.

    "uniform": integers in [lo, hi]; "loguniform": floor(exp(U(ln lo, ln hi)))
    clamped to [lo, hi]; "fixed": lo; "prefix": prefix_len + uniform tail in [lo, hi].
    """
    n = spec.num_seqs if n is None else n
    lo, hi = spec.ctx_lo, spec.ctx_hi
    if spec.ctx_kind == "uniform":
        c = rng.integers(lo, hi + 1, size=n)
    elif spec.ctx_kind == "loguniform":
        c = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
        c = np.clip(c, lo, hi)
    elif spec.ctx_kind == "fixed":
        c = np.full(n, lo)
    elif spec.ctx_kind == "prefix":
        c = spec.prefix_len + rng.integers(lo, hi + 1, size=n)
    else:
        raise ValueError(spec.ctx_kind)
    return c.astype(np.int32)


def pool_blocks_for(spec, context_lens, extra_blocks=0):
    """Pool size: the spec's fixed count, else ceil(1.25 x blocks the batch needs)."""
    if spec.pool_blocks:
        return spec.pool_blocks
    need = int(np.sum(-(-np.asarray(context_lens, dtype=np.int64) // BLOCK_SIZE))) + extra_blocks
    return int(math.ceil(1.25 * need))


def random_block_tables(rng, context_lens, num_blocks, max_blocks_per_seq, fill=-1):
    """Scattered tables: distinct random physical ids, ceil(ctx/16) per sequence.

    Unused entries hold ``fill``.  Raises if the pool is too small.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    nblk = -(-ctx // BLOCK_SIZE)
    if nblk.sum() > num_blocks:
        raise ValueError("pool too small for the batch")
    if nblk.max(initial=0) > max_blocks_per_seq:
        raise ValueError("table too narrow for the batch")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(ctx), max_blocks_per_seq), fill, dtype=np.int32)
    off = 0
    for s, nb in enumerate(nblk.tolist()):
        tables[s, :nb] = perm[off:off + nb]
        off += nb
    return tables


def make_decode_inputs(spec, seed, dtype=None, table_fill=-1):
    """One decode batch of ``spec``: lengths, scattered tables, pool, q and new K/V rows.

    Returns a dict of numpy arrays: ``context_lens`` [S] (each count includes the
    new token), ``block_tables`` [S, MB], ``key_cache``/``value_cache``
    [NB, 16, Hkv, D], ``q`` [S, Hq, D], ``k_new``/``v_new`` [S, Hkv, D] and
    ``scale`` = 1/sqrt(D) as float32.  Every pool slot holds N(0,1) data.
    """
    dt = dtype or spec.dtype
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    ctx = draw_context_lens(rng, spec)
    nb = pool_blocks_for(spec, ctx)
    mb = spec.max_blocks_per_seq
    tables = random_block_tables(rng, ctx, nb, mb, fill=table_fill)
    return {
        "spec": spec,
        "dtype": dt,
        "context_lens": ctx,
        "block_tables": tables,
        "num_blocks": nb,
        "key_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dt),
        "value_cache": normal_values(rng, (nb, BLOCK_SIZE, Hkv, D), dt),
        "q": normal_values(rng, (S, Hq, D), dt),
        "k_new": normal_values(rng, (S, Hkv, D), dt),
        "v_new": normal_values(rng, (S, Hkv, D), dt),
        "scale": np.float32(1.0 / math.sqrt(D)),
    }
