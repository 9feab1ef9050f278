"""Preemption by swapping on the GPU: device pool -> pinned host pool -> device pool.

A group of sequences (forks and copy-on-write included) is swapped out with
the allocator's pairs run by ``pkv_swap_blocks`` into a page-locked host pool;
the device blocks it gave up are poisoned and reused by a new sequence; the
group is swapped back into new device blocks.  Both copies must match the
oracle's pool-to-pool copy byte for byte over the whole destination pool, and
decode after the round trip must equal decode before it bit for bit (the
kernels' reduction order depends only on logical positions) and match the
oracle on the K/V the sequences held before they left ("vLLM and
PagedAttention", §3 continuous batching, on preemption).
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


def pinned_like(shape, dtype, fill_bits):
    t = torch.empty(shape, dtype=dtype, pin_memory=True)
    assert t.is_pinned()
    if dtype == torch.bfloat16:
        t.view(torch.int16).fill_(fill_bits)
    else:
        t.view(torch.int32).fill_(fill_bits)
    return t


def pool_bits(t):
    return host(t) if t.is_cuda else (t.view(torch.int16).numpy().view(np.uint16)
                                      if t.dtype == torch.bfloat16 else t.numpy())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swap_round_trip(dtype):
    S, Hq, Hkv, D = 24, 16, 4, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"swap round trip {dtype} S={S} Hq={Hq} Hkv={Hkv} D={D}")
    rng = np.random.default_rng(41)
    ctx0 = rng.integers(1, 700, size=S)
    nb = int(math.ceil(1.5 * np.sum(-(-ctx0 // 16)))) + 64
    nh = nb
    alloc = pkv.BlockAllocator(nb, 16, shuffle_seed=9)
    alloc.set_host_pool(nh)
    kc = torch.zeros((nb, 16, Hkv, D), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    # the oracle's copy of every write and copy-on-write the GPU makes
    mirror = [host(kc), host(vc)]

    def write(sid, n, seed):
        slots, cow = alloc.append(sid, n)
        if cow:
            pkv.pkv_copy_blocks(kc, vc, dev(np.array(cow, np.int32)))
            mirror[:] = oracle.copy_blocks(mirror[0], mirror[1], cow)
        k = normal_values_parallel(seed, (n, Hkv, D), dtype)
        v = normal_values_parallel(seed + 1, (n, Hkv, D), dtype)
        pkv.pkv_write(kc, vc, dev(k), dev(v), dev(np.array(slots, np.int32)))
        mirror[:] = oracle.write_kv(mirror[0], mirror[1], k, v, np.array(slots, np.int32))

    # sequences 0..S-1; 20..23 are forks of 0..3 with a few private tokens (CoW)
    for s in range(S - 4):
        alloc.add_seq(s)
        write(s, int(ctx0[s]), 1000 + 2 * s)
    for j in range(4):
        alloc.fork(j, S - 4 + j)
        write(S - 4 + j, int(rng.integers(1, 40)), 2000 + 2 * j)
    ids = np.arange(S, dtype=np.int64)
    mb = max(len(alloc.block_table(s)) for s in range(S)) + 2
    q = normal_values_parallel(77, (S, Hq, D), dtype)
    scale = np.float32(1.0 / math.sqrt(D))

    def decode():
        tables, lens = alloc.block_tables(ids, mb)
        out = torch.empty((S, Hq, D), dtype=tdt, device="cuda")
        pkv.pkv_attention_decode(out, dev(q), kc, vc, dev(tables), dev(lens), float(scale), int(lens.max()))
        torch.cuda.synchronize()
        return out, tables, lens

    out0, tables0, lens0 = decode()
    kh0, vh0 = mirror
    assert host(kc).tobytes() == kh0.tobytes() and host(vc).tobytes() == vh0.tobytes(), \
        "the writes and copies differ from the oracle's"

    # ---- swap out a group holding a parent with its fork, a fork without its parent, and others
    group = [0, 20, 21, 5, 6, 7, 11, 12]
    hk = pinned_like((nh, 16, Hkv, D), tdt, -1)          # all-ones bits: NaN in both dtypes
    hv = pinned_like((nh, 16, Hkv, D), tdt, -1)
    hk_before, hv_before = pool_bits(hk).copy(), pool_bits(hv).copy()
    pairs_out = alloc.swap_out(group)
    assert len(pairs_out) > 0
    pkv.pkv_swap_blocks(hk, hv, kc, vc, dev(np.array(pairs_out, np.int32)))
    torch.cuda.synchronize()
    want_k, want_v = oracle.swap_blocks(hk_before, hv_before, kh0, vh0, pairs_out)
    assert pool_bits(hk).tobytes() == want_k.tobytes() and pool_bits(hv).tobytes() == want_v.tobytes()
    say(f"  swap-out: {len(pairs_out)} blocks bit-exact over the host pool")

    # ---- poison every free device block, then a new sequence takes some of them
    free = [b for b in range(nb) if alloc.refcount(b) == 0]
    idx = torch.tensor(free, dtype=torch.long, device="cuda")
    kc.index_fill_(0, idx, float("nan"))
    vc.index_fill_(0, idx, float("inf"))
    alloc.add_seq(500)
    write(500, 16 * 20 + 3, 3000)

    # ---- swap back in to new device blocks
    kd_before, vd_before = host(kc), host(vc)
    pairs_in = alloc.swap_in(group)
    assert len(pairs_in) == len(pairs_out)
    pkv.pkv_swap_blocks(kc, vc, hk, hv, dev(np.array(pairs_in, np.int32)))
    torch.cuda.synchronize()
    want_k, want_v = oracle.swap_blocks(kd_before, vd_before, pool_bits(hk), pool_bits(hv), pairs_in)
    assert host(kc).tobytes() == want_k.tobytes() and host(vc).tobytes() == want_v.tobytes()
    say(f"  swap-in: {len(pairs_in)} blocks bit-exact over the device pool")

    out1, tables1, lens1 = decode()
    assert np.array_equal(lens1, lens0)
    assert host(out1).tobytes() == host(out0).tobytes()
    ref = oracle.decode_attention(q, kh0, vh0, tables0, lens0, scale)
    assert_close(host_f64(out1), ref, dtype, "decode after the round trip")


def test_pool_check_classifies_memory():
    """The pointer check pkv_swap_blocks relies on (host only, launches nothing)."""
    L = pkv.lib()
    d = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    p = torch.empty(1 << 20, dtype=torch.uint8, pin_memory=True)
    pageable = np.empty(1 << 20, np.uint8)
    assert L.pkv_check_pool(d.data_ptr(), d.numel()) == 0
    assert L.pkv_check_pool(p.data_ptr(), p.numel()) == 0
    assert L.pkv_check_pool(p.data_ptr() + 4096, p.numel() - 4096) == 0
    assert L.pkv_check_pool(pageable.ctypes.data, pageable.size) != 0
    assert L.pkv_check_pool(d.data_ptr(), 1 << 40) != 0
    assert L.pkv_check_pool(p.data_ptr(), 1 << 40) != 0
