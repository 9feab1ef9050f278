"""A decode step replayed as a HIP graph equals the same step run call by call.

The graph (``pkv_decode_graph_create``) records the step's launches once; each
replay reads the device buffers the host refreshed in place (new q, new K/V
rows, slots, tables and context lengths after the allocator's append).  Over
several replays, with the program's own eager work and synchronizations between
them, the graph's output and caches must equal an eager run of the same calls
on a second copy of the pools byte for byte, and the last step must match the
oracle ("vLLM and PagedAttention", §6 key engineering optimizations: a step's
kernel sequence launched as one graph).  Contexts cross 512-token partition
boundaries during the run, so the device-built work list changes shape between
replays of one graph.
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


@pytest.mark.parametrize("form", ["f32_write", "bf16_write", "bf16_append"])
def test_graph_replays_equal_eager(form):
    dtype = "f32" if form.startswith("f32") else "bf16"
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    append = form.endswith("append")
    S, Hq, Hkv, D = (4, 8, 8, 64) if dtype == "f32" else (16, 32, 8, 128)
    steps = 6
    rng = np.random.default_rng(91)
    ctx0 = rng.integers(1, 100, size=S) if dtype == "f32" else rng.integers(505, 1030, size=S)
    ctx0[0] = 510                                          # crosses 512 during the run
    bound = int(ctx0.max()) + steps
    say(f"graph replay {form} S={S} Hq={Hq} Hkv={Hkv} D={D} ctx {ctx0.min()}..{ctx0.max()}")
    nb = int(math.ceil(1.25 * np.sum(-(-(ctx0 + steps) // 16)))) + 8
    mb = -(-bound // 16) + 1
    alloc = pkv.BlockAllocator(nb, 16, shuffle_seed=5)
    ids = np.arange(S, dtype=np.int64)
    for s in range(S):
        alloc.add_seq(s)
    pre = [alloc.append(s, int(ctx0[s]) - 1)[0] for s in range(S)]
    kc = torch.zeros((nb, 16, Hkv, D), dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    slots0 = np.concatenate([np.array(p, np.int32) for p in pre])
    n0 = slots0.size
    k0, v0 = normal_values_parallel(1, (n0, Hkv, D), dtype), normal_values_parallel(2, (n0, Hkv, D), dtype)
    pkv.pkv_write(kc, vc, dev(k0), dev(v0), dev(slots0))
    kc2, vc2 = kc.clone(), vc.clone()                      # the eager run's pools
    exp_k, exp_v = oracle.write_kv(host(kc), host(vc), k0, v0, slots0)   # the oracle's pools

    # static buffers the graph reads
    q_b = torch.zeros((S, Hq, D), dtype=tdt, device="cuda")
    k_b = torch.zeros((S, Hkv, D), dtype=tdt, device="cuda")
    v_b = torch.zeros_like(k_b)
    slot_b = torch.zeros(S, dtype=torch.int32, device="cuda")
    tab_b = torch.zeros((S, mb), dtype=torch.int32, device="cuda")
    ctx_b = torch.zeros(S, dtype=torch.int32, device="cuda")
    out_g = torch.zeros((S, Hq, D), dtype=tdt, device="cuda")
    out_e = torch.zeros_like(out_g)
    scale = np.float32(1.0 / math.sqrt(D))
    graph = pkv.DecodeGraph(out_g, q_b, k_b, v_b, kc, vc, tab_b, ctx_b, float(scale), bound,
                            slot_mapping=None if append else slot_b)
    ws_e = pkv.decode_workspace(S, Hq, D, bound)
    for i in range(steps):
        slots, cow = alloc.append_batch(ids, np.ones(S, np.int32))
        assert len(cow) == 0
        tables, lens = alloc.block_tables(ids, mb, fill=0)
        q = normal_values_parallel(100 + 3 * i, (S, Hq, D), dtype)
        kn = normal_values_parallel(101 + 3 * i, (S, Hkv, D), dtype)
        vn = normal_values_parallel(102 + 3 * i, (S, Hkv, D), dtype)
        for b, a in ((q_b, q), (k_b, kn), (v_b, vn), (slot_b, slots), (tab_b, tables), (ctx_b, lens)):
            b.copy_(dev(a))
        graph.launch()
        # the eager step on the second pools, then a synchronization
        if append:
            pkv.pkv_attention_decode_append(out_e, dev(q), dev(kn), dev(vn), kc2, vc2, dev(tables), dev(lens),
                                            float(scale), bound, workspace=ws_e)
        else:
            pkv.pkv_write(kc2, vc2, dev(kn), dev(vn), dev(slots))
            pkv.pkv_attention_decode(out_e, dev(q), kc2, vc2, dev(tables), dev(lens), float(scale), bound,
                                     workspace=ws_e)
        torch.cuda.synchronize()
        exp_k, exp_v = oracle.write_kv(exp_k, exp_v, kn, vn, np.asarray(slots, np.int32))
        assert host(out_g).tobytes() == host(out_e).tobytes(), f"step {i}: graph output differs"
        assert host(kc).tobytes() == host(kc2).tobytes() and host(vc).tobytes() == host(vc2).tobytes(), i
        assert host(kc).tobytes() == exp_k.tobytes() and host(vc).tobytes() == exp_v.tobytes(), \
            f"step {i}: the pool differs from the oracle's writes"
    say(f"  {steps} replays equal to the eager calls byte for byte; contexts now {lens.min()}..{lens.max()}")
    ref = oracle.decode_attention(q, exp_k, exp_v, tables, lens, scale)
    assert_close(host_f64(out_g), ref, dtype, f"graph {form} last step")
    graph.close()


def test_graph_rejects_bad_arguments():
    """Creation validates like the captured calls and records nothing on an error."""
    S, Hq, Hkv, D = 2, 8, 8, 64
    z = lambda *sh, dt=torch.float32: torch.zeros(sh, dtype=dt, device="cuda")
    kc = z(8, 16, Hkv, D)
    with pytest.raises(pkv.PagedKVError):                  # append form is bf16 only
        pkv.DecodeGraph(z(S, Hq, D), z(S, Hq, D), z(S, Hkv, D), z(S, Hkv, D), kc, kc.clone(),
                        z(S, 4, dt=torch.int32), z(S, dt=torch.int32), 0.125, 64)
    with pytest.raises(pkv.PagedKVError):                  # context bound wider than the tables
        pkv.DecodeGraph(z(S, Hq, D), z(S, Hq, D), z(S, Hkv, D), z(S, Hkv, D), kc, kc.clone(),
                        z(S, 4, dt=torch.int32), z(S, dt=torch.int32), 0.125, 65,
                        slot_mapping=z(S, dt=torch.int32))
