#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

One step = one decode iteration for a batch of sequences, every stage of the
path included:
  1. host block allocator: one new token per sequence (a new block when the last
     one is full), slot of each new token, refreshed block tables and lengths,
     written into a pinned staging buffer (C++ allocator behind the C ABI);
  2. pkv_attention_decode_plan_upload on the compute stream: one launch builds
     the work list from the pinned lengths while its other workgroups copy the
     pinned slots and lengths, and the used entries of each table row, to the
     device (no copy engine, no second stream: a
     cross-stream wait costs the stream ~11 us, a copy-engine transfer more),
     and others merge the previous step's partials (step 5 of that step);
  3. pkv_copy_blocks for any copy-on-write pairs (none for unshared batches);
  4. bf16: pkv_attention_decode_partitions_append (split-context decode, the
     dominant kernel, which also stores each sequence's new K/V row in the cache);
     fp32: pkv_write of the new tokens' K/V, then pkv_attention_decode_partitions;
  5. the log-sum-exp merge of multi-partition sequences: inside the next step's
     launch of 2, or pkv_attention_decode_merge after the last step of a run.
Contexts grow by one token per step, as in real decoding.  Inputs (pool, q, new
K/V rows) are resident in HBM before timing starts.  R copies of the KV pool are
rotated step to step so each step's KV reads come from HBM, not the 256 MiB
last-level cache.

Prints ONE JSON line.  The partition kernel's duration comes from two HIP
events recorded on the compute stream around it in every ev_every(K)-th timed
step, at least ten launches per run (each timing event costs the stream a few
microseconds, so the other launches are not bracketed there); the write (fp32)
and merge durations come from a few extra steps after the timed region, with
events around every launch.  After those, plain read kernels (libpkvprobe.so)
read the same K/V blocks, in the same order, from the same rotated pools: the
line reports the partition kernel's KV-read rate against theirs as well as
against the 8 TB/s peak.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)



def ev_every(steps):
    """Timed steps per event-bracketed launch: at least ten bracketed launches
    per run (every step when there are ten or fewer)."""
    return max(1, steps // 10)


METRIC = "decode tokens/s + KV-read HBM GB/s (% of MI355X peak), bf16 GQA ctx 2k–8k"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "gqa32x8_bf16_s128_ctx512_8192"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partitions_traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_360_amd/csrc/kernels/decode_mfma.hip",
                  "paged_kv_cache_360_amd/csrc/kernels/decode_common.hpp",
                  "paged_kv_cache_360_amd/csrc/kernels/device_common.hpp",
                  "paged_kv_cache_360_amd/csrc/kernels/plan.hip"]         # the plan shapes the work items
MFMA_BF16_PEAK_TFLOPS = 2500.0          # MI355X dense bf16 matrix peak
COPY_PROBE_BYTES = 512 * 1024 * 1024   # pkv_copy_blocks in --copy-probe: read and written per launch


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--pool-copies", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain block copy of known size (counter calibration)")
    ap.add_argument("--prefix-cache-probe", action="store_true",
                    help="only time the host allocator admitting requests through the prefix cache "
                         "(a shared 1500-token system prompt; no GPU work)")
    ap.add_argument("--capacity-sim", action="store_true",
                    help="only run the host capacity simulator: static reservation against paged "
                         "blocks under continuous batching (no GPU work)")
    ap.add_argument("--swap-probe", action="store_true",
                    help="only time pkv_swap_blocks between the device pool and a pinned host pool "
                         "(8192 scattered 32 KiB blocks per cache each way) against one contiguous "
                         "copy of the same bytes")
    ap.add_argument("--graph-probe", action="store_true",
                    help="only time one decode step replayed as a HIP graph against the same launches "
                         "made one by one (4-sequence fp32 MHA batch and the default GQA batch)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the plain read kernels over a 1.5 GiB pool (blocks in random order; "
                         "whole blocks and per-head slices; random and zero-filled data)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="only run the chunked-prefill kernel's LDS operand reads by themselves (K, V, both; "
                         "4, 8 and 16 waves per compute unit)")
    ap.add_argument("--traffic-from", nargs=5, metavar="FILE", default=None,
                    help="rocprofv3 counter results (counter_collection CSV or results .db): FETCH_SIZE "
                         "and WRITE_SIZE of a bench run, "
                         "then of a --copy-probe run, and that bench run's --json-out line; writes the "
                         "partition kernel's HBM traffic per algorithmic byte for later bench lines, "
                         "and exits")
    return ap.parse_args()


def traffic_from_counters(paths, workload):
    """HBM traffic of the partition kernel per algorithmic byte, from rocprofv3 --pmc CSVs.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what they read for
    the copy probe, whose bytes are known (COPY_PROBE_BYTES each way), and
    averaged over the timed launches of the counted bench run (dispatches W ..
    W + K - 1 of the kernel, with W and K from that run's JSON line); the
    algorithmic bytes of the same launches come from that line.  The ratio is
    stored with the kernel sources' hash and the workload: a later bench line of
    the same kernel and workload reports traffic = ratio x its own algorithmic
    bytes per launch, and null once the kernel has changed.
    """
    import csv

    fetch, write, cfetch, cwrite, bench_json = paths
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    W, K = int(line["warmup"]), int(line["steps"])
    if line["config"]["workload"] != workload:
        raise SystemExit(f"{bench_json} is a run of {line['config']['workload']}, not {workload}")
    alg = float(line["roofline"]["algorithmic_bytes_mean_all_timed"])

    def rows_of(path, kernel_part):
        """(dispatch id, counter value) of the kernel's dispatches: a
        counter_collection CSV, or the SQLite results database rocprofv3
        writes by default."""
        if path.endswith(".db"):
            import sqlite3
            con = sqlite3.connect(path)
            q = "select dispatch_id, value, kernel_name from counters_collection"
            return [(int(d), float(v)) for d, v, k in con.execute(q) if kernel_part in k]
        return [(int(r["Dispatch_Id"]), float(r["Counter_Value"]))
                for r in csv.DictReader(open(path)) if kernel_part in r["Kernel_Name"]]

    def mean_kib(path, kernel_part, timed=False):
        rows = sorted(rows_of(path, kernel_part))
        vals = [v for _, v in rows]
        if timed:
            if len(vals) < W + K:
                raise SystemExit(f"{path}: {len(vals)} dispatches of {kernel_part}, fewer than "
                                 f"--warmup {W} + --steps {K}")
            vals = vals[W:W + K]
        if not vals:
            raise SystemExit(f"{path}: no dispatch of {kernel_part}")
        return sum(vals) / len(vals)

    kf = COPY_PROBE_BYTES / (mean_kib(cfetch, "copy_blocks_kernel") * 1024)
    kw = COPY_PROBE_BYTES / (mean_kib(cwrite, "copy_blocks_kernel") * 1024)
    fb = mean_kib(fetch, "decode_partition_mfma_kernel", timed=True) * 1024 * kf
    wb = mean_kib(write, "decode_partition_mfma_kernel", timed=True) * 1024 * kw
    out = {"kernel": "decode_partition_mfma_kernel", "workload": workload,
           "kernel_source_sha256": kernel_source_hash(), "counted_warmup": W, "counted_steps": K,
           "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
           "algorithmic_bytes_per_launch": int(alg),
           "traffic_over_algorithmic": round((fb + wb) / alg, 5),
           "fetch_scale": round(kf, 4), "write_scale": round(kw, 4)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_probe(torch, pkv):
    """pkv_copy_blocks over 8192 pairs of 32 KiB blocks per cache: reads 512 MiB, writes 512 MiB."""
    nb, hkv, d = 2 * 8192, 8, 128                     # 32 KiB bf16 blocks
    kc = torch.zeros((nb, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    half = nb // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).to(torch.int32).cuda()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for i in range(3):
        ev[i].record()
        pkv.pkv_copy_blocks(kc, vc, pairs)
    ev[3].record()
    torch.cuda.synchronize()
    moved = 2 * half * 16 * hkv * d * 2
    us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(1, 3)]   # the first launch warms up
    t = sum(us) / len(us) * 1e-6
    print(json.dumps({"probe": "pkv_copy_blocks", "bytes_read_per_launch": moved,
                      "bytes_written_per_launch": moved, "launches": 3,
                      "avg_launch_us": round(t * 1e6, 1), "read_plus_write_GBps": round(2 * moved / t / 1e9, 1),
                      "frac_of_hbm_peak": round(2 * moved / t / 1e9 / HBM_PEAK_GBPS, 4)}))


def swap_probe(torch, pkv, seed):
    """pkv_swap_blocks moving 8192 scattered 32 KiB blocks per cache (512 MiB in all)
    from the device pool to a pinned host pool and back, next to one contiguous
    copy of the same bytes each way (the host link's rate for a plain copy)."""
    n, hkv, d = 8192, 8, 128
    nb = 2 * n                                          # device pool twice the moved blocks
    kc = torch.randn((nb, 16, hkv, d), device="cuda").to(torch.bfloat16)
    vc = torch.randn((nb, 16, hkv, d), device="cuda").to(torch.bfloat16)
    hk = torch.empty((n, 16, hkv, d), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    g = torch.Generator().manual_seed(seed)
    dev_ids = torch.randperm(nb, generator=g)[:n]
    host_ids = torch.randperm(n, generator=g)
    out_pairs = torch.stack([dev_ids, host_ids], 1).to(torch.int32).cuda()
    in_pairs = torch.stack([host_ids, dev_ids], 1).to(torch.int32).cuda()
    moved = 2 * n * 16 * hkv * d * 2
    reps = 3

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        ev[0].record()
        fn()                                            # warm-up launch
        for i in range(reps):
            ev[i + 1].record()
            fn()
        ev[reps + 1].record()
        torch.cuda.synchronize()
        us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(1, reps + 1)]
        return sum(us) / len(us)

    res = {}
    res["swap_out_us"] = timed(lambda: pkv.pkv_swap_blocks(hk, hv, kc, vc, out_pairs))
    res["swap_in_us"] = timed(lambda: pkv.pkv_swap_blocks(kc, vc, hk, hv, in_pairs))
    dk = kc[:n]
    dv = vc[:n]
    res["contiguous_d2h_us"] = timed(lambda: (hk.copy_(dk, non_blocking=True), hv.copy_(dv, non_blocking=True)))
    res["contiguous_h2d_us"] = timed(lambda: (dk.copy_(hk, non_blocking=True), dv.copy_(hv, non_blocking=True)))
    line = {"probe": "pkv_swap_blocks", "blocks_per_cache": n, "block_bytes": 16 * hkv * d * 2,
            "bytes_per_direction": moved, "launches": reps}
    for k, us in res.items():
        line[k] = round(us, 1)
        line[k.replace("_us", "_GBps")] = round(moved / (us * 1e-6) / 1e9, 1)
    torch.cuda.synchronize()
    print(json.dumps(line))


def graph_probe(torch, np, pkv, seed):
    """One decode step (write + plan + partitions + merge; the append form for
    bf16) made with direct C-ABI calls, one launch at a time, against the same
    step replayed as a HIP graph (``pkv_decode_graph_launch``).  Inputs are
    resident and unchanged between steps, so the difference is launch cost."""
    import ctypes

    from paged_kv_cache_360_amd._lib import lib
    from workloads import SPECS, draw_context_lens

    L = lib()
    rng = np.random.default_rng(seed)
    lines = []
    for name, steps in (("tiny_f32_mha_s4_h8_d64", 400), (DEFAULT_WORKLOAD, 60)):
        spec = SPECS[name]
        S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
        bf16 = spec.dtype == "bf16"
        tdt = torch.bfloat16 if bf16 else torch.float32
        ctx = np.asarray(draw_context_lens(rng, spec), np.int64)
        nblk = -(-ctx // 16)
        nb = int(math.ceil(1.25 * nblk.sum())) if bf16 else 64
        mb = int(nblk.max())
        perm = rng.permutation(nb).astype(np.int32)
        tables = np.zeros((S, mb), np.int32)
        off = 0
        for i in range(S):
            tables[i, :nblk[i]] = perm[off:off + nblk[i]]
            off += int(nblk[i])
        slots = np.array([tables[i, (ctx[i] - 1) // 16] * 16 + (ctx[i] - 1) % 16 for i in range(S)], np.int32)
        kc = torch.randn((nb, 16, Hkv, D), device="cuda").to(tdt)
        vc = torch.randn((nb, 16, Hkv, D), device="cuda").to(tdt)
        q = torch.randn((S, Hq, D), device="cuda").to(tdt)
        kn = torch.randn((S, Hkv, D), device="cuda").to(tdt)
        vn = torch.randn((S, Hkv, D), device="cuda").to(tdt)
        out = torch.empty_like(q)
        t_d = torch.from_numpy(tables).cuda()
        c_d = torch.from_numpy(ctx.astype(np.int32)).cuda()
        s_d = torch.from_numpy(slots).cuda()
        max_ctx = int(ctx.max())
        ws = pkv.decode_workspace(S, Hq, D, max_ctx)
        ws_p, ws_n = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
        scale = 1.0 / math.sqrt(D)
        dt = 1 if bf16 else 0
        stream = torch.cuda.current_stream().cuda_stream
        p = lambda t: t.data_ptr()
        if bf16:
            a_app = (p(out), p(q), p(kn), p(vn), p(kc), p(vc), p(t_d), p(c_d), ctypes.c_float(scale), 16, Hq, Hkv,
                     D, S, mb, nb, max_ctx, dt, ws_p, ws_n, stream)

            def eager():
                L.pkv_attention_decode_append(*a_app)
        else:
            a_w = (p(kc), p(vc), p(kn), p(vn), p(s_d), S, nb, 16, Hkv, D, dt, stream)
            a_d = (p(out), p(q), p(kc), p(vc), p(t_d), p(c_d), ctypes.c_float(scale), 16, Hq, Hkv, D, S, mb, nb,
                   max_ctx, dt, ws_p, ws_n, stream)

            def eager():
                L.pkv_write(*a_w)
                L.pkv_attention_decode(*a_d)
        g = pkv.DecodeGraph(out, q, kn, vn, kc, vc, t_d, c_d, scale, max_ctx,
                            slot_mapping=None if bf16 else s_d, workspace=ws)

        def run(fn):
            """(device µs per step between events, host µs per step to issue)."""
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            t1 = time.perf_counter()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / steps, (t1 - t0) * 1e6 / steps

        us_e, host_e = run(eager)
        us_g, host_g = run(lambda: L.pkv_decode_graph_launch(g._h, stream))
        g.close()
        parts = -(-max_ctx // 512)
        lines.append({"workload": name, "steps": steps,
                      # bf16: plan, partitions (append form); fp32: write, partitions, and the
                      # plan only when a context spans partitions; a merge when one does
                      "kernels_per_step": 2 + (0 if bf16 else 1) - (0 if bf16 or parts > 1 else 1)
                      + (1 if parts > 1 else 0),
                      "eager_us_per_step": round(us_e, 2), "graph_us_per_step": round(us_g, 2),
                      "eager_host_issue_us_per_step": round(host_e, 2),
                      "graph_host_issue_us_per_step": round(host_g, 2),
                      "speedup": round(us_e / us_g, 3)})
    print(json.dumps({"probe": "decode_graph", "results": lines}))


def prefix_cache_probe(np, pkv, seed):
    """Host allocator with automatic prefix caching: requests made of a shared
    1500-token system prompt and a user part of 8..512 tokens (the shared-prefix
    batch's lengths) are admitted with add_seq_tokens, decoded for 16 tokens with
    append_tokens and released, 256 at a time in flight, on a pool that holds
    them.  Reports how many prompt tokens the cache served and the host time per
    admission."""
    rng = np.random.default_rng(seed)
    system = np.arange(1500, dtype=np.int32)
    n_req, in_flight = 4096, 256
    alloc = pkv.BlockAllocator(in_flight * 64 + 256, 16, shuffle_seed=seed)
    prompt_tokens = cached_tokens = 0
    t_admit = t_decode = 0.0
    live = []
    for r in range(n_req):
        user = 100_000 + rng.integers(0, 50_000, size=int(rng.integers(8, 513)), dtype=np.int32)
        toks = np.concatenate([system, user])
        t0 = time.perf_counter()
        _, c = alloc.add_seq_tokens(r, toks)
        t_admit += time.perf_counter() - t0
        prompt_tokens += toks.size
        cached_tokens += c
        t0 = time.perf_counter()
        alloc.append_tokens(r, rng.integers(0, 50_000, size=16, dtype=np.int32))
        t_decode += time.perf_counter() - t0
        live.append(r)
        if len(live) == in_flight:
            alloc.free_seq(live.pop(0))
    print(json.dumps({"probe": "prefix_cache_host_allocator", "requests": n_req, "in_flight": in_flight,
                      "system_prompt_tokens": 1500, "user_tokens": "uniform [8, 512]",
                      "prompt_tokens": int(prompt_tokens), "served_from_cache": int(cached_tokens),
                      "served_fraction": round(cached_tokens / prompt_tokens, 4),
                      "admit_us_per_request": round(t_admit / n_req * 1e6, 2),
                      "append16_us_per_request": round(t_decode / n_req * 1e6, 2)}))


def partial_slots(np, lens, per_item):
    """Partial results each decode row's merge combines (1: the row is written
    directly).  The matrix-core kernel (per_item) writes one partial per work
    item: items of two 512-token partitions, four for a sequence of nine
    partitions or more, the last item of a sequence with several split into
    one-partition pieces when it covers more than one; the vector-ALU kernel
    writes one per 512-token partition."""
    nparts = np.maximum(1, -(-lens // 512))
    if not per_item:
        return nparts
    ip = np.where(nparts >= 9, 4, 2)
    items = -(-nparts // ip)
    last_blocks = -(-lens // 16) - (items - 1) * ip * 32
    pieces = np.where((items > 1) & (last_blocks > 32), -(-last_blocks // 32), 1)
    return items - 1 + pieces


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "paged_kv_cache_360_amd", "libpkvprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    for fn in (lib.pkv_probe_read_blocks, lib.pkv_probe_read_slices):
        fn.restype = ctypes.c_int
    lib.pkv_probe_read_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.pkv_probe_read_slices.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
    return lib


def read_probe_on_blocks(torch, np, kcs, vcs, blk_ids, Hkv, D, es, rounds=4):
    """Plain read kernels over the K and V of the listed blocks (device pools,
    rotated like the decode step's), one launch per pool copy and round, the
    first round untimed.  Returns GB/s for whole blocks and for per-head slices
    (the partition kernel's pattern), or None without the probe library."""
    lib = _probe_lib()
    if lib is None:
        return None
    nb = kcs[0].shape[0]
    assert blk_ids.size > 0 and int(blk_ids.min()) >= 0 and int(blk_ids.max()) < nb, "block id outside the pool"
    ids = torch.from_numpy(np.ascontiguousarray(blk_ids, np.int32)).cuda()
    grid = 2048
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    row_bytes = D * es
    block_bytes = 16 * Hkv * row_bytes
    moved = int(blk_ids.size) * 2 * block_bytes
    res = {"bytes_per_launch": moved, "blocks": int(blk_ids.size)}
    for name, launch in (
            ("blocks", lambda r: lib.pkv_probe_read_blocks(kcs[r].data_ptr(), vcs[r].data_ptr(), ids.data_ptr(),
                                                           int(blk_ids.size), block_bytes, grid, sink.data_ptr(),
                                                           stream.cuda_stream)),
            ("slices", lambda r: lib.pkv_probe_read_slices(kcs[r].data_ptr(), vcs[r].data_ptr(), ids.data_ptr(),
                                                           int(blk_ids.size), Hkv, row_bytes, grid,
                                                           sink.data_ptr(), stream.cuda_stream))):
        ts = []
        for rd in range(rounds):
            for r in range(len(kcs)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = launch(r)
                e1.record(stream)
                if rc != 0:
                    raise RuntimeError(f"read probe {name}: HIP error {rc}")
                if rd > 0:
                    ts.append((e0, e1))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in ts]
        res[f"{name}_GBps"] = round(moved / (float(np.mean(us)) * 1e-6) / 1e9, 1)
        res[f"{name}_avg_launch_us"] = round(float(np.mean(us)), 2)
    res["launches_timed_each"] = (rounds - 1) * len(kcs)
    return res


def read_probe_standalone(torch, np, seed):
    """The read kernels alone over two 768 MiB pools of 32 KiB blocks (GQA 32/8,
    head_dim 128, bf16), every block once, in a seeded random order (as a block
    table scatters them) and in pool order, with N(0,1) data and with zeros."""
    nb, Hkv, D = 24576, 8, 128
    orders = {"random_order": np.random.default_rng(seed).permutation(nb).astype(np.int32),
              "pool_order": np.arange(nb, dtype=np.int32)}
    lines = {}
    for fill in ("random", "zeros"):
        kcs, vcs = [], []
        for _ in range(2):
            if fill == "random":
                kcs.append(torch.randn((nb, 16, Hkv, D), device="cuda").to(torch.bfloat16))
                vcs.append(torch.randn((nb, 16, Hkv, D), device="cuda").to(torch.bfloat16))
            else:
                kcs.append(torch.zeros((nb, 16, Hkv, D), dtype=torch.bfloat16, device="cuda"))
                vcs.append(torch.zeros((nb, 16, Hkv, D), dtype=torch.bfloat16, device="cuda"))
        for name, ids in orders.items():
            lines[f"{fill}_{name}"] = read_probe_on_blocks(torch, np, kcs, vcs, ids, Hkv, D, 2)
        del kcs, vcs
        torch.cuda.empty_cache()
    print(json.dumps({"probe": "read", "pool_blocks": nb, "block_bytes": 16 * Hkv * D * 2, "pool_copies": 2,
                      "results": lines}))


def lds_probe(torch, np):
    """The chunked-prefill kernel's LDS operand reads by themselves
    (libpkvprobe.so): one workgroup per compute unit with that kernel's LDS
    layout at head_dim 128 (padded rows, or its unit-column layouts), each wave repeating the K reads (eight 16-byte reads
    per lane), the transposing V reads (sixteen 8-byte reads per lane) or both,
    as one wave does in one 32-token step.  Reports the median loop cycles per
    iteration and wave (s_memtime, the counter the kernel's own step stamps
    use) and the LDS read rate of the whole device from HIP events.  "units"
    lines use the kernel's unit-column layouts instead of padded rows."""
    import ctypes
    lib = _probe_lib()
    if lib is None:
        raise RuntimeError("libpkvprobe.so is not built")
    fn = lib.pkv_probe_lds_reads
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    stream = torch.cuda.current_stream()
    results = []
    for waves in (4, 8, 16):
        sink = torch.zeros(grid * waves * 64, dtype=torch.int32, device="cuda")
        cyc = torch.zeros(grid * waves, dtype=torch.int64, device="cuda")
        for mode, name in ((1, "K"), (2, "V"), (3, "K+V"), (5, "K units"), (6, "V units"), (7, "K+V units")):
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = fn(mode, waves, iters, grid, sink.data_ptr(), cyc.data_ptr(), stream.cuda_stream)
                e1.record(stream)
                if rc != 0:
                    raise RuntimeError(f"lds probe: error {rc}")
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
            per_wave = (8 * 1024 if mode & 1 else 0) + (16 * 512 if mode & 2 else 0)
            cycles = float(np.median(cyc.cpu().numpy())) / iters
            results.append({"reads": name, "waves_per_cu": waves, "bytes_per_wave_iter": per_wave,
                            "median_cycles_per_iter": round(cycles, 1),
                            "bytes_per_cycle_per_cu_if_concurrent": round(waves * per_wave / cycles, 1),
                            "device_TBps_events": round(grid * waves * per_wave * iters / (best * 1e-3) / 1e12, 2),
                            "launch_ms": round(best, 3)})
    print(json.dumps({"probe": "lds_operand_reads", "compute_units": grid, "iters": iters, "results": results}))


def main():
    args = parse_args()
    if args.traffic_from:
        return traffic_from_counters(args.traffic_from, args.workload)
    if args.prefix_cache_probe:
        import numpy as np

        import paged_kv_cache_360_amd as pkv
        return prefix_cache_probe(np, pkv, args.seed)
    if args.capacity_sim:
        import numpy as np

        from paged_kv_cache_360_amd import capacity
        reqs = capacity.draw_requests(np.random.default_rng(args.seed), 1500, 64, 512, 200, 1536)
        res = {p: capacity.simulate(reqs, 65536, 1536, p) for p in ("static", "paged")}
        print(json.dumps({"probe": "capacity_sim", "requests": 1500, "prompt": "uniform [64, 512]",
                          "output": "geometric mean 200, capped at 1536", "memory_slots": 65536,
                          "static": res["static"], "paged": res["paged"],
                          "running_ratio": round(res["paged"]["mean_running"] / res["static"]["mean_running"], 2),
                          "iterations_ratio": round(res["static"]["iterations"] / res["paged"]["iterations"], 2)}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; this paged-attention path runs on a single MI355X and has no "
              "multi-GPU code.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_360_amd as pkv
    from workloads import SPECS, draw_context_lens, normal_values_parallel, pool_blocks_for

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe(torch, pkv)
        return
    if args.swap_probe:
        swap_probe(torch, pkv, args.seed)
        return
    if args.graph_probe:
        graph_probe(torch, np, pkv, args.seed)
        return
    if args.read_probe:
        read_probe_standalone(torch, np, args.seed)
        return
    if args.lds_probe:
        lds_probe(torch, np)
        return

    spec = SPECS[args.workload]
    if spec.chunk_rows:
        return mixed_main(args, spec)
    prefix = spec.ctx_kind == "prefix"                  # sequences forked from one shared prefix
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    es = 2 if spec.dtype == "bf16" else 4
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    W, K, R = args.warmup, args.steps, max(1, args.pool_copies)
    P = 8                                               # detail steps after the timed region
    n_steps = W + K + P

    # ---- workload: lengths, allocator state, pool, queries ------------------
    t0 = time.time()
    rng = np.random.default_rng(args.seed)
    ctx0 = draw_context_lens(rng, spec)                 # context at the first step (new token included)
    final_ctx = ctx0.astype(np.int64) + n_steps - 1
    MB = int(-(-final_ctx.max() // 16))
    max_ctx_bound = int(final_ctx.max())
    ids = np.arange(S, dtype=np.int64)
    cow_pairs = np.zeros((0, 2), np.int32)
    if prefix:
        # the prefix's full blocks are shared by every sequence; each sequence's
        # copy of the partial prefix block (copy-on-write) and its tail are its own
        Pn = spec.prefix_len
        shared_tokens = Pn // 16 * 16
        nb = int(math.ceil(1.25 * (Pn // 16 + int(np.sum(-(-final_ctx // 16) - Pn // 16)))))
        alloc = pkv.BlockAllocator(nb, 16, shuffle_seed=args.seed)
        alloc.add_seq(0)
        alloc.append(0, Pn)
        for s in range(1, S):
            alloc.fork(0, s)
        _, cow_pairs = alloc.append_batch(ids, ctx0 - 1 - Pn)   # tails written before the first step
    else:
        shared_tokens = 0
        nb = pool_blocks_for(spec, final_ctx)
        alloc = pkv.BlockAllocator(nb, 16, shuffle_seed=args.seed)
        for s in range(S):
            alloc.add_seq(int(s))
        alloc.append_batch(ids, ctx0 - 1)               # prefilled tokens; the pool holds their K/V

    pool_host_k = normal_values_parallel(args.seed * 10 + 1, (nb, 16, Hkv, D), spec.dtype)
    pool_host_v = normal_values_parallel(args.seed * 10 + 2, (nb, 16, Hkv, D), spec.dtype)
    for src, dst in np.asarray(cow_pairs).reshape(-1, 2):  # the host copy (oracle baseline) mirrors the device one
        pool_host_k[dst] = pool_host_k[src]
        pool_host_v[dst] = pool_host_v[src]

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
        return t.view(tdt) if a.dtype == np.uint16 else t

    kcs, vcs = [up(pool_host_k)], [up(pool_host_v)]
    if len(cow_pairs):                                  # copy-on-write of the shared partial block (setup)
        pkv.pkv_copy_blocks(kcs[0], vcs[0], torch.from_numpy(np.ascontiguousarray(cow_pairs, np.int32)).cuda())
        torch.cuda.synchronize()
    for _ in range(R - 1):
        kcs.append(kcs[0].clone())
        vcs.append(vcs[0].clone())
    q_host = normal_values_parallel(args.seed * 10 + 3, (n_steps, S, Hq, D), spec.dtype)
    qs = up(q_host)
    knew = up(normal_values_parallel(args.seed * 10 + 4, (n_steps, S, Hkv, D), spec.dtype))
    vnew = up(normal_values_parallel(args.seed * 10 + 5, (n_steps, S, Hkv, D), spec.dtype))
    out = torch.empty((S, Hq, D), dtype=tdt, device="cuda")
    # one workspace per staging set: consecutive steps alternate between them
    wss = [pkv.decode_workspace(S, Hq, D, max_ctx_bound) for _ in range(2)]
    scale = float(np.float32(1.0 / math.sqrt(D)))

    # pinned staging: [slots S | lens S | pad to 16 bytes | tables S*MB] int32, two
    # sets; the slots and lengths go up as bytes, the tables row by row (only
    # the entries each context uses)
    head = 2 * S + (-2 * S) % 4
    meta_len = head + S * MB
    stage = [torch.empty(meta_len, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    dmeta = [torch.empty(meta_len, dtype=torch.int32, device="cuda") for _ in range(2)]
    views = []
    for b in range(2):
        h = stage[b].numpy()
        views.append((h[:S], h[S:2 * S], h[head:].reshape(S, MB)))
    ones = np.ones(S, dtype=np.int32)
    main = torch.cuda.current_stream()
    h2d_done = [torch.cuda.Event() for _ in range(2)]   # the upload of staging set b has run
    log(f"[bench] setup {time.time() - t0:.1f}s: {spec.name} S={S} Hq={Hq} Hkv={Hkv} D={D} "
        f"pool={nb} blocks x{R} MB={MB}")

    step_lens = []
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K + P)]

    # The step calls the C ABI directly with precomputed pointers: per-call
    # tensor checks in the Python wrappers cost more host time than the
    # kernels take, and the host must stay ahead of the device.
    L = pkv.lib()
    dt = pkv.PKV_BF16 if spec.dtype == "bf16" else pkv.PKV_F32
    q_stride = S * Hq * D * es
    kv_stride = S * Hkv * D * es
    q0, knew0, vnew0, out_p = qs.data_ptr(), knew.data_ptr(), vnew.data_ptr(), out.data_ptr()
    main_h = main.cuda_stream
    dptr = [m.data_ptr() for m in dmeta]
    sptr = [st.data_ptr() for st in stage]
    head_bytes = head * 4
    ws_arg = [(w.data_ptr(), w.numel()) for w in wss]
    kc_p = [t.data_ptr() for t in kcs]
    vc_p = [t.data_ptr() for t in vcs]
    check = pkv.check
    fused = spec.dtype == "bf16"                        # the append form is bf16
    host_alloc_s = []
    host_step_s = []

    def attn_args(i, b, r, stream):
        d = dptr[b]
        return (out_p, q0 + i * q_stride, kc_p[r], vc_p[r], d + 4 * head, d + 4 * S, scale, 16, Hq, Hkv,
                D, S, MB, nb, max_ctx_bound, dt, ws_arg[b][0], ws_arg[b][1], stream)

    # The merge of step i runs inside step i+1's upload + plan launch (the two
    # are latency-bound and overlap); `pending` is the step whose merge is still
    # due, flushed with a plain merge launch at the end of each phase.  The
    # detail steps after the timed region keep the launches apart to time them.
    pending = [None]

    def flush():
        if pending[0] is not None:
            pi, pb, pr = pending[0]
            check("pkv_attention_decode_merge", L.pkv_attention_decode_merge(*attn_args(pi, pb, pr, main_h)))
            pending[0] = None

    def step(i, timed, detail=False):
        b = i % 2
        slots_h, lens_h, tables_h = views[b]
        h2d_done[b].synchronize()                       # staging set b is free again (step i-2's upload ran)
        ta = time.perf_counter()
        _, pairs = alloc.append_batch(ids, ones, slots_out=slots_h)
        alloc.block_tables(ids, MB, fill=-1, tables_out=tables_h, lens_out=lens_h)
        host_alloc_s.append(time.perf_counter() - ta)
        if timed:
            step_lens.append(lens_h.copy())
        r = i % R
        bracket = detail or (timed and (i - W) % ev_every(K) == 0)
        ev = events[i - W] if bracket else None
        if detail:
            flush()
            ev[0].record(main)
        merge_out, merge_ws = None, None
        if pending[0] is not None:                      # the previous step's merge rides along
            merge_out, merge_ws = out_p, ws_arg[pending[0][1]][0]
            pending[0] = None
        # metadata upload + work list (+ that merge), one launch on the compute
        # stream; the lengths it plans from are the staging's, at offset S
        check("pkv_attention_decode_plan_upload", L.pkv_attention_decode_plan_upload(
            *attn_args(i, b, r, None)[:-1], sptr[b] + 4 * S, sptr[b], dptr[b], head_bytes, sptr[b] + 4 * head,
            merge_out, merge_ws, main_h))
        h2d_done[b].record(main)
        if len(pairs):
            pkv.pkv_copy_blocks(kcs[r], vcs[r], torch.from_numpy(pairs).cuda())
        if not fused:
            check("pkv_write", L.pkv_write(kc_p[r], vc_p[r], knew0 + i * kv_stride, vnew0 + i * kv_stride,
                                           dptr[b], S, nb, 16, Hkv, D, dt, main_h))
        if bracket:
            ev[1].record(main)
        args_m = attn_args(i, b, r, main_h)
        if fused:   # the new K/V rows go to the cache inside the partition launch
            a = args_m
            check("pkv_attention_decode_partitions_append", L.pkv_attention_decode_partitions_append(
                a[0], a[1], knew0 + i * kv_stride, vnew0 + i * kv_stride, *a[2:]))
        else:
            check("pkv_attention_decode_partitions", L.pkv_attention_decode_partitions(*args_m))
        if bracket:
            ev[2].record(main)
        if detail:
            check("pkv_attention_decode_merge", L.pkv_attention_decode_merge(*args_m))
            ev[3].record(main)
        else:
            pending[0] = (i, b, r)
        host_step_s.append(time.perf_counter() - ta)

    for i in range(W):
        step(i, False)
    flush()
    torch.cuda.synchronize()
    log(f"[bench] warmup {W} steps done")
    t_start = time.perf_counter()
    for i in range(W, W + K):
        step(i, True)
    flush()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] timed {K} steps: {wall * 1e3:.2f} ms")
    for i in range(W + K, W + K + P):
        step(i, False, detail=True)
    torch.cuda.synchronize()

    # ---- per-kernel durations and algorithmic bytes --------------------------
    timed_ev = list(range(0, K, ev_every(K)))          # timed steps whose launch was bracketed
    t_part = [events[k][1].elapsed_time(events[k][2]) * 1e-3 for k in timed_ev]
    # detail steps: the upload + plan launch (no merge rides along there), plus the
    # write for fp32 (bf16: fused into the partitions); the merge on its own
    t_write = [e[0].elapsed_time(e[1]) * 1e-3 for e in events[K:]]
    t_merge = [e[2].elapsed_time(e[3]) * 1e-3 for e in events[K:]]
    kv_b, part_b, merge_b, logical_b = [], [], [], []
    for lens in step_lens:
        lens = lens.astype(np.int64)
        slots = partial_slots(np, lens, fused)
        # K/V bytes the launch must bring in: a shared prefix block counts once
        kv = (int(lens.sum()) - (S - 1) * shared_tokens) * 2 * Hkv * D * es
        logical_b.append(int(lens.sum()) * 2 * Hkv * D * es)
        q_out = S * Hq * D * es + int((slots == 1).sum()) * Hq * D * es
        meta = int((4 * -(-lens // 16)).sum()) + 4 * S
        partials = int(slots[slots > 1].sum()) * Hq * (D + 2) * 4
        # append form: the new K/V rows are read from the inputs and stored to the cache
        append = 4 * S * Hkv * D * es if fused else 0
        kv_b.append(kv)
        part_b.append(kv + q_out + meta + partials + append)
        merge_b.append(partials + int((slots > 1).sum()) * Hq * D * es + 4 * S)
    sum_tp = sum(t_part)
    achieved = sum(part_b[k] for k in timed_ev) / sum_tp / 1e9
    kv_gbps = sum(kv_b[k] for k in timed_ev) / sum_tp / 1e9
    ms_per_step = wall / K * 1e3
    value = S * K / wall
    alg_bracketed = float(np.mean([part_b[k] for k in timed_ev]))

    # HBM traffic: the counted ratio of counter bytes to algorithmic bytes for
    # this kernel source and workload, times this run's algorithmic bytes
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_source_sha256") == kernel_source_hash() and tr.get("workload") == spec.name
                and "traffic_over_algorithmic" in tr):
            traffic = int(round(tr["traffic_over_algorithmic"] * alg_bracketed))

    # plain read kernels over the same blocks (the contexts of the last step)
    tables_f, lens_f = alloc.block_tables(ids, MB)
    blk_ids = np.concatenate([tables_f[s, :-(-int(lens_f[s]) // 16)] for s in range(S)]).astype(np.int32)
    probe = read_probe_on_blocks(torch, np, kcs, vcs, blk_ids, Hkv, D, es)
    kv_probe_bytes = int(blk_ids.size) * 2 * 16 * Hkv * D * es

    roofline = {
        "kernel": ("decode_partition_mfma_kernel (pkv_attention_decode_partitions_append)" if fused
                   else "decode_partition_kernel (pkv_attention_decode_partitions)"),
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": int(alg_bracketed),
        "algorithmic_bytes_mean_all_timed": int(np.mean(part_b)),
        "avg_launch_us": round(sum_tp / len(timed_ev) * 1e6, 2),
        "median_launch_us": round(float(np.median(t_part)) * 1e6, 2),
        "launches_timed": len(timed_ev),
    }

    # ---- CPU oracle baseline (bounded sample of the same batch) --------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, spec, q_host[W + K - 1], pool_host_k, pool_host_v, alloc, ids, MB,
                           scale, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": 16, "partition_tokens": 512,
            "context": f"{spec.ctx_kind}[{spec.ctx_lo},{spec.ctx_hi}] + 1 per step",
            "mean_context": round(float(np.mean([l.mean() for l in step_lens])), 1),
            "pool_blocks": nb, "pool_copies": R, "seed": args.seed,
        },
        # K/V bytes per partition launch over that launch's time (kernel only) ...
        "kv_read_GBps_kernel": round(kv_gbps, 1),
        **({"kv_logical_read_GBps": round(sum(logical_b[k] for k in timed_ev) / sum_tp / 1e9, 1),
            "prefix_len": spec.prefix_len, "cow_pairs": int(len(cow_pairs))} if prefix else {}),
        "kv_read_frac_of_peak_kernel": round(kv_gbps / HBM_PEAK_GBPS, 4),
        # ... and over the whole step (wall time per step, every launch and gap included)
        "kv_read_GBps_step": round(float(np.mean(kv_b)) / (wall / K) / 1e9, 1),
        "kv_read_frac_of_peak_step": round(float(np.mean(kv_b)) / (wall / K) / 1e9 / HBM_PEAK_GBPS, 4),
        "read_probe": probe,
        **({"kv_read_frac_of_read_probe": round(kv_gbps / max(probe["blocks_GBps"], probe["slices_GBps"]), 4)}
           if probe and not prefix else {}),
        "kernels_us": {
            ("upload_plan" if fused else "upload_plan_write"): round(float(np.mean(t_write)) * 1e6, 2),
            "decode_partitions": round(float(np.mean(t_part)) * 1e6, 2),
            "merge": round(float(np.mean(t_merge)) * 1e6, 2),
        },
        "host_alloc_us": round(float(np.mean(host_alloc_s[W:W + K])) * 1e6, 2),
        "host_step_us": round(float(np.mean(host_step_s[W:W + K])) * 1e6, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def mixed_main(args, spec):
    """Chunked-prefill mixed step: one prefill chunk batched with decode sequences.

    Sequence 0 holds a context of spec.chunk_ctx tokens whose last spec.chunk_rows
    are the chunk's query rows (written every step into the same slots, so each
    step has the same shape); sequences 1..S append one decode token per step.
    One step, all on the compute stream = host allocation into pinned staging
    + pkv_attention_varlen_plan_upload (the work lists planned from the pinned
    lengths while the step's slots, lengths and used table entries are copied
    to the device, one launch) + pkv_write of all new rows from the uploaded
    slots + pkv_attention_varlen_partitions (decode partitions, prefill tiles,
    merge).  The upload + plan, write and attention launches of every
    ev_every(K)-th timed step are bracketed by events.
    """
    import numpy as np
    import torch

    import paged_kv_cache_360_amd as pkv
    from workloads import draw_context_lens, normal_values_parallel, pool_blocks_for

    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    C, CC = spec.chunk_rows, spec.chunk_ctx
    W, K, R = args.warmup, args.steps, max(1, args.pool_copies)
    n_steps = W + K
    rng = np.random.default_rng(args.seed)
    dec0 = draw_context_lens(rng, spec)
    final = dec0.astype(np.int64) + n_steps - 1
    MB = int(-(-max(int(final.max()), CC) // 16))
    nb = pool_blocks_for(spec, np.concatenate([[CC], final]))
    alloc = pkv.BlockAllocator(nb, 16, shuffle_seed=args.seed)
    ids = np.arange(S + 1, dtype=np.int64)
    for s in ids:
        alloc.add_seq(int(s))
    chunk_slots, _ = alloc.append(0, CC)
    chunk_slots = np.asarray(chunk_slots[CC - C:], np.int32)
    alloc.append_batch(ids[1:], dec0 - 1)
    tdt = torch.bfloat16

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(tdt)

    kcs = [up(normal_values_parallel(args.seed * 10 + 1, (nb, 16, Hkv, D), "bf16"))]
    vcs = [up(normal_values_parallel(args.seed * 10 + 2, (nb, 16, Hkv, D), "bf16"))]
    for _ in range(R - 1):
        kcs.append(kcs[0].clone())
        vcs.append(vcs[0].clone())
    T = C + S
    qs = up(normal_values_parallel(args.seed * 10 + 3, (n_steps, T, Hq, D), "bf16"))
    knew = up(normal_values_parallel(args.seed * 10 + 4, (n_steps, T, Hkv, D), "bf16"))
    vnew = up(normal_values_parallel(args.seed * 10 + 5, (n_steps, T, Hkv, D), "bf16"))
    out = torch.empty((T, Hq, D), dtype=tdt, device="cuda")
    max_ctx = max(int(final.max()), CC)
    ws = pkv.varlen_workspace(S + 1, T, Hq, Hkv, D, C, max_ctx)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    qsl = torch.from_numpy(np.concatenate([[0], C + np.arange(S + 1)]).astype(np.int32)).cuda()

    # pinned staging, two sets: [slots T | lens S+1 | pad to 16 bytes | tables
    # (S+1)*MB] int32; the slots and lengths go up as bytes, the tables by rows
    head = T + (S + 1) + (-(T + S + 1)) % 4
    meta_len = head + (S + 1) * MB
    stage = [torch.zeros(meta_len, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    dmeta = [torch.zeros(meta_len, dtype=torch.int32, device="cuda") for _ in range(2)]
    views = []
    for b in range(2):
        h = stage[b].numpy()
        h[:C] = chunk_slots                               # the chunk rewrites the same slots each step
        views.append((h[:T], h[T:T + S + 1], h[head:].reshape(S + 1, MB)))
    ones = np.ones(S, np.int32)
    main = torch.cuda.current_stream()
    up_done = [torch.cuda.Event() for _ in range(2)]     # the upload launch of staging set b has run
    events, lens_log = [], []

    # direct C-ABI calls with precomputed pointers (as in the decode step)
    L = pkv.lib()
    check = pkv.check
    q_stride, kv_stride = T * Hq * D * 2, T * Hkv * D * 2
    q0, knew0, vnew0, out_p = qs.data_ptr(), knew.data_ptr(), vnew.data_ptr(), out.data_ptr()
    kc_p = [t.data_ptr() for t in kcs]
    vc_p = [t.data_ptr() for t in vcs]
    dptr = [m.data_ptr() for m in dmeta]
    sptr = [st.data_ptr() for st in stage]
    qsl_p, ws_p, ws_n, main_h = qsl.data_ptr(), ws.data_ptr(), ws.numel(), main.cuda_stream

    def step(i, timed):
        b = i % 2
        slots_h, lens_h, tables_h = views[b]
        up_done[b].synchronize()                          # staging set b is free (step i-2's upload ran)
        _, pairs = alloc.append_batch(ids[1:], ones, slots_out=slots_h[C:])
        alloc.block_tables(ids, MB, fill=-1, tables_out=tables_h, lens_out=lens_h)
        r = i % R
        bracket = timed and (i - W) % ev_every(K) == 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if bracket else None
        if timed:
            lens_log.append(lens_h.copy())
        if bracket:
            ev[0].record(main)
        d = dptr[b]
        args = (out_p, q0 + i * q_stride, kc_p[r], vc_p[r], d + 4 * head, d + 4 * T, qsl_p, T, C, scale, 16,
                Hq, Hkv, D, S + 1, MB, nb, max_ctx, pkv.PKV_BF16, ws_p, ws_n)
        check("pkv_attention_varlen_plan_upload", L.pkv_attention_varlen_plan_upload(
            *args, sptr[b] + 4 * T, sptr[b], d, 4 * head, sptr[b] + 4 * head, main_h))
        up_done[b].record(main)
        if bracket:
            ev[1].record(main)
        check("pkv_write", L.pkv_write(kc_p[r], vc_p[r], knew0 + i * kv_stride, vnew0 + i * kv_stride, d, T, nb,
                                       16, Hkv, D, pkv.PKV_BF16, main_h))
        if bracket:
            ev[2].record(main)
        check("pkv_attention_varlen_partitions", L.pkv_attention_varlen_partitions(*args, main_h))
        if bracket:
            ev[3].record(main)
            events.append(ev)

    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_up = [e[0].elapsed_time(e[1]) * 1e-3 for e in events]
    t_write = [e[1].elapsed_time(e[2]) * 1e-3 for e in events]
    t_attn = [e[2].elapsed_time(e[3]) * 1e-3 for e in events]
    # algorithmic bytes of the attention call: K/V each row group reads once
    # (decode rows: their context; the chunk: its 4096-token context), q, out,
    # and the partials of rows spanning several partitions
    es, row_kv = 2, 2 * Hkv * D * 2
    keys_chunk = CC - C + np.arange(C) + 1
    flops_prefill = 4 * D * Hq * int(keys_chunk.sum())
    att_b = []
    for lens in lens_log:
        dec = lens[1:].astype(np.int64)
        dslots = partial_slots(np, dec, True)
        b = int(dec.sum()) * row_kv + CC * row_kv
        b += 2 * T * Hq * D * es
        pc = -(-keys_chunk // 512)
        b += 2 * (int(dslots[dslots > 1].sum()) + int(pc[pc > 1].sum())) * Hq * (D + 2) * 4
        att_b.append(b)
    ta = float(np.mean(t_attn))

    # The chunk alone (after the timed region): the same varlen call over
    # sequence 0's 512 rows only (plan, prefill tiles, merge; its decode launch
    # has no work), and its four launches made one by one with HIP events
    # around the prefill-tile launch, the kernel's own rate against the dense
    # bf16 peak.
    tab0, len0 = alloc.block_tables(ids[:1], MB)
    t0_d = torch.from_numpy(tab0).cuda()
    c0_d = torch.tensor([CC], dtype=torch.int32, device="cuda")
    qsl0 = torch.tensor([0, C], dtype=torch.int32, device="cuda")
    q0_d = qs[n_steps - 1, :C].contiguous()
    out0 = torch.empty((C, Hq, D), dtype=tdt, device="cuda")
    ws0 = pkv.varlen_workspace(1, C, Hq, Hkv, D, C, CC)
    chunk_call = lambda: pkv.pkv_attention_varlen(out0, q0_d, kcs[0], vcs[0], t0_d, c0_d, qsl0, scale, C, CC,
                                                  workspace=ws0)
    for _ in range(3):
        chunk_call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        chunk_call()
    e1.record()
    torch.cuda.synchronize()
    t_chunk = e0.elapsed_time(e1) * 1e-3 / 10
    cargs = (out0, q0_d, kcs[0], vcs[0], t0_d, c0_d, qsl0, scale, C, CC)
    tile_ev = []
    for i in range(13):
        pkv.pkv_attention_varlen_plan(*cargs, workspace=ws0)
        pkv.pkv_attention_varlen_decode_partitions(*cargs, workspace=ws0)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        pkv.pkv_attention_varlen_prefill_tiles(*cargs, workspace=ws0)
        a1.record()
        pkv.pkv_attention_varlen_merge(*cargs, workspace=ws0)
        if i >= 3:
            tile_ev.append((a0, a1))
    torch.cuda.synchronize()
    t_tiles = [a.elapsed_time(b) * 1e-3 for a, b in tile_ev]
    t_tile = float(np.mean(t_tiles))
    res = {
        "metric": "mixed chunked-prefill step: query rows/s (prefill chunk + decode rows), bf16 GQA",
        "value": round(T * K / wall, 1),
        "unit": "query rows/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "chunk_rows": C, "chunk_context": CC, "decode_seqs": S,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": 16,
                   "partition_tokens": 512, "pool_blocks": nb, "pool_copies": R, "seed": args.seed},
        "kernels_us": {"upload_plan": round(float(np.mean(t_up)) * 1e6, 2),
                       "write": round(float(np.mean(t_write)) * 1e6, 2),
                       "varlen_partitions": round(ta * 1e6, 2)},
        "decode_tokens_per_s": round(S * K / wall, 1),
        "prefill_gflop_per_step": round(flops_prefill / 1e9, 2),
        "roofline": {
            "kernel": "pkv_attention_varlen_partitions (decode partitions + prefill tiles + merge)",
            "bound": "hbm", "achieved": round(float(np.mean(att_b)) / ta / 1e9, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(float(np.mean(att_b)) / ta / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": int(np.mean(att_b)), "avg_launch_us": round(ta * 1e6, 2),
        },
        "roofline_prefill": {
            "kernel": "prefill_mfma_kernel (pkv_attention_varlen_prefill_tiles over the chunk alone; "
                      "HIP events around 10 launches)",
            "bound": "mfma", "achieved": round(flops_prefill / t_tile / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(flops_prefill / t_tile / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": int(flops_prefill), "avg_launch_us": round(t_tile * 1e6, 2),
            "median_launch_us": round(float(np.median(t_tiles)) * 1e6, 2), "launches_timed": len(t_tiles),
            "call_level": {"call": "pkv_attention_varlen over the chunk alone (plan + prefill tiles + merge)",
                           "avg_call_us": round(t_chunk * 1e6, 2),
                           "TFLOPs": round(flops_prefill / t_chunk / 1e12, 1)},
        },
        "cpu_baseline": None,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ORACLE_WORKER = {}


def _oracle_worker_init(shm_names, shape, dtype, q, tables, lens, scale):
    """Process-pool worker set-up: attach the shared K/V pools (no copy)."""
    from multiprocessing import shared_memory

    import numpy as np

    shms = [shared_memory.SharedMemory(name=nm) for nm in shm_names]
    _ORACLE_WORKER.update(shms=shms, k=np.ndarray(shape, dtype, buffer=shms[0].buf),
                          v=np.ndarray(shape, dtype, buffer=shms[1].buf), q=q, tables=tables, lens=lens,
                          scale=scale)


def _oracle_worker_run(seqs):
    """The oracle over a few sequences of the shared batch; returns their tokens."""
    import oracle
    w = _ORACLE_WORKER
    for s in seqs:
        oracle.decode_attention(w["q"][s:s + 1], w["k"], w["v"], w["tables"][s:s + 1], w["lens"][s:s + 1],
                                w["scale"])
    return int(sum(int(w["lens"][s]) for s in seqs))


def cpu_baseline(np, spec, q_last, pool_k, pool_v, alloc, ids, MB, scale, budget_s):
    """The fp64 oracle on the host for about ``budget_s`` seconds, sequence by
    sequence over the last timed step's batch (repeated passes; the last may
    stop part way): a third of the time on one process, the rest over a pool
    of up to 16 worker processes (started fresh, so none inherits this
    process's GPU state; the K/V pools are shared, not copied; one BLAS thread
    each).  The oracle itself is unchanged; ``value`` is the pool's rate."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import shared_memory

    import oracle
    from threadpoolctl import threadpool_limits

    tables, lens = alloc.block_tables(ids, MB)
    n = len(ids)
    es = 2 if spec.dtype == "bf16" else 4
    row = 2 * spec.num_kv_heads * spec.head_dim * es

    with threadpool_limits(limits=1):
        done1, kv1, t0 = 0, 0, time.perf_counter()
        while True:
            s = done1 % n
            oracle.decode_attention(q_last[s:s + 1], pool_k, pool_v, tables[s:s + 1], lens[s:s + 1], scale)
            kv1 += int(lens[s])
            done1 += 1
            if time.perf_counter() - t0 >= budget_s / 3:
                break
        el1 = time.perf_counter() - t0

    workers = max(1, min(16, os.cpu_count() or 1))
    shms = []
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        for a in (pool_k, pool_v):
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            shms.append(shm)
            np.ndarray(a.shape, a.dtype, buffer=shm.buf)[...] = a
        for k in saved:
            os.environ[k] = "1"                      # the workers' BLAS: one thread each
        ctx = mp.get_context("spawn")
        with ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_oracle_worker_init,
                                 initargs=([m.name for m in shms], pool_k.shape, pool_k.dtype, q_last, tables,
                                           lens, scale)) as ex:
            list(ex.map(_oracle_worker_run, [[k % n] for k in range(workers)]))   # start-up, untimed
            chunk = 2
            done, kv, t0 = 0, 0, time.perf_counter()
            while time.perf_counter() - t0 < 2 * budget_s / 3:
                batch = [[(done + k * chunk + j) % n for j in range(chunk)] for k in range(workers * 2)]
                kv += sum(ex.map(_oracle_worker_run, batch))
                done += chunk * len(batch)
            el = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        for m in shms:
            m.close()
            m.unlink()
    return {
        "value": round(done / el, 3),
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{done} sequence decodes on {workers} processes ({done / n:.2f} passes over the {n} sequences "
                  f"of the last timed step's batch, mean context {float(lens.mean()):.0f}), fp64 NumPy, one BLAS "
                  f"thread each, {el:.1f} s; on one process: {done1} decodes in {el1:.1f} s; host "
                  f"{os.cpu_count()} logical CPUs, {_cpu_model()}",
        "one_process_value": round(done1 / el1, 3),
        "kv_GBps": round(kv * row / el / 1e9, 4),
    }


if __name__ == "__main__":
    main()
