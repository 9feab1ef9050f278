"""The C-ABI library on the CPU: symbols, host-side argument checks, the allocator.

Nothing here launches a kernel.  Error-path calls use fake (non-null, aligned)
device addresses: validation rejects them before any HIP call.
"""

import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_cache_360_amd as pkv
from allocator_checks import (check_enomem_atomic, check_fork_and_cow, check_hundred_tokens,
                              check_invariants, check_paged_waste_under_one_block, random_ops)
from paged_kv_cache_360_amd._lib import (PKV_BF16, PKV_EINVAL, PKV_ENOSEQ, PKV_EUNSUPPORTED,
                                         PKV_EWORKSPACE, PKV_F32, PKV_OK, lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # aligned, never dereferenced


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pkv_\w+)\s*\(", text))
    return sorted(names)


def test_header_is_plain_c():
    """include/*.h compiles as C99 and as C++17 on its own: no C++ or torch types cross the ABI."""
    import shutil
    import subprocess
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not fn.endswith(".h"):
            continue
        path = os.path.join(ROOT, "include", fn)
        for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++17", "c++")):
            if shutil.which(cc) is None:
                pytest.skip(f"{cc} not available")
            r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", lang, path],
                               capture_output=True, text=True)
            assert r.returncode == 0, f"{fn} as {lang}: {r.stderr}"


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    handle = lib()
    for n in names:
        assert hasattr(handle, n), n


def test_strerror_and_last_error():
    assert lib().pkv_strerror(PKV_EWORKSPACE) == b"PKV_EWORKSPACE"
    code = lib().pkv_write(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 15, 2, 64, PKV_BF16, None)
    assert code == PKV_EUNSUPPORTED
    assert b"block_size" in lib().pkv_last_error()


def _decode(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, tables=FAKE, ctx=FAKE, scale=0.125, bs=16, hq=32,
             hkv=8, d=128, s=4, mb=128, nb=1000, maxctx=2048, dt=PKV_BF16, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib().pkv_attention_decode(a["out"], a["q"], a["kc"], a["vc"], a["tables"], a["ctx"],
                                      a["scale"], a["bs"], a["hq"], a["hkv"], a["d"], a["s"], a["mb"],
                                      a["nb"], a["maxctx"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=32), PKV_EUNSUPPORTED),
    (dict(d=96), PKV_EUNSUPPORTED),
    (dict(hq=12, hkv=8), PKV_EINVAL),
    (dict(hq=48, hkv=3), PKV_EUNSUPPORTED),       # G = 16 not built
    (dict(dt=7), PKV_EUNSUPPORTED),
    (dict(q=0), PKV_EINVAL),
    (dict(tables=0), PKV_EINVAL),
    (dict(out=FAKE + 2), PKV_EINVAL),             # misaligned
    (dict(maxctx=128 * 16 + 1), PKV_EINVAL),      # beyond the table width
    (dict(ws=0), PKV_EWORKSPACE),
    (dict(wsb=100), PKV_EWORKSPACE),
    (dict(scale=float("nan")), PKV_EINVAL),
    (dict(scale=0.0), PKV_EINVAL),                # the softmax scale must be positive
    (dict(scale=-1.0), PKV_EINVAL),
    (dict(s=-1), PKV_EINVAL),
    (dict(s=0), PKV_OK),                          # empty batch: nothing to launch
])
def test_decode_argument_errors(kw, code):
    assert _decode(**kw) == code


def _append(name="pkv_attention_decode_append", **kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, tables=FAKE, ctx=FAKE, scale=0.125,
             bs=16, hq=32, hkv=8, d=128, s=4, mb=128, nb=1000, maxctx=2048, dt=PKV_BF16, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return getattr(lib(), name)(a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["tables"],
                                a["ctx"], a["scale"], a["bs"], a["hq"], a["hkv"], a["d"], a["s"], a["mb"],
                                a["nb"], a["maxctx"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("name", ["pkv_attention_decode_append", "pkv_attention_decode_partitions_append"])
@pytest.mark.parametrize("kw,code", [
    (dict(dt=PKV_F32), PKV_EUNSUPPORTED),         # bf16 only
    (dict(kn=0), PKV_EINVAL),
    (dict(vn=FAKE + 4), PKV_EINVAL),              # misaligned
    (dict(bs=32), PKV_EUNSUPPORTED),              # the decode checks apply too
    (dict(ws=FAKE + 16), PKV_EWORKSPACE),
    (dict(s=0), PKV_OK),                          # empty batch: nothing launched
])
def test_append_argument_errors(name, kw, code):
    assert _append(name, **kw) == code


def test_decode_workspace_sizes():
    f = lib().pkv_decode_workspace_bytes
    one = f(64, 32, 128, 512)                      # one partition: header + work list only
    assert 256 + 64 * 4 * 4 <= one < 4096
    n = f(128, 32, 128, 8192)                      # 16 partitions
    rows = 128 * 32 * 16
    assert n >= rows * (128 + 2) * 4 + 128 * 16 * 4 * 4
    assert f(0, 32, 128, 8192) == 0


def test_decode_workspace_alignment_is_checked():
    assert _decode(ws=FAKE + 16) == PKV_EWORKSPACE


def _varlen(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, tables=FAKE, ctx=FAKE, qsl=FAKE, t=40, mq=32,
             scale=0.125, bs=16, hq=32, hkv=8, d=128, s=4, mb=128, nb=1000, maxctx=2048, dt=PKV_BF16,
             ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib().pkv_attention_varlen(a["out"], a["q"], a["kc"], a["vc"], a["tables"], a["ctx"],
                                      a["qsl"], a["t"], a["mq"], a["scale"], a["bs"], a["hq"], a["hkv"],
                                      a["d"], a["s"], a["mb"], a["nb"], a["maxctx"], a["dt"], a["ws"],
                                      a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=PKV_F32), PKV_EUNSUPPORTED),          # matrix-core path: bf16 only
    (dict(qsl=0), PKV_EINVAL),
    (dict(mq=0), PKV_EINVAL),
    (dict(t=-1), PKV_EINVAL),
    (dict(hq=48, hkv=3), PKV_EUNSUPPORTED),
    (dict(d=96), PKV_EUNSUPPORTED),
    (dict(ws=0), PKV_EWORKSPACE),
    (dict(wsb=1000), PKV_EWORKSPACE),
    (dict(maxctx=128 * 16 + 1), PKV_EINVAL),
    (dict(scale=0.0), PKV_EINVAL),                  # prefill rows mask before scaling: scale > 0
    (dict(scale=-1.0), PKV_EINVAL),
    (dict(t=0), PKV_OK),                            # no query rows: nothing to launch
    (dict(s=0), PKV_OK),
])
def test_varlen_argument_errors(kw, code):
    assert _varlen(**kw) == code


def test_varlen_workspace_sizes():
    f = lib().pkv_varlen_workspace_bytes
    dec = lib().pkv_decode_workspace_bytes(193, 32, 128, 4096)
    assert f(193, 193, 32, 8, 128, 1, 4096) == dec     # all one-row sequences: the decode layout
    big = f(193, 704, 32, 8, 128, 512, 4096)            # a 512-row chunk + 192 decode rows
    rows, parts = 704 * 32, 8
    assert big >= rows * parts * (128 + 2) * 4
    assert f(193, 704, 32, 8, 128, 0, 4096) == 0        # max_query_len must be >= 1
    assert f(4, 40, 12, 8, 128, 8, 512) == 0            # 12 q heads over 8 KV heads


def test_write_and_copy_argument_errors():
    w = lib().pkv_write
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 16, 2, 64, PKV_BF16, None) == PKV_OK
    assert w(FAKE, FAKE, FAKE, FAKE, 0, 3, 8, 16, 2, 64, PKV_BF16, None) == PKV_EINVAL
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 16, 1, 4, PKV_BF16, None) == PKV_EUNSUPPORTED
    assert w(FAKE, FAKE, FAKE + 8, FAKE, FAKE, 3, 8, 16, 2, 64, PKV_F32, None) == PKV_EINVAL
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 16, 2, 64, PKV_F32, None) == PKV_EINVAL
    c = lib().pkv_copy_blocks
    assert c(FAKE, FAKE, FAKE, 0, 8, 16, 2, 64, PKV_BF16, None) == PKV_OK
    assert c(FAKE, FAKE, 0, 2, 8, 16, 2, 64, PKV_BF16, None) == PKV_EINVAL
    assert c(FAKE, FAKE, FAKE, 2, 8, 8, 2, 64, PKV_BF16, None) == PKV_EUNSUPPORTED
    m = lib().pkv_lse_merge
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 128, PKV_F32, None) == PKV_OK
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 80, PKV_F32, None) == PKV_EUNSUPPORTED
    assert m(FAKE, 0, FAKE, FAKE, FAKE, 3, 4, 128, PKV_F32, None) == PKV_EINVAL


def test_graph_and_plan_upload_argument_errors():
    """Rejected before any HIP call: nothing is captured, uploaded or launched."""
    import ctypes
    L = lib()
    g = ctypes.c_void_p(0)
    ws = 1 << 20
    # (out, q, k_new, v_new, slots, n_new, kc, vc, tables, lens, scale, bs, Hq, Hkv, D, S, MB, NB, max_ctx, dt, ws, ws_bytes)
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 0.125, 16, 8, 8, 64, 4, 8, 64, 100, PKV_F32,
          0x100000, ws]

    def create(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.pkv_decode_graph_create(ctypes.addressof(g), *a)

    assert L.pkv_decode_graph_create(None, *ok) == PKV_EINVAL              # no handle to fill
    assert create(a15=0) == PKV_EINVAL                                    # no sequences
    assert create(a4=None) == PKV_EUNSUPPORTED                            # append form is bf16 only
    assert create(a5=-1) == PKV_EINVAL                                    # negative token count
    assert create(a11=32) == PKV_EUNSUPPORTED                             # block size
    assert create(a18=200) == PKV_EINVAL                                  # bound wider than the tables
    assert create(a20=0x100010) == PKV_EWORKSPACE                          # workspace misaligned
    assert g.value in (None, 0)
    assert L.pkv_decode_graph_launch(None, None) == PKV_EINVAL
    L.pkv_decode_graph_destroy(None)
    # plan_upload: (decode args without stream) + host lens, src, dst, bytes, host tables, merge out, merge ws,
    # stream
    d = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, 16, 8, 8, 64, 4, 8, 64, 100, PKV_F32, 0x100000, ws]
    pu = L.pkv_attention_decode_plan_upload
    assert pu(*d[:11], 0, *d[12:], FAKE, FAKE, FAKE, 64, None, None, None, None) == PKV_EINVAL        # no sequences
    assert pu(*d, FAKE, FAKE, FAKE, 60, None, None, None, None) == PKV_EINVAL                         # not 16-byte words
    assert pu(*d[:7], 32, *d[8:], FAKE, FAKE, FAKE, 64, None, None, None, None) == PKV_EUNSUPPORTED   # block size
    assert L.pkv_check_pool(None, 64) == PKV_EINVAL and L.pkv_check_pool(FAKE, 0) == PKV_EINVAL


def test_host_table_and_slot_checks():
    tables = np.array([[3, 1, -1], [0, 7, 2]], np.int32)
    pkv.pkv_check_tables(tables, [20, 40], 8)
    with pytest.raises(pkv.PagedKVError):
        pkv.pkv_check_tables(tables, [20, 40], 7)          # id 7 out of an 7-block pool
    with pytest.raises(pkv.PagedKVError):
        pkv.pkv_check_tables(tables, [33, 40], 8)          # third entry (-1) is used
    pkv.pkv_check_slots(np.array([5, -1, 17, 127], np.int32), 8)
    with pytest.raises(pkv.PagedKVError):
        pkv.pkv_check_slots(np.array([5, 17, 5], np.int32), 8)
    with pytest.raises(pkv.PagedKVError):
        pkv.pkv_check_slots(np.array([128], np.int32), 8)


# ------------------------------------------------------------------ C++ allocator
def make(nb=64, seed=0):
    return pkv.BlockAllocator(nb, 16, shuffle_seed=seed)


def test_allocator_hundred_tokens():
    check_hundred_tokens(make(seed=3))


def test_allocator_waste_under_one_block():
    check_paged_waste_under_one_block(make(nb=1024, seed=5), np.random.default_rng(1))


def test_allocator_fork_and_cow():
    check_fork_and_cow(make(seed=9))


def test_allocator_enomem_atomic():
    check_enomem_atomic(make(nb=20, seed=11), MemoryError)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_allocator_random_ops(seed):
    random_ops(make(nb=48, seed=seed), np.random.default_rng(100 + seed), 400, MemoryError)


def test_allocator_shuffle():
    a = make(nb=32, seed=0)
    a.add_seq(1)
    a.append(1, 32 * 16)
    assert a.block_table(1) == list(range(32))           # seed 0: ids in order
    b = make(nb=32, seed=1234)
    b.add_seq(1)
    b.append(1, 32 * 16)
    t = b.block_table(1)
    assert sorted(t) == list(range(32)) and t != list(range(32))


def test_allocator_errors():
    a = make(nb=8)
    a.add_seq(1)
    with pytest.raises(pkv.PagedKVError):
        a.add_seq(1)
    with pytest.raises(pkv.PagedKVError) as e:
        a.append(99, 1)
    assert e.value.code == PKV_ENOSEQ
    with pytest.raises(pkv.PagedKVError):
        a.fork(42, 2)
    assert lib().pkv_alloc_create(0, 16, 0) is None
    assert lib().pkv_alloc_create(8, 32, 0) is None


def _renaming_equal(ta, tb, mapping):
    for x, y in zip(ta, tb):
        if mapping.setdefault(x, y) != y:
            return False
    return len(ta) == len(tb)


@pytest.mark.parametrize("seed", [7, 8])
def test_allocator_matches_oracle_model_up_to_renaming(seed):
    """Same operations on the C++ allocator and the oracle's model: equal up to block renaming."""
    rng = np.random.default_rng(seed)
    nb = 40
    cpp = make(nb=nb, seed=seed)
    ref = oracle.BlockAllocatorModel(nb, 16)
    live, nxt = [], 0
    for _ in range(300):
        op = rng.integers(0, 8)
        if op == 0 or not live:
            cpp.add_seq(nxt); ref.add_seq(nxt); live.append(nxt); nxt += 1
        elif op == 1:
            p = live[rng.integers(len(live))]
            cpp.fork(p, nxt); ref.fork(p, nxt); live.append(nxt); nxt += 1
        elif op == 2 and len(live) > 1:
            sid = live.pop(rng.integers(len(live)))
            cpp.free_seq(sid); ref.free_seq(sid)
        else:
            sid = live[rng.integers(len(live))]
            n = int(rng.integers(0, 30))
            ra = rb = None
            try:
                ra = cpp.append(sid, n)
            except MemoryError:
                ra = "oom"
            try:
                rb = ref.append(sid, n)
            except MemoryError:
                rb = "oom"
            assert (ra == "oom") == (rb == "oom")
            if ra != "oom":
                assert len(ra[1]) == len(rb[1])
                assert [s % 16 for s in ra[0]] == [s % 16 for s in rb[0]]
        mapping = {}
        for sid in live:
            assert cpp.seq_len(sid) == ref.seq_len(sid)
            assert _renaming_equal(cpp.block_table(sid), ref.block_table(sid), mapping)
        assert cpp.num_free() == ref.num_free()
        check_invariants(cpp, live)


def test_append_batch_all_or_nothing():
    a = make(nb=10, seed=2)
    for s in range(3):
        a.add_seq(s)
    slots, pairs = a.append_batch([0, 1, 2], [16, 17, 5])      # 1 + 2 + 1 blocks
    assert len(slots) == 38 and len(pairs) == 0 and a.num_free() == 6
    a.fork(2, 3)
    a.fork(2, 4)
    before = [a.block_table(s) for s in range(5)], a.num_free()
    with pytest.raises(MemoryError):
        a.append_batch([3, 4, 0], [1, 1, 16 * 6])              # 2 CoW + 6 blocks > 6 free
    assert ([a.block_table(s) for s in range(5)], a.num_free()) == before
    slots, pairs = a.append_batch([3, 4, 2], [1, 1, 1])        # 2 copies; the last sharer writes in place
    assert len(pairs) == 2 and a.num_free() == 4
    tables, lens = a.block_tables([0, 1, 2, 3, 4], 4, fill=-7)
    assert list(lens) == [16, 17, 6, 6, 6] and tables[0, 1] == -7
    with pytest.raises(pkv.PagedKVError):
        a.append_batch([0, 0], [1, 1])                         # duplicate ids


@pytest.mark.parametrize("name", ["pkv_attention_decode_plan", "pkv_attention_decode_partitions",
                                  "pkv_attention_decode_merge", "pkv_attention_decode_partitions_append",
                                  "pkv_attention_decode_plan_upload", "pkv_attention_varlen_plan",
                                  "pkv_attention_varlen_decode_partitions", "pkv_attention_varlen_prefill_tiles",
                                  "pkv_attention_varlen_merge", "pkv_attention_varlen_partitions"])
def test_split_wrappers_need_the_callers_workspace(name):
    """The split launches read the work list the plan left in the workspace: the
    Python wrappers refuse to make a fresh (empty) one, before touching any tensor."""
    with pytest.raises(ValueError, match="workspace is required"):
        if name == "pkv_attention_decode_partitions_append":
            getattr(pkv, name)(None, None, None, None, None, None, None, None, 0.125, 100)
        elif name == "pkv_attention_decode_plan_upload":
            getattr(pkv, name)(None, None, None, None, None, None, 0.125, 100, None, None, None)
        elif name.startswith("pkv_attention_varlen_"):
            getattr(pkv, name)(None, None, None, None, None, None, None, 0.125, 4, 100)
        else:
            getattr(pkv, name)(None, None, None, None, None, None, 0.125, 100)


def test_varlen_split_argument_errors():
    """pkv_attention_varlen_plan_upload / _partitions refuse bad arguments before
    any launch (fake device addresses; page-locked checks fail for them)."""
    L = lib()
    # out q kc vc tables ctx qsl | T mq scale bs Hq Hkv D S MB NB max_ctx dt | ws ws_bytes
    base = [FAKE] * 7 + [40, 32, 0.125, 16, 32, 8, 128, 4, 128, 1000, 2048, PKV_BF16, FAKE, 1 << 30]

    def up(args, upload_bytes=64):
        return L.pkv_attention_varlen_plan_upload(*args, FAKE, FAKE, FAKE, upload_bytes, None, None)

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a
    assert up(base) == PKV_EINVAL                       # host lengths are not page-locked memory
    assert up(with_(7, 0)) == PKV_EINVAL                # no query rows
    assert up(with_(18, PKV_F32)) == PKV_EUNSUPPORTED   # matrix-core path: bf16 only
    assert up(base, upload_bytes=60) == PKV_EINVAL      # not a multiple of 16
    assert up(with_(19, 0)) == PKV_EWORKSPACE
    part = L.pkv_attention_varlen_partitions
    assert part(*with_(6, 0), None) == PKV_EINVAL       # null query_start_loc
    assert part(*with_(19, 0), None) == PKV_EWORKSPACE
    assert part(*with_(9, -1.0), None) == PKV_EINVAL    # negative scale
    assert part(*with_(7, 0), None) == PKV_OK           # no query rows: nothing to launch
